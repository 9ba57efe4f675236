// Host-side pieces of libft: error reporting, thread pool, host expert FFN, LRU policy.
#pragma once

#include <atomic>
#include <condition_variable>
#include <functional>
#include <mutex>
#include <string>
#include <thread>
#include <vector>

#include "ft_internal.h"

namespace ft {

// thread-local last error
void set_error(const std::string& msg);
int fail(int code, const std::string& msg);
// The handler of an entry point's function-try-block: no C++ exception crosses the C ABI.
// Running out of host memory or threads gives FT_ENOMEM, any other exception FT_ESTATE, each
// with a message naming the entry point.
int caught(const char* who);
#define FT_CATCH(who) \
  catch (...) { return ft::caught(who); }

// Fixed set of worker threads; run(fn) calls fn(i, n) for i in [0, n) on the workers and the
// calling thread (i = n - 1) and returns when all have finished.  Jobs are short (one expert's
// FFN, a few blob reads) and come in bursts, so a worker spins for a while after each job
// before it sleeps, and the caller spins for the workers to finish: a sleeping thread's
// wake-up costs more than such a job's share.
class ThreadPool {
 public:
  explicit ThreadPool(int n_threads);
  ~ThreadPool();
  int size() const { return n_; }
  void run(const std::function<void(int, int)>& fn);
  // Bind every worker thread to the given CPUs (the calling thread, which takes a share of
  // every job, is left alone).  Returns the workers bound.
  int pin(const std::vector<int>& cpus);

 private:
  void worker(int id);
  int n_;
  std::vector<std::thread> threads_;
  std::mutex mu_;
  std::condition_variable cv_;
  const std::function<void(int, int)>* job_ = nullptr;
  std::atomic<uint64_t> gen_{0};
  std::atomic<int> pending_{0};
  std::atomic<int> sleepers_{0};
  std::atomic<bool> stop_{false};
};

// Host placement: the NUMA node of a PCI device ("0000:75:00.0"; -1 when the platform
// reports none), the CPUs of a node that this process may run on, and the Linux cpulist
// format ("0-3,8,10-11") they are read in.
int pci_numa_node(const char* pci_bus_id);
std::vector<int> numa_node_cpus(int node);
std::vector<int> parse_cpulist(const char* text);

// SwiGLU FFN of one expert blob on host cores: y[t] = W_d bf16(silu(W_g x_t) * (W_u x_t)),
// fp32 accumulation, x as bf16 bits [T][H], y fp32 [T][H].  pool may be null.
int host_expert_ffn(ThreadPool* pool, const BlobLayout& L, const uint8_t* blob,
                    const uint16_t* x, int T, float* y);

// The split rule: q = floor(m Bp / Bh + 1/2) clamped to [0, m].
int qstar_split(int m, double Bp, double Bh, int* q, double* qstar);
// Its makespan variant: the integer q in [0, m] minimising max(q / Bp, (m - q) / (Bh - Bp)),
// lowest q on ties; Bh <= Bp gives m.
int qstar_makespan(int m, double Bp, double Bh, int* q);
// The load variant: the q in [0, m] minimising max(max(g0 t_gpu, q blob / Bp) + q t_gpu,
// (m - q) blob / (Bh - Bp)), lowest q on ties; Bh <= Bp gives m.
int qstar_load(int m, int g0, double Bp, double Bh, double blob, double t_gpu, int* q);
// One step of the running estimate of a bandwidth: est + alpha (obs - est); observations
// that are not positive and finite leave it unchanged.
double bandwidth_update(double est, double obs, double alpha);

// Expert-slot LRU: streamed misses are admitted into the lowest empty slot, else into the
// slot with the oldest last use among slots not used in this step (ties: lower slot).
struct LruState {
  std::vector<int32_t> e2s, s2e;
  std::vector<int64_t> last_use;
  std::vector<uint8_t> pref;   // slot filled by a cross-layer prefetch and not used since
  int64_t step = 0;
  void init(int E, int S, bool resident);
  // returns the slot to admit into and the evicted expert (-1 if none), or slot -1 when no
  // slot can be taken in this step
  int take_slot(int64_t now, int32_t* evicted) const;
};

}  // namespace ft
