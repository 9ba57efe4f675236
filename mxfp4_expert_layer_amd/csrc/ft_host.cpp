// Host-side pieces of libft: errors, thread pool, host expert FFN, split rule, LRU.
#include "ft_host.h"

#include <immintrin.h>

#include <algorithm>
#include <chrono>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <new>
#include <system_error>
#include <cctype>
#include <fstream>
#include <string>

#include <pthread.h>
#include <sched.h>

namespace ft {

static thread_local std::string g_last_error;

void set_error(const std::string& msg) { g_last_error = msg; }
int fail(int code, const std::string& msg) {
  g_last_error = msg;
  return code;
}

int caught(const char* who) {
  try {
    throw;
  } catch (const std::bad_alloc&) {
    return fail(FT_ENOMEM, std::string(who) + ": out of host memory");
  } catch (const std::system_error& e) {
    return fail(FT_ENOMEM, std::string(who) + ": " + e.what());
  } catch (const std::exception& e) {
    return fail(FT_ESTATE, std::string(who) + ": " + e.what());
  } catch (...) {
    return fail(FT_ESTATE, std::string(who) + ": unknown exception");
  }
}

}  // namespace ft

extern "C" FT_API const char* ft_last_error(void) { return ft::g_last_error.c_str(); }

namespace ft {

// ---- thread pool ------------------------------------------------------------------------
ThreadPool::ThreadPool(int n_threads) : n_(std::max(1, n_threads)) {
  for (int i = 0; i < n_ - 1; ++i) threads_.emplace_back([this, i] { worker(i); });
}

ThreadPool::~ThreadPool() {
  {
    std::lock_guard<std::mutex> lk(mu_);
    stop_.store(true);
  }
  cv_.notify_all();
  for (auto& t : threads_) t.join();
}

void ThreadPool::worker(int id) {
  using sclock = std::chrono::steady_clock;
  constexpr auto kSpin = std::chrono::microseconds(500);
  uint64_t seen = 0;
  for (;;) {
    // spin for the next job, then sleep until one comes (gen_ changes under mu_, and a
    // sleeper registers under mu_, so no wake-up is lost)
    uint64_t g = gen_.load(std::memory_order_acquire);
    const auto t0 = sclock::now();
    for (int i = 0; g == seen && !stop_.load(std::memory_order_relaxed); ++i) {
      __builtin_ia32_pause();
      if ((i & 255) == 255 && sclock::now() - t0 > kSpin) {
        std::unique_lock<std::mutex> lk(mu_);
        sleepers_.fetch_add(1);
        cv_.wait(lk, [&] { return stop_.load() || gen_.load() != seen; });
        sleepers_.fetch_sub(1);
      }
      g = gen_.load(std::memory_order_acquire);
    }
    if (stop_.load()) return;
    seen = g;
    (*job_)(id, n_);
    pending_.fetch_sub(1, std::memory_order_release);
  }
}

int ThreadPool::pin(const std::vector<int>& cpus) {
  if (cpus.empty()) return 0;
  cpu_set_t set;
  CPU_ZERO(&set);
  for (int c : cpus)
    if (c >= 0 && c < CPU_SETSIZE) CPU_SET(c, &set);
  int n = 0;
  for (auto& t : threads_)
    if (pthread_setaffinity_np(t.native_handle(), sizeof(set), &set) == 0) ++n;
  return n;
}

std::vector<int> parse_cpulist(const char* text) {
  std::vector<int> out;
  const char* p = text;
  while (p && *p) {
    while (*p == ',' || *p == ' ' || *p == '\n') ++p;
    if (!*p) break;
    char* end = nullptr;
    const long a = std::strtol(p, &end, 10);
    if (end == p || a < 0) return {};
    long b = a;
    p = end;
    if (*p == '-') {
      b = std::strtol(p + 1, &end, 10);
      if (end == p + 1 || b < a) return {};
      p = end;
    }
    for (long c = a; c <= b && c < 1 << 16; ++c) out.push_back((int)c);
    if (*p && *p != ',' && *p != '\n' && *p != ' ') return {};
  }
  return out;
}

static std::string read_text(const std::string& path) {
  std::ifstream f(path);
  std::string s;
  if (f) std::getline(f, s);
  return s;
}

int pci_numa_node(const char* pci_bus_id) {
  std::string id(pci_bus_id ? pci_bus_id : "");
  for (auto& c : id) c = (char)std::tolower((unsigned char)c);
  const std::string v = read_text("/sys/bus/pci/devices/" + id + "/numa_node");
  if (v.empty()) return -1;
  return std::atoi(v.c_str());
}

std::vector<int> numa_node_cpus(int node) {
  if (node < 0) return {};
  const std::string v =
      read_text("/sys/devices/system/node/node" + std::to_string(node) + "/cpulist");
  std::vector<int> cpus = parse_cpulist(v.c_str()), out;
  cpu_set_t allowed;
  CPU_ZERO(&allowed);
  if (sched_getaffinity(0, sizeof(allowed), &allowed) != 0) return {};
  for (int c : cpus)
    if (c < CPU_SETSIZE && CPU_ISSET(c, &allowed)) out.push_back(c);
  return out;
}

void ThreadPool::run(const std::function<void(int, int)>& fn) {
  if (n_ == 1) {
    fn(0, 1);
    return;
  }
  job_ = &fn;
  pending_.store(n_ - 1, std::memory_order_relaxed);
  {
    std::lock_guard<std::mutex> lk(mu_);
    gen_.fetch_add(1, std::memory_order_release);
  }
  if (sleepers_.load() > 0) cv_.notify_all();
  fn(n_ - 1, n_);
  while (pending_.load(std::memory_order_acquire) != 0) __builtin_ia32_pause();
}

// ---- host expert FFN ------------------------------------------------------------------------
// E2M1 magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6} with the sign bit (OCP MX v1.0 FP4 table).
static const float kE2M1[16] = {0.f,  0.5f,  1.f,  1.5f,  2.f,  3.f,  4.f,  6.f,
                                -0.f, -0.5f, -1.f, -1.5f, -2.f, -3.f, -4.f, -6.f};

static inline float e8m0_value(uint8_t e) {
  if (e == 255) return NAN;
  if (e == 0) return std::ldexp(1.0f, -127);
  return std::ldexp(1.0f, (int)e - 127);
}

static inline float e4m3_value(uint8_t c) {
  const int e = (c >> 3) & 15, m = c & 7;
  float v;
  if (e == 15 && m == 7) v = NAN;
  else if (e == 0) v = std::ldexp((float)m / 8.f, -6);
  else v = std::ldexp(1.f + (float)m / 8.f, e - 7);
  return (c & 0x80) ? -v : v;
}

static inline float bf16_to_f32(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

static inline float round_to_bf16(float f) {
  uint32_t b;
  std::memcpy(&b, &f, 4);
  if ((b & 0x7fffffffu) > 0x7f800000u) return f;
  b += 0x7fffu + ((b >> 16) & 1u);
  b &= 0xffff0000u;
  std::memcpy(&f, &b, 4);
  return f;
}

// acc[t][r] += sum over K of W[r][K] * xs[t][K] for rows [rt0*16, rt1*16) of a tiled matrix.
// Block sums are formed on unscaled E2M1 values and scaled once per 32 (MXFP4) or 16 (NVFP4)
// elements; with power-of-two MX scales this is exact reassociation.
static void gemv_tiles(const BlobLayout& L, const uint8_t* codes, const uint8_t* scales, int K,
                       int rt0, int rt1, const float* xs, int T, float tensor_scale,
                       float* acc /* [T][R] */, int R) {
  const int KC = K / kTileK;
  const bool mx = L.fmt == FT_MXFP4;
  for (int rt = rt0; rt < rt1; ++rt) {
    for (int kc = 0; kc < KC; ++kc) {
      const uint64_t tile = (uint64_t)rt * KC + kc;
      const uint8_t* c = codes + tile * kTileCodeBytes;
      const uint8_t* s = scales + tile * (mx ? 64 : 128);
      for (int l = 0; l < 64; ++l) {
        const int row = rt * kTileRows + (l & 15);
        const int k0 = kc * kTileK + 32 * (l >> 4);
        float w[32];
        const uint8_t* cb = c + 16 * l;
        for (int b = 0; b < 16; ++b) {
          w[2 * b] = kE2M1[cb[b] & 15];
          w[2 * b + 1] = kE2M1[cb[b] >> 4];
        }
        float s0, s1;
        if (mx) {
          s0 = s1 = e8m0_value(s[l]);
        } else {
          s0 = e4m3_value(s[2 * l]) * tensor_scale;
          s1 = e4m3_value(s[2 * l + 1]) * tensor_scale;
        }
        for (int t = 0; t < T; ++t) {
          const float* xv = xs + (uint64_t)t * K + k0;
          float p0 = 0.f, p1 = 0.f;
          for (int q = 0; q < 16; ++q) p0 += w[q] * xv[q];
          for (int q = 16; q < 32; ++q) p1 += w[q] * xv[q];
          acc[(uint64_t)t * R + row] += p0 * s0 + p1 * s1;
        }
      }
    }
  }
}

// AVX-512 (BF16) path for MXFP4 tiles.  Per 32-value lane block: the 16 code bytes expand
// to 32 nibble indices in 16-bit lanes, which index a 16-entry bf16 table of E2M1 values
// scaled by the block's E8M0 scale (the scale is added to the exponent field of the nonzero
// entries), and vdpbf16ps accumulates the products with the bf16 activations into 16 fp32
// lanes per row.  acc[row] sums for rows rt*16 .. rt*16+15.  The table trick is exact when
// every scaled E2M1 value is a normal bf16 number.  Adding s - 127 to the exponent field
// keeps 0.5 (field 126) at or above 1 for s >= 2 and 6.0 (field 129) at or below 254 for
// s <= 252, so the scale codes taken here are 2..252 (0.5 * 2^-125 .. 6 * 2^125); at 253 the
// entries of 4 and 6 would land on the infinity/NaN field.  A row tile with any other scale
// code (including the NaN code 255) goes to the scalar path, which follows the format
// definition for every code (xs: x as fp32).
// Whether the KC * 64 E8M0 codes of one row tile all lie in 2..252.
__attribute__((target("avx512f,avx512bw")))
static bool mx_scale_row_in_range(const uint8_t* s, int KC) {
  __mmask64 bad = 0;
  for (int kc = 0; kc < KC; ++kc) {
    const __m512i v = _mm512_loadu_si512((const void*)(s + 64 * kc));
    bad |= _mm512_cmp_epu8_mask(v, _mm512_set1_epi8(2), _MM_CMPINT_LT) |
           _mm512_cmp_epu8_mask(v, _mm512_set1_epi8((char)252), _MM_CMPINT_NLE);
  }
  return bad == 0;
}

__attribute__((target("avx512f,avx512bw,avx512bf16,avx512vl")))
static void gemv_tiles_mx_avx512(const BlobLayout& L, const uint8_t* codes,
                                 const uint8_t* scales, int K, int rt0, int rt1,
                                 const uint16_t* xb, const float* xs, int T, float* acc_out,
                                 int R) {
  const int KC = K / kTileK;
  // bf16 bits of E2M1 codes 0..15 (0, .5, 1, 1.5, 2, 3, 4, 6 and their negatives)
  alignas(64) static const uint16_t kBase[32] = {
      0x0000, 0x3F00, 0x3F80, 0x3FC0, 0x4000, 0x4040, 0x4080, 0x40C0,
      0x8000, 0xBF00, 0xBF80, 0xBFC0, 0xC000, 0xC040, 0xC080, 0xC0C0,
      0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
  const __m512i base = _mm512_load_si512((const void*)kBase);
  const __mmask32 nonzero = 0x0000FEFEu;  // entries 1..7 and 9..15
  const __m512i m15 = _mm512_set1_epi32(15);
  for (int rt = rt0; rt < rt1; ++rt) {
    if (!mx_scale_row_in_range(scales + (uint64_t)rt * KC * 64, KC)) {
      gemv_tiles(L, codes, scales, K, rt, rt + 1, xs, T, 1.0f, acc_out, R);
      continue;
    }
    for (int t = 0; t < T; ++t) {
      const uint16_t* xt = xb + (uint64_t)t * K;
      __m512 acc[16];
      for (int r = 0; r < 16; ++r) acc[r] = _mm512_setzero_ps();
      for (int kc = 0; kc < KC; ++kc) {
        const uint64_t tile = (uint64_t)rt * KC + kc;
        const uint8_t* c = codes + tile * kTileCodeBytes;
        const uint8_t* sc = scales + tile * 64;
        __m512bh xv[4];
        for (int g = 0; g < 4; ++g)
          xv[g] = (__m512bh)_mm512_loadu_si512((const void*)(xt + kc * kTileK + 32 * g));
        for (int l = 0; l < 64; ++l) {
          const __m512i bytes = _mm512_cvtepu8_epi32(_mm_loadu_si128((const __m128i*)(c + 16 * l)));
          const __m512i idx = _mm512_or_si512(_mm512_and_si512(bytes, m15),
                                              _mm512_slli_epi32(_mm512_srli_epi32(bytes, 4), 16));
          // (s - 127) << 7 as a 16-bit two's-complement pattern (unsigned arithmetic: a left
          // shift of a negative value is undefined)
          const __m512i shift =
              _mm512_set1_epi16((short)(uint16_t)(((uint32_t)sc[l] - 127u) << 7));
          const __m512i table = _mm512_mask_add_epi16(base, nonzero, base, shift);
          const __m512bh w = (__m512bh)_mm512_permutexvar_epi16(idx, table);
          acc[l & 15] = _mm512_dpbf16_ps(acc[l & 15], w, xv[l >> 4]);
        }
      }
      for (int r = 0; r < 16; ++r)
        acc_out[(uint64_t)t * R + rt * kTileRows + r] += _mm512_reduce_add_ps(acc[r]);
    }
  }
}

static bool have_avx512_bf16() {
  static const bool ok = __builtin_cpu_supports("avx512f") && __builtin_cpu_supports("avx512bw") &&
                         __builtin_cpu_supports("avx512bf16");
  return ok;
}

int host_expert_ffn(ThreadPool* pool, const BlobLayout& L, const uint8_t* blob,
                    const uint16_t* x, int T, float* y) {
  const int H = L.H, I = L.I;
  BlobHeader hdr;
  std::memcpy(&hdr, blob, sizeof(hdr));
  if (hdr.magic != kBlobMagic || hdr.fmt != L.fmt || hdr.H != H || hdr.I != I)
    return fail(FT_EINVAL, "host_expert_ffn: blob header does not match the layer");
  std::vector<float> xs((size_t)T * H), g((size_t)T * I, 0.f), u((size_t)T * I, 0.f),
      h((size_t)T * I);
  std::vector<uint16_t> hb((size_t)T * I);
  std::fill(y, y + (size_t)T * H, 0.f);
  const int RTg = I / kTileRows, RTd = H / kTileRows;
  const char* force_scalar = std::getenv("FT_HOST_SCALAR");
  const bool fast = L.fmt == FT_MXFP4 && have_avx512_bf16() &&
                    !(force_scalar && *force_scalar == '1');
  for (size_t i = 0; i < xs.size(); ++i) xs[i] = bf16_to_f32(x[i]);
  if (fast) {
    auto part = [&](int n, int i, int total, int* a, int* b) {
      *a = (int)((int64_t)total * i / n);
      *b = (int)((int64_t)total * (i + 1) / n);
    };
    auto job = [&](int i, int n) {
      int a, b;
      part(n, i, RTg, &a, &b);
      gemv_tiles_mx_avx512(L, blob + L.off[0], blob + L.off[1], H, a, b, x, xs.data(), T,
                           g.data(), I);
      gemv_tiles_mx_avx512(L, blob + L.off[2], blob + L.off[3], H, a, b, x, xs.data(), T,
                           u.data(), I);
      // SwiGLU of this thread's rows
      for (int t = 0; t < T; ++t)
        for (int r = a * kTileRows; r < b * kTileRows; ++r) {
          const size_t q = (size_t)t * I + r;
          const float z = g[q];
          const float hv = round_to_bf16(z / (1.0f + std::exp(-z)) * u[q]);
          uint32_t bits;
          std::memcpy(&bits, &hv, 4);
          hb[q] = (uint16_t)(bits >> 16);
          h[q] = hv;
        }
    };
    if (pool) pool->run(job); else job(0, 1);
    auto job2 = [&](int i, int n) {
      int a, b;
      part(n, i, RTd, &a, &b);
      gemv_tiles_mx_avx512(L, blob + L.off[4], blob + L.off[5], I, a, b, hb.data(), h.data(), T,
                           y, H);
    };
    if (pool) pool->run(job2); else job2(0, 1);
    return FT_OK;
  }
  auto part = [&](int n, int i, int total, int* a, int* b) {
    *a = (int)((int64_t)total * i / n);
    *b = (int)((int64_t)total * (i + 1) / n);
  };
  auto job = [&](int i, int n) {
    int a, b;
    part(n, i, RTg, &a, &b);
    gemv_tiles(L, blob + L.off[0], blob + L.off[1], H, a, b, xs.data(), T, hdr.tensor_scale[0],
               g.data(), I);
    gemv_tiles(L, blob + L.off[2], blob + L.off[3], H, a, b, xs.data(), T, hdr.tensor_scale[1],
               u.data(), I);
    for (int t = 0; t < T; ++t)      // SwiGLU of this thread's rows
      for (int r = a * kTileRows; r < b * kTileRows; ++r) {
        const size_t q = (size_t)t * I + r;
        h[q] = round_to_bf16(g[q] / (1.0f + std::exp(-g[q])) * u[q]);
      }
  };
  auto job2 = [&](int i, int n) {
    int a, b;
    part(n, i, RTd, &a, &b);
    gemv_tiles(L, blob + L.off[4], blob + L.off[5], I, a, b, h.data(), T, hdr.tensor_scale[2],
               y, H);
  };
  if (pool) pool->run(job); else job(0, 1);
  if (pool) pool->run(job2); else job2(0, 1);
  return FT_OK;
}

// ---- split rule ----------------------------------------------------------------------------
int qstar_split(int m, double Bp, double Bh, int* q, double* qstar) {
  if (m < 0 || !(Bp > 0.0) || !(Bh > 0.0))
    return fail(FT_EINVAL, "ft_qstar_split: need m >= 0, Bp > 0 and Bh > 0");
  const double qs = (double)m * Bp / Bh;
  double r = std::floor(qs + 0.5);
  if (r < 0) r = 0;
  if (r > m) r = m;
  if (qstar) *qstar = qs;
  if (q) *q = (int)r;
  return FT_OK;
}

// Both sides of the split run at once: q experts over PCIe at Bp while the host computes the
// other m - q with the bandwidth the copies leave it, Bh - Bp (lowalt article, section 二).
// The finishing time of q is the later of the two.
int qstar_makespan(int m, double Bp, double Bh, int* q) {
  if (m < 0 || !(Bp > 0.0) || !(Bh > 0.0))
    return fail(FT_EINVAL, "ft_qstar_split_makespan: need m >= 0, Bp > 0 and Bh > 0");
  int best = m;
  if (Bh > Bp) {
    double best_t = 0.0;
    for (int c = 0; c <= m; ++c) {
      const double t = std::max((double)c / Bp, (double)(m - c) / (Bh - Bp));
      if (c == 0 || t < best_t) { best = c; best_t = t; }
    }
  }
  if (q) *q = best;
  return FT_OK;
}

int qstar_load(int m, int g0, double Bp, double Bh, double blob, double t_gpu, int* q) {
  if (m < 0 || g0 < 0 || !(Bp > 0.0) || !(Bh > 0.0) || !(blob > 0.0) || !(t_gpu >= 0.0) ||
      !std::isfinite(t_gpu))
    return fail(FT_EINVAL, "ft_qstar_split_load: need m, g0 >= 0, Bp, Bh, blob > 0 and a "
                           "finite t_gpu >= 0");
  int best = m;
  if (Bh > Bp) {
    double best_t = 0.0;
    for (int c = 0; c <= m; ++c) {
      const double gpu = std::max(g0 * t_gpu, c * blob / Bp) + c * t_gpu;
      const double host = (m - c) * blob / (Bh - Bp);
      const double t = std::max(gpu, host);
      if (c == 0 || t < best_t) { best = c; best_t = t; }
    }
  }
  if (q) *q = best;
  return FT_OK;
}

double bandwidth_update(double est, double obs, double alpha) {
  if (!(obs > 0.0) || !std::isfinite(obs)) return est;
  return est + alpha * (obs - est);
}

// ---- LRU ------------------------------------------------------------------------------------
void LruState::init(int E, int S, bool resident) {
  e2s.assign(E, -1);
  s2e.assign(S, -1);
  last_use.assign(S, -1);
  pref.assign(S, 0);
  step = 0;
  if (resident)
    for (int e = 0; e < E && e < S; ++e) { e2s[e] = e; s2e[e] = e; }
}

int LruState::take_slot(int64_t now, int32_t* evicted) const {
  *evicted = -1;
  const int S = (int)s2e.size();
  for (int s = 0; s < S; ++s)
    if (s2e[s] < 0) return s;
  int best = -1;
  for (int s = 0; s < S; ++s)
    if (last_use[s] < now && (best < 0 || last_use[s] < last_use[best])) best = s;
  if (best >= 0) *evicted = s2e[best];
  return best;
}

}  // namespace ft
