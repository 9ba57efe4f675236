// C ABI of libft: contexts, layers, decode (resident and miss paths), probes, test hooks.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <system_error>
#include <stdexcept>
#include <chrono>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <memory>
#include <new>
#include <string>
#include <vector>

#include "ft_ftw.h"
#include "ft_host.h"

using namespace ft;

// kernel launchers (ft_decode.hip, ft_debug.hip)
extern "C" int ftk_logits(const uint16_t* x, const float* wr, const float* b, int T, int H, int E,
                          float* logits, hipStream_t st);
extern "C" int ftk_topk(const float* logits, int T, int E, int k, int32_t* idx_out, float* w_out,
                        int32_t* idx_host, float* w_host, const uint16_t* x, uint16_t* x_host,
                        int H, hipStream_t st);
extern "C" int ftk_decode_experts(const DecodeLaunch* a, hipStream_t st, const hipEvent_t* ev);
extern "C" int ftk_down_combines(const DecodeLaunch* a);
extern "C" int ftk_route_small(const RouteSmall* a, hipStream_t st);
extern "C" int ftk_read_probe(const void* buf, uint64_t bytes, uint32_t* sink, int grid,
                              int lds_form, hipStream_t st);
extern "C" int ftk_residual(const uint16_t* x, const float* y, float sc, int64_t n, uint16_t* out,
                            hipStream_t st);
extern "C" int ftk_combine(const float* P, const float* w, int T, int H, int k, int n_shared,
                           float* y, hipStream_t st);
extern "C" int ftk_dequant(const uint8_t* blob, const BlobLayout* L, int matrix, float ts,
                           float* out, hipStream_t st);
extern "C" int ftk_split_router(const float* wr, int E, int H, uint16_t* planes, hipStream_t st);
extern "C" int ftk_prefill(const PrefillLaunch* a, hipStream_t st, const hipEvent_t* ev);
extern "C" int ftk_nv_to_mx(const uint8_t* src, uint8_t* dst, const BlobLayout* S,
                            const BlobLayout* D, hipStream_t st);
extern "C" int ftk_static_scratch(int device, void** addr, size_t* bytes);
extern "C" int ftk_untile_h(const PrefillLaunch* a, uint8_t* codes, uint8_t* scales,
                            hipStream_t st);

namespace {

using clk = std::chrono::steady_clock;
double us_since(clk::time_point t0) {
  return std::chrono::duration<double, std::micro>(clk::now() - t0).count();
}

#define HIP_TRY(expr)                                                                   \
  do {                                                                                   \
    hipError_t e_ = (expr);                                                              \
    if (e_ != hipSuccess)                                                                \
      return fail(FT_EHIP, std::string(#expr) + ": " + hipGetErrorString(e_));           \
  } while (0)

int env_int(const char* name, int dflt) {
  const char* v = std::getenv(name);
  return v && *v ? std::atoi(v) : dflt;
}

}  // namespace

struct ft_ctx {
  int device = 0;
  hipStream_t copy_stream = nullptr;
  std::unique_ptr<ThreadPool> pool;
  // device address and size of the library's static scratch on this device
  // (ft_moe_prefill_noalloc), looked up once per device at context creation
  void* scratch = nullptr;
  size_t scratch_bytes = 0;
  // host placement: the GPU's NUMA node (-1 if the platform reports none) and the CPUs of
  // that node the pool's workers are bound to (0: not bound)
  int numa_node = -1;
  int pinned_cpus = 0;
};

namespace ft {
ThreadPool* ctx_pool(ft_ctx* c) { return c ? c->pool.get() : nullptr; }
}  // namespace ft

struct ft_layer {
  ft_ctx* ctx = nullptr;
  ft_layer_desc d{};
  BlobLayout L{};
  int kk = 0;            // k + n_shared
  int max_items = 0;     // work-list entries per call
  bool all_resident = false;
  // device workspace (one allocation)
  void* dev = nullptr;
  float* logits = nullptr;
  int32_t* idx = nullptr;
  float* w = nullptr;
  // n_items, e2s_dev, s2e_dev and items are one block laid out as the pinned n_items_h ..
  // items_h block, so the miss path refreshes them with one copy
  WorkItem* items = nullptr;     // 2 * max_items (miss path: hits, then streamed misses)
  int* n_items = nullptr;        // [2]
  uint16_t* h = nullptr;
  float* P = nullptr;
  int32_t* e2s_dev = nullptr;
  int32_t* s2e_dev = nullptr;
  unsigned int* route_counter = nullptr;   // k_route_small's workgroup counter
  uint32_t* route_flag_h = nullptr;        // pinned: the last routing launch's sequence number
  uint32_t route_seq = 0;
  uint16_t* wr_planes = nullptr;  // bf16 split of router_w in MFMA operand order (prefill router)
  // MXFP4 weights of the scaled-FP4 prefill: the pool itself (MXFP4 layers) or a transcoded
  // copy owned here (NVFP4 layers created with FT_LAYER_PREFILL_MXFP4); null if neither
  const uint8_t* mx_pool = nullptr;
  uint64_t mx_stride = 0;
  void* mx_owned = nullptr;
  // pinned host staging
  void* pin = nullptr;
  uint8_t* pin_dev = nullptr;    // device address of the mapped pinned staging
  int32_t* idx_h = nullptr;
  float* w_h = nullptr;
  uint16_t* x_h = nullptr;
  WorkItem* items_h = nullptr;   // 2 * max_items
  int* n_items_h = nullptr;      // [2]
  float* P_h = nullptr;          // host expert outputs [T * kk][H]
  int32_t* e2s_h = nullptr;
  int32_t* s2e_h = nullptr;
  hipEvent_t ev_copy = nullptr;
  hipEvent_t ev_route = nullptr;
  hipEvent_t ev_cp0 = nullptr, ev_cp1 = nullptr;   // timing events around streamed copies
  hipEvent_t ev_g0 = nullptr, ev_g1 = nullptr;     // around the hit experts' kernels
  int pend_gpu_items = 0;        // experts of the last call timed by ev_g0/ev_g1
  double t_gpu = 0.0;            // GPU seconds per expert (FT_SPLIT_LOAD)
  // policy state
  LruState lru;
  double bp = 0.0, bh = 0.0;
  int force_q = -1;
  int split_rule = FT_SPLIT_ROUND;
  double alpha = 0.0;            // running-estimate weight (0: Bp and Bh fixed)
  uint64_t pend_copy_bytes = 0;  // streamed bytes of the last call, timed by ev_cp0/ev_cp1
  hipEvent_t ev_done = nullptr;  // after the kernels of the last miss-path call
  // cross-layer prefetch: this layer predicts and fills `next`'s pool (ft_set_prefetch)
  ft_layer* next = nullptr;
  ft_layer* prev = nullptr;      // the layer whose calls prefetch into this one
  int pf_depth = 0;
  void* pf_dev = nullptr;        // prediction logits [16][1024], idx, w [16][16]
  float* pf_logits = nullptr;
  int32_t* pf_idx = nullptr;
  float* pf_w = nullptr;
  void* pf_pin = nullptr;        // mapped pinned idx, w of the prediction
  int32_t* pf_idx_h = nullptr;
  float* pf_w_h = nullptr;
  int32_t* pf_idx_hd = nullptr;  // their device addresses
  float* pf_w_hd = nullptr;
  hipEvent_t ev_pref = nullptr;  // after the prefetch copies into this layer's pool
  bool pref_pending = false;
  // host-memory tier over an FTW file (ft_layer_set_disk_tier): n_ram slots in `ram`
  ft_ftw* ftw = nullptr;
  uint8_t* ram = nullptr;
  int n_ram = 0;
  LruState ram_lru;
  // kernel timing events: [n][4] = gate/up start, stop, down start, stop
  std::vector<hipEvent_t> prof;
  int prof_n = 0, prof_i = 0;
};

// the four timing events of the next profiled call, or null
static const hipEvent_t* prof_events(ft_layer* l) {
  if (l->prof_i >= l->prof_n) return nullptr;
  return &l->prof[(size_t)4 * l->prof_i++];
}

// ---- blobs ------------------------------------------------------------------------------------
// H, I multiples of 128, and one blob under 2 GiB: the GEMM kernels address a blob through
// buffer resources, whose extent and offsets are 32-bit.
static bool dims_ok(int format, int H, int I) {
  return (format == FT_MXFP4 || format == FT_NVFP4) && H > 0 && I > 0 && H % kTileK == 0 &&
         I % kTileK == 0 && blob_layout(format, H, I).bytes < (1ull << 31);
}

extern "C" FT_API int ft_blob_bytes(int format, int H, int I, uint64_t* bytes) try {
  if (!bytes || !dims_ok(format, H, I))
    return fail(FT_EINVAL, "ft_blob_bytes: format must be FT_MXFP4/FT_NVFP4 and H, I positive "
                           "multiples of 128 with a blob under 2 GiB");
  *bytes = blob_layout(format, H, I).bytes;
  return FT_OK;
} FT_CATCH("ft_blob_bytes")

static void pack_matrix(int fmt, int R, int K, const uint8_t* codes, const uint8_t* scales,
                        uint8_t* dst_codes, uint8_t* dst_scales) {
  const int KC = K / kTileK, RT = R / kTileRows;
  const int B = fmt == FT_MXFP4 ? 32 : 16;
  const int sbytes = scale_tile_bytes(fmt);
  for (int rt = 0; rt < RT; ++rt)
    for (int kc = 0; kc < KC; ++kc) {
      const uint64_t tile = (uint64_t)rt * KC + kc;
      uint8_t* tc = dst_codes + tile * kTileCodeBytes;
      uint8_t* ts = dst_scales + tile * sbytes;
      for (int l = 0; l < 64; ++l) {
        const int row = rt * kTileRows + (l & 15);
        const int k0 = kc * kTileK + 32 * (l >> 4);
        std::memcpy(tc + 16 * l, codes + (uint64_t)row * (K / 2) + k0 / 2, 16);
        if (fmt == FT_MXFP4) {
          ts[l] = scales[(uint64_t)row * (K / B) + k0 / B];
        } else {
          ts[2 * l] = scales[(uint64_t)row * (K / B) + k0 / B];
          ts[2 * l + 1] = scales[(uint64_t)row * (K / B) + k0 / B + 1];
        }
      }
    }
}

extern "C" FT_API int ft_pack_expert(int format, int H, int I, const uint8_t* gc,
                                     const uint8_t* gs, const uint8_t* uc, const uint8_t* us,
                                     const uint8_t* dc, const uint8_t* ds,
                                     const float* tensor_scales, void* blob) try {
  if (!dims_ok(format, H, I)) return fail(FT_EINVAL, "ft_pack_expert: bad format or sizes");
  if (!gc || !gs || !uc || !us || !dc || !ds || !blob)
    return fail(FT_EINVAL, "ft_pack_expert: null pointer");
  const BlobLayout L = blob_layout(format, H, I);
  uint8_t* b = (uint8_t*)blob;
  std::memset(b, 0, kAlign);
  BlobHeader hdr{};
  hdr.magic = kBlobMagic;
  hdr.fmt = format;
  hdr.H = H;
  hdr.I = I;
  for (int i = 0; i < 3; ++i) hdr.tensor_scale[i] = tensor_scales ? tensor_scales[i] : 1.0f;
  std::memcpy(b, &hdr, sizeof(hdr));
  // zero the alignment padding so blobs are byte-deterministic
  for (int i = 0; i < 6; ++i) {
    const uint64_t end = (i + 1 < 6) ? L.off[i + 1] : L.bytes;
    std::memset(b + L.off[i], 0, end - L.off[i]);
  }
  pack_matrix(format, I, H, gc, gs, b + L.off[0], b + L.off[1]);
  pack_matrix(format, I, H, uc, us, b + L.off[2], b + L.off[3]);
  pack_matrix(format, H, I, dc, ds, b + L.off[4], b + L.off[5]);
  return FT_OK;
} FT_CATCH("ft_pack_expert")

// ---- context ----------------------------------------------------------------------------------
extern "C" FT_API int ft_ctx_create(int device, ft_ctx** out) try {
  if (!out) return fail(FT_EINVAL, "ft_ctx_create: out is null");
  int n = 0;
  HIP_TRY(hipGetDeviceCount(&n));
  if (device < 0 || device >= n) return fail(FT_EINVAL, "ft_ctx_create: no such device");
  HIP_TRY(hipSetDevice(device));
  std::unique_ptr<ft_ctx> c(new (std::nothrow) ft_ctx);
  if (!c) return fail(FT_ENOMEM, "ft_ctx_create: out of host memory");
  c->device = device;
  HIP_TRY((hipError_t)ftk_static_scratch(device, &c->scratch, &c->scratch_bytes));
  HIP_TRY(hipStreamCreateWithFlags(&c->copy_stream, hipStreamNonBlocking));
  const int hw = (int)std::thread::hardware_concurrency();
  const int nt = env_int("FT_HOST_THREADS", std::max(1, std::min(16, hw)));
  c->pool.reset(new ThreadPool(std::max(1, nt)));
  // the host experts read pinned host memory and the copies cross PCIe from it: keep the
  // pool's workers on the GPU's NUMA node (FT_HOST_AFFINITY=0 leaves them unbound)
  char bus[64] = {0};
  if (hipDeviceGetPCIBusId(bus, (int)sizeof(bus), device) == hipSuccess) {
    c->numa_node = pci_numa_node(bus);
    if (env_int("FT_HOST_AFFINITY", 1) != 0) {
      const std::vector<int> cpus = numa_node_cpus(c->numa_node);
      if (!cpus.empty() && c->pool->pin(cpus) > 0) c->pinned_cpus = (int)cpus.size();
    }
  }
  *out = c.release();
  return FT_OK;
} FT_CATCH("ft_ctx_create")

extern "C" FT_API int ft_ctx_numa(const ft_ctx* ctx, int* node, int* pinned_cpus) try {
  if (!ctx || !node || !pinned_cpus) return fail(FT_EINVAL, "ft_ctx_numa: null argument");
  *node = ctx->numa_node;
  *pinned_cpus = ctx->pinned_cpus;
  return FT_OK;
} FT_CATCH("ft_ctx_numa")

extern "C" FT_API int ft_debug_parse_cpulist(const char* text, int32_t* cpus, int cap,
                                             int* n) try {
  if (!text || !n || (cap > 0 && !cpus)) return fail(FT_EINVAL, "ft_debug_parse_cpulist: null");
  const std::vector<int> v = parse_cpulist(text);
  *n = (int)v.size();
  for (int i = 0; i < (int)v.size() && i < cap; ++i) cpus[i] = v[i];
  return FT_OK;
} FT_CATCH("ft_debug_parse_cpulist")

extern "C" FT_API int ft_ctx_destroy(ft_ctx* ctx) try {
  if (!ctx) return FT_OK;
  if (ctx->copy_stream) {
    hipSetDevice(ctx->device);
    hipStreamSynchronize(ctx->copy_stream);
    hipStreamDestroy(ctx->copy_stream);
  }
  delete ctx;
  return FT_OK;
} FT_CATCH("ft_ctx_destroy")

// ---- layer ------------------------------------------------------------------------------------
template <class T>
static T* carve(uint8_t*& p, size_t n) {
  T* r = (T*)p;
  p += align_up(n * sizeof(T), 256);
  return r;
}

static void free_layer(ft_layer* l) {
  if (!l) return;
  for (hipEvent_t e : l->prof) hipEventDestroy(e);
  if (l->ev_copy) hipEventDestroy(l->ev_copy);
  if (l->ev_route) hipEventDestroy(l->ev_route);
  if (l->ev_cp0) hipEventDestroy(l->ev_cp0);
  if (l->ev_cp1) hipEventDestroy(l->ev_cp1);
  if (l->ev_g0) hipEventDestroy(l->ev_g0);
  if (l->ev_g1) hipEventDestroy(l->ev_g1);
  if (l->ev_done) hipEventDestroy(l->ev_done);
  if (l->ev_pref) hipEventDestroy(l->ev_pref);
  if (l->pf_dev) hipFree(l->pf_dev);
  if (l->pf_pin) hipHostFree(l->pf_pin);
  if (l->dev) hipFree(l->dev);
  if (l->mx_owned) hipFree(l->mx_owned);
  if (l->pin) hipHostFree(l->pin);
  delete l;
}

extern "C" FT_API int ft_layer_create(ft_ctx* ctx, const ft_layer_desc* desc, ft_layer** out) try {
  if (!ctx || !desc || !out) return fail(FT_EINVAL, "ft_layer_create: null argument");
  const ft_layer_desc& d = *desc;
  if (!dims_ok(d.format, d.H, d.I)) return fail(FT_EINVAL, "ft_layer_create: bad format or H/I");
  if (d.E < 1 || d.E > 1024 || d.k < 1 || d.k > FT_MAX_TOPK || d.k > d.E)
    return fail(FT_EINVAL, "ft_layer_create: need 1 <= k <= min(E, 16) and E <= 1024");
  if (d.n_shared < 0 || d.n_shared > 4) return fail(FT_EINVAL, "ft_layer_create: n_shared 0..4");
  if (d.n_slots < 1 || d.n_slots > d.E) return fail(FT_EINVAL, "ft_layer_create: n_slots 1..E");
  if (d.max_tokens < 1 || d.max_tokens > FT_MAX_DECODE_TOKENS)
    return fail(FT_EINVAL, "ft_layer_create: max_tokens 1..16");
  if (!d.router_w || !d.pool) return fail(FT_EINVAL, "ft_layer_create: router_w/pool null");
  if (d.n_shared > 0 && !d.shared_blobs)
    return fail(FT_EINVAL, "ft_layer_create: shared_blobs null with n_shared > 0");
  const BlobLayout L = blob_layout(d.format, d.H, d.I);
  if (d.blob_stride < L.bytes || d.blob_stride % kAlign)
    return fail(FT_EINVAL, "ft_layer_create: blob_stride below ft_blob_bytes() or not a "
                           "multiple of 4096");
  if (d.resident && d.n_slots != d.E)
    return fail(FT_EINVAL, "ft_layer_create: resident layers need n_slots == E");
  if (d.flags & ~FT_LAYER_PREFILL_MXFP4)
    return fail(FT_EINVAL, "ft_layer_create: unknown flags");
  if ((d.flags & FT_LAYER_PREFILL_MXFP4) && d.format == FT_NVFP4 && !d.resident)
    return fail(FT_EINVAL, "ft_layer_create: FT_LAYER_PREFILL_MXFP4 needs a resident layer");
  HIP_TRY(hipSetDevice(ctx->device));

  std::unique_ptr<ft_layer, void (*)(ft_layer*)> l(new (std::nothrow) ft_layer, free_layer);
  if (!l) return fail(FT_ENOMEM, "ft_layer_create: out of host memory");
  l->ctx = ctx;
  l->d = d;
  l->L = L;
  l->kk = d.k + d.n_shared;
  l->max_items = d.max_tokens * d.k + d.n_shared;
  l->all_resident = d.resident != 0;
  const int T = d.max_tokens;

  size_t need = 0;
  auto add = [&](size_t bytes) { need += align_up(bytes, 256); };
  add((size_t)T * d.E * 4);                        // logits
  add((size_t)T * d.k * 4);                        // idx
  add((size_t)T * d.k * 4);                        // w
  add((size_t)2 * l->max_items * sizeof(WorkItem));
  add(2 * sizeof(int));
  add((size_t)l->max_items * kMaxCols * d.I * 2);  // h
  add((size_t)T * l->kk * d.H * 4);                // P
  add((size_t)d.E * 4);
  add((size_t)d.n_slots * 4);
  add(router_plane_bytes(d.E, d.H));               // router planes
  add(sizeof(unsigned int));                       // routing counter
  if (hipMalloc(&l->dev, need) != hipSuccess)
    return fail(FT_ENOMEM, "ft_layer_create: device workspace allocation failed");
  HIP_TRY(hipMemset(l->dev, 0, need));
  uint8_t* p = (uint8_t*)l->dev;
  l->logits = carve<float>(p, (size_t)T * d.E);
  l->idx = carve<int32_t>(p, (size_t)T * d.k);
  l->w = carve<float>(p, (size_t)T * d.k);
  l->n_items = carve<int>(p, 2);
  l->e2s_dev = carve<int32_t>(p, d.E);
  l->s2e_dev = carve<int32_t>(p, d.n_slots);
  l->items = carve<WorkItem>(p, (size_t)2 * l->max_items);
  l->h = carve<uint16_t>(p, (size_t)l->max_items * kMaxCols * d.I);
  l->P = carve<float>(p, (size_t)T * l->kk * d.H);
  l->wr_planes = carve<uint16_t>(p, router_plane_bytes(d.E, d.H) / 2);
  l->route_counter = carve<unsigned int>(p, 1);
  HIP_TRY((hipError_t)ftk_split_router(d.router_w, d.E, d.H, l->wr_planes, nullptr));
  if (d.format == FT_MXFP4 && d.resident) {
    l->mx_pool = (const uint8_t*)d.pool;
    l->mx_stride = d.blob_stride;
  } else if (d.format == FT_NVFP4 && (d.flags & FT_LAYER_PREFILL_MXFP4)) {
    const BlobLayout ML = blob_layout(FT_MXFP4, d.H, d.I);
    if (hipMalloc(&l->mx_owned, (size_t)d.E * ML.bytes) != hipSuccess)
      return fail(FT_ENOMEM, "ft_layer_create: MXFP4 weight copy allocation failed");
    HIP_TRY(hipMemset(l->mx_owned, 0, (size_t)d.E * ML.bytes));
    for (int e = 0; e < d.E; ++e)
      HIP_TRY((hipError_t)ftk_nv_to_mx((const uint8_t*)d.pool + (uint64_t)e * d.blob_stride,
                                       (uint8_t*)l->mx_owned + (uint64_t)e * ML.bytes, &L, &ML,
                                       nullptr));
    l->mx_pool = (const uint8_t*)l->mx_owned;
    l->mx_stride = ML.bytes;
  }
  HIP_TRY(hipDeviceSynchronize());

  size_t pneed = 0;
  auto padd = [&](size_t bytes) { pneed += align_up(bytes, 256); };
  padd((size_t)T * d.k * 4);
  padd((size_t)T * d.k * 4);
  padd((size_t)T * d.H * 2);
  padd((size_t)2 * l->max_items * sizeof(WorkItem));
  padd(2 * sizeof(int));
  padd((size_t)T * l->kk * d.H * 4);
  padd((size_t)d.E * 4);
  padd((size_t)d.n_slots * 4);
  padd(sizeof(uint32_t));
  if (hipHostMalloc(&l->pin, pneed, hipHostMallocMapped) != hipSuccess)
    return fail(FT_ENOMEM, "ft_layer_create: pinned staging allocation failed");
  {
    void* dp = nullptr;
    HIP_TRY(hipHostGetDevicePointer(&dp, l->pin, 0));
    l->pin_dev = (uint8_t*)dp;
  }
  uint8_t* q = (uint8_t*)l->pin;
  l->idx_h = carve<int32_t>(q, (size_t)T * d.k);
  l->w_h = carve<float>(q, (size_t)T * d.k);
  l->x_h = carve<uint16_t>(q, (size_t)T * d.H);
  l->n_items_h = carve<int>(q, 2);
  l->e2s_h = carve<int32_t>(q, d.E);
  l->s2e_h = carve<int32_t>(q, d.n_slots);
  l->items_h = carve<WorkItem>(q, (size_t)2 * l->max_items);
  l->P_h = carve<float>(q, (size_t)T * l->kk * d.H);
  l->route_flag_h = carve<uint32_t>(q, 1);
  *l->route_flag_h = 0;

  l->lru.init(d.E, d.n_slots, l->all_resident);
  std::copy(l->lru.e2s.begin(), l->lru.e2s.end(), l->e2s_h);
  std::copy(l->lru.s2e.begin(), l->lru.s2e.end(), l->s2e_h);
  HIP_TRY(hipMemcpy(l->e2s_dev, l->e2s_h, (size_t)d.E * 4, hipMemcpyHostToDevice));
  HIP_TRY(hipMemcpy(l->s2e_dev, l->s2e_h, (size_t)d.n_slots * 4, hipMemcpyHostToDevice));
  HIP_TRY(hipEventCreateWithFlags(&l->ev_copy, hipEventDisableTiming));
  HIP_TRY(hipEventCreateWithFlags(&l->ev_route, hipEventDisableTiming));
  HIP_TRY(hipEventCreate(&l->ev_cp0));
  HIP_TRY(hipEventCreate(&l->ev_cp1));
  HIP_TRY(hipEventCreate(&l->ev_g0));
  HIP_TRY(hipEventCreate(&l->ev_g1));
  HIP_TRY(hipEventCreateWithFlags(&l->ev_done, hipEventDisableTiming));
  HIP_TRY(hipEventCreateWithFlags(&l->ev_pref, hipEventDisableTiming));
  HIP_TRY(hipEventRecord(l->ev_done, nullptr));
  HIP_TRY(hipEventRecord(l->ev_copy, nullptr));
  *out = l.release();
  return FT_OK;
} FT_CATCH("ft_layer_create")

extern "C" FT_API int ft_layer_destroy(ft_layer* layer) try {
  if (!layer) return FT_OK;
  hipSetDevice(layer->ctx->device);
  hipDeviceSynchronize();
  // unlink prefetching in both directions
  if (layer->prev && layer->prev->next == layer) {
    layer->prev->next = nullptr;
    layer->prev->pf_depth = 0;
  }
  if (layer->next && layer->next->prev == layer) layer->next->prev = nullptr;
  free_layer(layer);
  return FT_OK;
} FT_CATCH("ft_layer_destroy")

// ---- routing / decode ---------------------------------------------------------------------
static int check_call(const ft_ctx* ctx, const ft_layer* layer, const void* x, int T,
                      const char* who) {
  if (!ctx || !layer || !x) return fail(FT_EINVAL, std::string(who) + ": null argument");
  if (layer->ctx != ctx) return fail(FT_EINVAL, std::string(who) + ": layer of another context");
  if (T < 1 || T > layer->d.max_tokens)
    return fail(FT_EINVAL, std::string(who) + ": T must be in 1..max_tokens");
  return FT_OK;
}

extern "C" FT_API int ft_route(ft_ctx* ctx, const ft_layer* layer, const uint16_t* x, int T,
                               int32_t* idx, float* w, void* stream) try {
  int rc = check_call(ctx, layer, x, T, "ft_route");
  if (rc) return rc;
  if (!idx || !w) return fail(FT_EINVAL, "ft_route: idx/w null");
  const ft_layer_desc& d = layer->d;
  HIP_TRY(hipSetDevice(ctx->device));
  hipStream_t st = (hipStream_t)stream;
  HIP_TRY((hipError_t)ftk_logits(x, d.router_w, d.router_b, T, d.H, d.E, layer->logits, st));
  HIP_TRY((hipError_t)ftk_topk(layer->logits, T, d.E, d.k, idx, w, nullptr, nullptr, nullptr,
                               nullptr, d.H, st));
  return FT_OK;
} FT_CATCH("ft_route")

static DecodeLaunch launch_args(ft_layer* l, const uint16_t* x, int T, int route, WorkItem* items,
                                int* n_items, int max_items) {
  const ft_layer_desc& d = l->d;
  DecodeLaunch a{};
  a.x = x;
  a.T = T; a.H = d.H; a.I = d.I; a.E = d.E; a.k = d.k; a.n_shared = d.n_shared;
  a.route = route;
  a.logits = l->logits;
  a.e2s = l->e2s_dev;
  a.idx_out = l->idx;
  a.w_out = l->w;
  a.items = items;
  a.n_items = n_items;
  a.max_items = max_items;
  a.pool = (const uint8_t*)d.pool;
  a.shared = (const uint8_t*)d.shared_blobs;
  a.stride = d.blob_stride;
  a.L = l->L;
  a.h = l->h;
  a.P = l->P;
  return a;
}

static int decode_resident(ft_layer* l, const uint16_t* x, int T, float* y, hipStream_t st) {
  const ft_layer_desc& d = l->d;
  HIP_TRY((hipError_t)ftk_logits(x, d.router_w, d.router_b, T, d.H, d.E, l->logits, st));
  // few tokens: the gate/up kernel takes the top-k itself (one launch less); more tokens:
  // a top-k kernel with one wave per token first, so no workgroup routes tokens serially
  // (measured: in-kernel routing wins up to 4 tokens, the separate pass from 8)
  const int route = T <= 4 ? 1 : 2;
  if (route == 2)
    HIP_TRY((hipError_t)ftk_topk(l->logits, T, d.E, d.k, l->idx, l->w, nullptr, nullptr, nullptr,
                                 nullptr, d.H, st));
  DecodeLaunch a = launch_args(l, x, T, route, l->items, l->n_items, T * d.k + d.n_shared);
  a.y = y;
  HIP_TRY((hipError_t)ftk_decode_experts(&a, st, prof_events(l)));
  if (!ftk_down_combines(&a))
    HIP_TRY((hipError_t)ftk_combine(l->P, l->w, T, d.H, d.k, d.n_shared, y, st));
  return FT_OK;
}

static void add_item(WorkItem* list, int* n, int expert, int slot) {
  WorkItem& it = list[(*n)++];
  std::memset(&it, 0, sizeof(it));
  it.expert = expert;
  it.slot = slot;
}

// Wait for the routing kernel's host-memory flag to reach seq: it is set once the routing is
// in host memory, so neither an event round trip nor a sleeping thread's wake-up sits on the
// critical path of the call.  The launch's event bounds the spin: once the kernel has
// finished, the flag must be there.
static hipError_t wait_route(const uint32_t* flag, uint32_t seq, hipEvent_t ev) {
  for (uint32_t n = 1;; ++n) {
    if (__atomic_load_n(flag, __ATOMIC_ACQUIRE) == seq) return hipSuccess;
    __builtin_ia32_pause();
    if ((n & 1023) == 0) {
      const hipError_t e = hipEventQuery(ev);
      if (e == hipErrorNotReady) continue;
      if (e != hipSuccess) return e;
      if (__atomic_load_n(flag, __ATOMIC_ACQUIRE) == seq) return hipSuccess;
      return hipErrorLaunchFailure;
    }
  }
}

// Cross-layer prefetch into nx's pool for its next call, from the predicted routing idx/w
// [T][k of nx]: the predicted experts already resident are marked used at that call's step
// (so this batch evicts none of them); the others, by descending summed predicted weight
// (ties to the lower id), are admitted through the pool's slot rule at that step, at most
// depth of them, and copied on the copy stream once nx's previous kernels are done.
static int prefetch_into(ft_ctx* ctx, ft_layer* nx, const int32_t* idx, const float* w, int T,
                         int depth, int32_t* n_admitted) {
  const ft_layer_desc& nd = nx->d;
  const int k = nd.k, E = nd.E;
  const int64_t now = nx->lru.step;
  std::vector<double> ws(E, 0.0);
  std::vector<char> sel(E, 0);
  for (int t = 0; t < T; ++t)
    for (int j = 0; j < k; ++j) {
      const int e = idx[t * k + j];
      if (e < 0 || e >= E) return fail(FT_ESTATE, "ft_moe_decode: prediction gave a bad index");
      sel[e] = 1;
      ws[e] += w[t * k + j];
    }
  std::vector<int> order;
  for (int e = 0; e < E; ++e)
    if (sel[e]) order.push_back(e);
  std::stable_sort(order.begin(), order.end(), [&](int a, int b) {
    return ws[a] > ws[b] || (ws[a] == ws[b] && a < b);
  });
  LruState& P = nx->lru;
  for (int e : order)
    if (P.e2s[e] >= 0) P.last_use[P.e2s[e]] = now;
  std::vector<std::pair<int, int>> adm;   // (expert, slot)
  for (int e : order) {
    if ((int)adm.size() >= depth) break;
    if (P.e2s[e] >= 0) continue;
    int32_t old = -1;
    const int s = P.take_slot(now, &old);
    if (s < 0) break;
    if (old >= 0) P.e2s[old] = -1;
    P.s2e[s] = e;
    P.e2s[e] = s;
    P.last_use[s] = now;
    P.pref[s] = 1;
    adm.emplace_back(e, s);
  }
  if (!adm.empty()) {
    HIP_TRY(hipStreamWaitEvent(ctx->copy_stream, nx->ev_done, 0));
    for (const auto& es : adm)
      HIP_TRY(hipMemcpyAsync((uint8_t*)nd.pool + (uint64_t)es.second * nd.blob_stride,
                             (const uint8_t*)nd.host_blobs + (uint64_t)es.first * nd.blob_stride,
                             nx->L.bytes, hipMemcpyHostToDevice, ctx->copy_stream));
    HIP_TRY(hipEventRecord(nx->ev_pref, ctx->copy_stream));
    nx->pref_pending = true;
  }
  *n_admitted = (int32_t)adm.size();
  return FT_OK;
}

// One call's use of the host-memory tier (see ft_layer_set_disk_tier): `needed`, the call's
// VRAM misses in miss order, must be in host memory.  The ones there are marked used at the
// tier's call counter first; the others take slots by the pool's slot rule and are read from
// the FTW file in 1 MiB requests over the host threads.
static int host_tier_step(ft_ctx* ctx, ft_layer* l, const std::vector<int>& needed,
                          ft_decode_stats* S) {
  LruState& P = l->ram_lru;
  const int64_t now = P.step;
  for (int e : needed)
    if (P.e2s[e] >= 0) P.last_use[P.e2s[e]] = now;
  std::vector<int32_t> ids;
  std::vector<uint8_t*> dst;
  for (int e : needed) {
    if (P.e2s[e] >= 0) continue;
    int32_t old = -1;
    const int s = P.take_slot(now, &old);
    if (s < 0) return fail(FT_ESTATE, "ft_moe_decode: host-memory tier smaller than the call's misses");
    if (old >= 0) P.e2s[old] = -1;
    P.s2e[s] = e;
    P.e2s[e] = s;
    P.last_use[s] = now;
    ids.push_back(e);
    dst.push_back(l->ram + (uint64_t)s * l->d.blob_stride);
  }
  P.step++;
  if (ids.empty()) return FT_OK;
  // a refilled slot may still be the source of this layer's earlier copies
  HIP_TRY(hipEventSynchronize(l->ev_copy));
  const auto t0 = clk::now();
  // 1 MiB requests spread over the host threads: a whole-blob request is one queue entry,
  // and small requests pay per-request costs (measured on an MI355X host: 1 MiB direct reads move
  // 7.1 GB/s, 64 KiB 4.8 GB/s, 4 KiB 0.7 GB/s)
  const int rc = ftw_read(ctx->pool.get(), l->ftw, ids.data(), (int)ids.size(), dst.data(),
                          1u << 20);
  S->disk_us = us_since(t0);
  S->n_disk = (int32_t)ids.size();
  return rc;
}

static int decode_miss_path(ft_ctx* ctx, ft_layer* l, const uint16_t* x, int T, float* y,
                            ft_decode_stats* stats, hipStream_t st) {
  const ft_layer_desc& d = l->d;
  const int k = d.k, kk = l->kk, E = d.E;
  ft_decode_stats S{};
  if (!l->ftw && !d.host_blobs)
    return fail(FT_ESTATE, "ft_moe_decode: the layer has neither host_blobs nor a disk tier");
  // checked before anything runs, so a refused call leaves the pool untouched
  if (l->bp <= 0.0 || l->bh <= 0.0)
    return fail(FT_ESTATE, "ft_moe_decode: Bp/Bh unknown; call ft_measure_bandwidth or "
                           "ft_set_bandwidth first");
  auto t0 = clk::now();
  // routing in one launch, written straight into the mapped pinned staging: the layer's own
  // and, for a linked next layer, that layer's router on the same input (the prediction)
  ft_layer* nx = (l->next && l->pf_depth > 0) ? l->next : nullptr;
  auto dev_of = [&](const void* hp) { return l->pin_dev + ((const uint8_t*)hp - (const uint8_t*)l->pin); };
  RouteSmall ra{};
  ra.x = x;
  ra.x_host = (uint16_t*)dev_of(l->x_h);
  ra.T = T;
  ra.H = d.H;
  ra.n_routers = nx ? 2 : 1;
  ra.wr[0] = d.router_w;
  ra.b[0] = d.router_b;
  ra.E[0] = E;
  ra.k[0] = k;
  ra.logits[0] = l->logits;
  ra.idx[0] = l->idx;
  ra.w[0] = l->w;
  ra.idx_host[0] = (int32_t*)dev_of(l->idx_h);
  ra.w_host[0] = (float*)dev_of(l->w_h);
  if (nx) {
    ra.wr[1] = nx->d.router_w;
    ra.b[1] = nx->d.router_b;
    ra.E[1] = nx->d.E;
    ra.k[1] = nx->d.k;
    ra.logits[1] = l->pf_logits;
    ra.idx[1] = l->pf_idx;
    ra.w[1] = l->pf_w;
    ra.idx_host[1] = l->pf_idx_hd;
    ra.w_host[1] = l->pf_w_hd;
  }
  ra.counter = l->route_counter;
  ra.flag_host = (uint32_t*)dev_of(l->route_flag_h);
  if (++l->route_seq == 0) ++l->route_seq;   // 0 is the flag's initial value
  ra.seq = l->route_seq;
  // the previous call's device work (perhaps on another stream) still reads this layer's
  // pinned staging, which the host rewrites once this routing is back
  HIP_TRY(hipStreamWaitEvent(st, l->ev_done, 0));
  HIP_TRY((hipError_t)ftk_route_small(&ra, st));
  HIP_TRY(hipEventRecord(l->ev_route, st));
  HIP_TRY(wait_route(l->route_flag_h, ra.seq, l->ev_route));
  S.wait_us = us_since(t0);

  // classify: selected experts with their summed routing weight
  const int64_t now = l->lru.step;
  std::vector<double> wsum(E, 0.0);
  std::vector<char> sel(E, 0);
  for (int t = 0; t < T; ++t)
    for (int j = 0; j < k; ++j) {
      const int e = l->idx_h[t * k + j];
      if (e < 0 || e >= E) return fail(FT_ESTATE, "ft_moe_decode: routing produced a bad index");
      sel[e] = 1;
      wsum[e] += l->w_h[t * k + j];
    }
  std::vector<int> hits, misses;
  for (int e = 0; e < E; ++e) {
    if (!sel[e]) continue;
    ++S.n_selected;
    if (l->lru.e2s[e] >= 0) {
      hits.push_back(e);
      const int s = l->lru.e2s[e];
      l->lru.last_use[s] = now;
      if (l->lru.pref[s]) { ++S.n_prefetch_hits; l->lru.pref[s] = 0; }
    } else {
      misses.push_back(e);
    }
  }
  std::stable_sort(misses.begin(), misses.end(), [&](int a, int b) {
    return wsum[a] > wsum[b] || (wsum[a] == wsum[b] && a < b);
  });
  const int m = (int)misses.size();
  int q = 0;
  double qstar = 0.0;
  // the previous call's streamed copies have finished by now (its kernels waited for them
  // before the routing of this call ran): their copy time gives an observation of Bp
  if (l->pend_copy_bytes > 0 && hipEventQuery(l->ev_cp1) == hipSuccess) {
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, l->ev_cp0, l->ev_cp1) == hipSuccess && ms > 0.f)
      S.bp_obs = (double)l->pend_copy_bytes / (ms * 1e-3);
    l->pend_copy_bytes = 0;
    if (l->alpha > 0.0) l->bp = bandwidth_update(l->bp, S.bp_obs, l->alpha);
  }
  // the previous call's hit experts have run by now too: their GPU time per expert is an
  // observation of the GPU's load
  if (l->pend_gpu_items > 0 && hipEventQuery(l->ev_g1) == hipSuccess) {
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, l->ev_g0, l->ev_g1) == hipSuccess && ms > 0.f) {
      S.gpu_us_obs = ms * 1e3;
      const double obs = ms * 1e-3 / l->pend_gpu_items;
      l->t_gpu = (l->alpha > 0.0 && l->t_gpu > 0.0) ? bandwidth_update(l->t_gpu, obs, l->alpha)
                                                     : obs;
    }
    l->pend_gpu_items = 0;
  }
  int rc = qstar_split(m, l->bp, l->bh, &q, &qstar);
  if (rc) return rc;
  if (l->split_rule == FT_SPLIT_MAKESPAN) {
    rc = qstar_makespan(m, l->bp, l->bh, &q);
    if (rc) return rc;
  } else if (l->split_rule == FT_SPLIT_LOAD) {
    rc = qstar_load(m, (int)hits.size() + d.n_shared, l->bp, l->bh, (double)l->L.bytes,
                    l->t_gpu, &q);
    if (rc) return rc;
  }
  S.t_gpu = l->t_gpu;
  if (l->force_q >= 0) q = std::min(m, l->force_q);
  std::vector<int> streamed, host;
  for (int n = 0; n < m; ++n) {
    const int e = misses[n];
    if (n >= q) { host.push_back(e); continue; }
    int32_t old = -1;
    const int s = l->lru.take_slot(now, &old);
    if (s < 0) { host.push_back(e); continue; }
    if (old >= 0) { l->lru.e2s[old] = -1; ++S.n_evicted; }
    l->lru.s2e[s] = e;
    l->lru.e2s[e] = s;
    l->lru.last_use[s] = now;
    l->lru.pref[s] = 0;
    streamed.push_back(e);
  }
  l->lru.step++;
  S.n_hits = (int)hits.size();
  S.n_miss = m;
  S.q = q;
  S.qstar = qstar;
  S.n_streamed = (int)streamed.size();
  S.n_host = (int)host.size();
  S.bp = l->bp;
  S.bh = l->bh;
  S.step = (int)now;

  // work lists: list 0 = hits + shared experts, list 1 = streamed misses right after it;
  // each column carries its routing weight (for a down kernel that combines)
  WorkItem* L0 = l->items_h;
  int n0 = 0, n1 = 0;
  auto fill_cols = [&](WorkItem& it, int e) {
    int c = 0;
    for (int t = 0; t < T; ++t)
      for (int j = 0; j < k; ++j)
        if (l->idx_h[t * k + j] == e) {
          it.tok[c] = t;
          it.pair[c] = t * kk + j;
          it.wt[c] = l->w_h[t * k + j];
          ++c;
        }
    it.ntok = c;
  };
  for (int e : hits) { add_item(L0, &n0, e, l->lru.e2s[e]); fill_cols(L0[n0 - 1], e); }
  for (int s = 0; s < d.n_shared; ++s) {
    add_item(L0, &n0, -1 - s, -1 - s);
    WorkItem& it = L0[n0 - 1];
    it.ntok = T;
    for (int t = 0; t < T; ++t) { it.tok[t] = t; it.pair[t] = t * kk + k + s; it.wt[t] = 1.f; }
  }
  WorkItem* L1 = L0 + n0;
  for (int e : streamed) { add_item(L1, &n1, e, l->lru.e2s[e]); fill_cols(L1[n1 - 1], e); }
  l->n_items_h[0] = n0;
  l->n_items_h[1] = n1;
  std::copy(l->lru.e2s.begin(), l->lru.e2s.end(), l->e2s_h);
  std::copy(l->lru.s2e.begin(), l->lru.s2e.end(), l->s2e_h);

  // every miss's blob in host memory: from host_blobs, or through the host-memory tier
  if (l->ftw) {
    rc = host_tier_step(ctx, l, misses, &S);
    if (rc) return rc;
  }
  auto host_src = [&](int e) -> const uint8_t* {
    return l->ftw ? l->ram + (uint64_t)l->ram_lru.e2s[e] * d.blob_stride
                  : (const uint8_t*)d.host_blobs + (uint64_t)e * d.blob_stride;
  };
  // copies of streamed experts into their slots, on the copy stream (timed), after this
  // layer's previous kernels (which may have run on another stream) are done with the slots
  if (!streamed.empty()) {
    HIP_TRY(hipStreamWaitEvent(ctx->copy_stream, l->ev_done, 0));
    HIP_TRY(hipEventRecord(l->ev_cp0, ctx->copy_stream));
    l->pend_copy_bytes = (uint64_t)streamed.size() * l->L.bytes;
  }
  for (int e : streamed) {
    const int s = l->lru.e2s[e];
    HIP_TRY(hipMemcpyAsync((uint8_t*)d.pool + (uint64_t)s * d.blob_stride, host_src(e),
                           l->L.bytes, hipMemcpyHostToDevice, ctx->copy_stream));
  }
  if (!streamed.empty()) {
    HIP_TRY(hipEventRecord(l->ev_cp1, ctx->copy_stream));
    HIP_TRY(hipEventRecord(l->ev_copy, ctx->copy_stream));
  }
  // counts, tables and both work lists to the device in one copy (compute stream, before the
  // kernels): the pinned block and the device block have the same layout
  HIP_TRY(hipMemcpyAsync(l->n_items, l->n_items_h,
                         (size_t)((const uint8_t*)(l->items_h + n0 + n1) - (const uint8_t*)l->n_items_h),
                         hipMemcpyHostToDevice, st));
  // hits may sit in slots a prefetch from the previous layer is still filling
  if (l->pref_pending) {
    HIP_TRY(hipStreamWaitEvent(st, l->ev_pref, 0));
    l->pref_pending = false;
  }
  // every expert of the call a hit (or shared): list 0's down kernel also combines into y
  const bool fuse = n1 == 0 && host.empty();
  if (n0 > 0) {
    DecodeLaunch a = launch_args(l, x, T, 0, l->items, l->n_items, n0);
    if (fuse) {
      a.fuse_combine = 1;
      a.y = y;
    }
    const bool timed = l->split_rule == FT_SPLIT_LOAD;
    if (timed) HIP_TRY(hipEventRecord(l->ev_g0, st));
    HIP_TRY((hipError_t)ftk_decode_experts(&a, st, nullptr));
    if (timed) {
      HIP_TRY(hipEventRecord(l->ev_g1, st));
      l->pend_gpu_items = n0;
    }
  }
  if (n1 > 0) {
    HIP_TRY(hipStreamWaitEvent(st, l->ev_copy, 0));
    const DecodeLaunch a = launch_args(l, x, T, 0, l->items + n0, l->n_items + 1, n1);
    HIP_TRY((hipError_t)ftk_decode_experts(&a, st, nullptr));
  }
  // prefetch for the next layer, behind this layer's own copies, while its kernels run
  if (nx) {
    rc = prefetch_into(ctx, nx, l->pf_idx_h, l->pf_w_h, T, l->pf_depth, &S.n_prefetched);
    if (rc) return rc;
  }

  // host experts, concurrently with the GPU work enqueued above
  auto th = clk::now();
  double ffn_s = 0.0;   // wall time in the expert FFN itself
  std::vector<float> yt((size_t)T * d.H);
  std::vector<uint16_t> xt((size_t)T * d.H);
  for (int e : host) {
    // the tokens routed to e, packed
    int cols[FT_MAX_DECODE_TOKENS], js[FT_MAX_DECODE_TOKENS], c = 0;
    for (int t = 0; t < T; ++t)
      for (int j = 0; j < k; ++j)
        if (l->idx_h[t * k + j] == e) { cols[c] = t; js[c] = j; ++c; }
    for (int i = 0; i < c; ++i)
      std::memcpy(&xt[(size_t)i * d.H], l->x_h + (size_t)cols[i] * d.H, (size_t)d.H * 2);
    const auto tf = clk::now();
    rc = host_expert_ffn(ctx->pool.get(), l->L, host_src(e), xt.data(), c, yt.data());
    if (rc) return rc;
    ffn_s += us_since(tf) * 1e-6;
    for (int i = 0; i < c; ++i) {
      const int pair = cols[i] * kk + js[i];
      std::memcpy(l->P_h + (size_t)pair * d.H, &yt[(size_t)i * d.H], (size_t)d.H * 4);
      HIP_TRY(hipMemcpyAsync(l->P + (size_t)pair * d.H, l->P_h + (size_t)pair * d.H,
                             (size_t)d.H * 4, hipMemcpyHostToDevice, st));
    }
  }
  S.host_us = us_since(th);
  // an observation of Bh: the host experts' rate, plus the bandwidth the copies took from
  // the host while they ran alongside
  if (!host.empty() && ffn_s > 0.0) {
    S.bh_obs = (double)host.size() * l->L.bytes / ffn_s + (streamed.empty() ? 0.0 : l->bp);
    if (l->alpha > 0.0) l->bh = bandwidth_update(l->bh, S.bh_obs, l->alpha);
  }
  if (!fuse) HIP_TRY((hipError_t)ftk_combine(l->P, l->w, T, d.H, k, d.n_shared, y, st));
  HIP_TRY(hipEventRecord(l->ev_done, st));
  if (stats) *stats = S;
  return FT_OK;
}

extern "C" FT_API int ft_moe_decode(ft_ctx* ctx, ft_layer* layer, const uint16_t* x, int T,
                                    float* y, ft_decode_stats* stats, void* stream) try {
  int rc = check_call(ctx, layer, x, T, "ft_moe_decode");
  if (rc) return rc;
  if (!y) return fail(FT_EINVAL, "ft_moe_decode: y null");
  HIP_TRY(hipSetDevice(ctx->device));
  hipStream_t st = (hipStream_t)stream;
  if (layer->all_resident) {
    if (stats) {
      std::memset(stats, 0, sizeof(*stats));
      stats->bp = layer->bp;
      stats->bh = layer->bh;
      stats->step = (int)layer->lru.step;
    }
    layer->lru.step++;
    return decode_resident(layer, x, T, y, st);
  }
  return decode_miss_path(ctx, layer, x, T, y, stats, st);
} FT_CATCH("ft_moe_decode")

// ---- split rule and probes ----------------------------------------------------------------
extern "C" FT_API int ft_qstar_split(int m, double Bp, double Bh, int* q, double* qstar) try {
  return qstar_split(m, Bp, Bh, q, qstar);
} FT_CATCH("ft_qstar_split")

extern "C" FT_API int ft_set_bandwidth(ft_layer* layer, double Bp, double Bh) try {
  if (!layer || !(Bp > 0.0) || !(Bh > 0.0))
    return fail(FT_EINVAL, "ft_set_bandwidth: need a layer and Bp, Bh > 0");
  layer->bp = Bp;
  layer->bh = Bh;
  return FT_OK;
} FT_CATCH("ft_set_bandwidth")

extern "C" FT_API int ft_qstar_split_makespan(int m, double Bp, double Bh, int* q) try {
  return qstar_makespan(m, Bp, Bh, q);
} FT_CATCH("ft_qstar_split_makespan")

extern "C" FT_API int ft_qstar_split_load(int m, int g0, double Bp, double Bh, double blob,
                                          double t_gpu, int* q) try {
  return qstar_load(m, g0, Bp, Bh, blob, t_gpu, q);
} FT_CATCH("ft_qstar_split_load")

extern "C" FT_API int ft_set_miss_policy(ft_layer* layer, int rule, double alpha) try {
  if (!layer) return fail(FT_EINVAL, "ft_set_miss_policy: null layer");
  if (rule != FT_SPLIT_ROUND && rule != FT_SPLIT_MAKESPAN && rule != FT_SPLIT_LOAD)
    return fail(FT_EINVAL, "ft_set_miss_policy: unknown split rule");
  if (!(alpha >= 0.0 && alpha <= 1.0))
    return fail(FT_EINVAL, "ft_set_miss_policy: alpha must be in [0, 1]");
  layer->split_rule = rule;
  layer->alpha = alpha;
  return FT_OK;
} FT_CATCH("ft_set_miss_policy")

extern "C" FT_API int ft_set_prefetch(ft_layer* layer, ft_layer* next, int depth) try {
  if (!layer) return fail(FT_EINVAL, "ft_set_prefetch: null layer");
  if (depth < 0) return fail(FT_EINVAL, "ft_set_prefetch: depth must be >= 0");
  auto unlink = [&]() {
    if (layer->next && layer->next->prev == layer) layer->next->prev = nullptr;
    layer->next = nullptr;
    layer->pf_depth = 0;
  };
  if (!next || depth == 0) {
    unlink();
    return FT_OK;
  }
  if (next == layer) return fail(FT_EINVAL, "ft_set_prefetch: a layer cannot prefetch for itself");
  if (next->ctx != layer->ctx) return fail(FT_EINVAL, "ft_set_prefetch: layers of different contexts");
  if (layer->all_resident || next->all_resident)
    return fail(FT_EINVAL, "ft_set_prefetch: both layers need a partial pool (miss path)");
  if (next->d.H != layer->d.H) return fail(FT_EINVAL, "ft_set_prefetch: hidden sizes differ");
  if (depth > next->d.n_slots) return fail(FT_EINVAL, "ft_set_prefetch: depth above next's slots");
  if (next->prev && next->prev != layer)
    return fail(FT_EINVAL, "ft_set_prefetch: next is already the target of another layer");
  if (layer->ftw || next->ftw)
    return fail(FT_EINVAL, "ft_set_prefetch: a layer with a disk tier cannot be linked");
  if (!next->d.host_blobs) return fail(FT_EINVAL, "ft_set_prefetch: next has no host_blobs");
  HIP_TRY(hipSetDevice(layer->ctx->device));
  if (!layer->pf_dev) {
    const size_t nl = (size_t)FT_MAX_DECODE_TOKENS * 1024, nk = (size_t)FT_MAX_DECODE_TOKENS * FT_MAX_TOPK;
    if (hipMalloc(&layer->pf_dev, nl * 4 + 2 * nk * 4) != hipSuccess)
      return fail(FT_ENOMEM, "ft_set_prefetch: device allocation failed");
    layer->pf_logits = (float*)layer->pf_dev;
    layer->pf_idx = (int32_t*)(layer->pf_logits + nl);
    layer->pf_w = (float*)(layer->pf_idx + nk);
    if (hipHostMalloc(&layer->pf_pin, 2 * nk * 4, hipHostMallocMapped) != hipSuccess)
      return fail(FT_ENOMEM, "ft_set_prefetch: pinned allocation failed");
    layer->pf_idx_h = (int32_t*)layer->pf_pin;
    layer->pf_w_h = (float*)(layer->pf_idx_h + nk);
    void* dp = nullptr;
    HIP_TRY(hipHostGetDevicePointer(&dp, layer->pf_pin, 0));
    layer->pf_idx_hd = (int32_t*)dp;
    layer->pf_w_hd = (float*)(layer->pf_idx_hd + nk);
  }
  unlink();
  layer->next = next;
  next->prev = layer;
  layer->pf_depth = depth;
  return FT_OK;
} FT_CATCH("ft_set_prefetch")

extern "C" FT_API int ft_residual_bf16(ft_ctx* ctx, const uint16_t* x, const float* y, float scale,
                                       int64_t n, uint16_t* out, void* stream) try {
  if (!ctx || n < 0) return fail(FT_EINVAL, "ft_residual_bf16: null context or n < 0");
  if (n == 0) return FT_OK;
  if (!x || !y || !out) return fail(FT_EINVAL, "ft_residual_bf16: null array");
  HIP_TRY(hipSetDevice(ctx->device));
  HIP_TRY((hipError_t)ftk_residual(x, y, scale, n, out, (hipStream_t)stream));
  return FT_OK;
} FT_CATCH("ft_residual_bf16")

extern "C" FT_API int ft_layer_set_disk_tier(ft_layer* layer, ft_ftw* f, void* ram, int n_ram) try {
  if (!layer) return fail(FT_EINVAL, "ft_layer_set_disk_tier: null layer");
  if (layer->all_resident) return fail(FT_EINVAL, "ft_layer_set_disk_tier: the layer is resident");
  if (layer->next || layer->prev)
    return fail(FT_EINVAL, "ft_layer_set_disk_tier: the layer is linked by ft_set_prefetch");
  const ft_layer_desc& d = layer->d;
  if (!f) {
    layer->ftw = nullptr;
    layer->ram = nullptr;
    layer->n_ram = 0;
    return FT_OK;
  }
  int fmt, H, I, E, ns;
  ftw_dims(f, &fmt, &H, &I, &E, &ns);
  if (fmt != d.format || H != d.H || I != d.I || E != d.E || ns != d.n_shared)
    return fail(FT_EINVAL, "ft_layer_set_disk_tier: the file's dimensions differ from the layer's");
  if (n_ram < d.max_tokens * d.k || n_ram > d.E)
    return fail(FT_EINVAL, "ft_layer_set_disk_tier: n_ram must be in [max_tokens * k, E]");
  if (!ram || (uintptr_t)ram % kAlign)
    return fail(FT_EINVAL, "ft_layer_set_disk_tier: ram must be 4096-aligned");
  HIP_TRY(hipSetDevice(layer->ctx->device));
  hipPointerAttribute_t pa{};
  if (hipPointerGetAttributes(&pa, ram) != hipSuccess || pa.type != hipMemoryTypeHost) {
    (void)hipGetLastError();
    return fail(FT_EINVAL, "ft_layer_set_disk_tier: ram is not pinned host memory");
  }
  HIP_TRY(hipEventSynchronize(layer->ev_copy));   // copies from the previous source are done
  layer->ftw = f;
  layer->ram = (uint8_t*)ram;
  layer->n_ram = n_ram;
  layer->ram_lru.init(d.E, n_ram, false);
  return FT_OK;
} FT_CATCH("ft_layer_set_disk_tier")

extern "C" FT_API int ft_debug_host_tier(const ft_layer* layer, int32_t* e2r, int32_t* r2e) try {
  if (!layer || !e2r || !r2e) return fail(FT_EINVAL, "ft_debug_host_tier: null argument");
  if (!layer->ftw) return fail(FT_ESTATE, "ft_debug_host_tier: the layer has no disk tier");
  std::copy(layer->ram_lru.e2s.begin(), layer->ram_lru.e2s.end(), e2r);
  std::copy(layer->ram_lru.s2e.begin(), layer->ram_lru.s2e.end(), r2e);
  return FT_OK;
} FT_CATCH("ft_debug_host_tier")

extern "C" FT_API int ft_force_q(ft_layer* layer, int q) try {
  if (!layer) return fail(FT_EINVAL, "ft_force_q: null layer");
  layer->force_q = q < 0 ? -1 : q;
  return FT_OK;
} FT_CATCH("ft_force_q")

static double median(std::vector<double> v) {
  std::sort(v.begin(), v.end());
  return v.empty() ? 0.0 : v[v.size() / 2];
}

extern "C" FT_API int ft_measure_bandwidth(ft_ctx* ctx, ft_layer* layer, double* Bp, double* Bh) try {
  if (!ctx || !layer) return fail(FT_EINVAL, "ft_measure_bandwidth: null argument");
  const ft_layer_desc& d = layer->d;
  HIP_TRY(hipSetDevice(ctx->device));
  // probe sources: up to 8 distinct host blobs (more bytes than a host's last-level cache
  // holds, so the host FFN reads DRAM as it does in decode), from host_blobs or read into the
  // first slots of a disk tier that no decode call has used yet
  constexpr int kProbeBlobs = 8;
  const uint8_t* srcs[kProbeBlobs];
  int nsrc = 0;
  if (d.host_blobs) {
    nsrc = std::min(kProbeBlobs, d.E);
    for (int i = 0; i < nsrc; ++i)
      srcs[i] = (const uint8_t*)d.host_blobs + (uint64_t)i * d.blob_stride;
  } else if (layer->ftw) {
    for (int32_t e : layer->ram_lru.s2e)
      if (e >= 0) return fail(FT_ESTATE, "ft_measure_bandwidth: the disk tier is already in use");
    nsrc = std::min(kProbeBlobs, std::min(layer->n_ram, d.E));
    int32_t ids[kProbeBlobs];
    uint8_t* dst[kProbeBlobs];
    for (int i = 0; i < nsrc; ++i) {
      ids[i] = i;
      dst[i] = layer->ram + (uint64_t)i * d.blob_stride;
    }
    const int rc = ftw_read(ctx->pool.get(), layer->ftw, ids, nsrc, dst, 1u << 20);
    if (rc) return rc;
    for (int i = 0; i < nsrc; ++i) srcs[i] = dst[i];
  } else {
    return fail(FT_ESTATE, "ft_measure_bandwidth: the layer has neither host_blobs nor a disk tier");
  }
  const uint64_t bytes = layer->L.bytes;
  void* tmp = nullptr;
  if (hipMalloc(&tmp, bytes) != hipSuccess)
    return fail(FT_ENOMEM, "ft_measure_bandwidth: probe buffer allocation failed");
  hipEvent_t a = nullptr, b = nullptr;
  std::vector<double> bps;
  const int reps = env_int("FT_PROBE_REPS", 7);
  hipError_t he = hipEventCreate(&a);
  if (he == hipSuccess) he = hipEventCreate(&b);
  for (int r = 0; r < reps + 1 && he == hipSuccess; ++r) {
    const uint8_t* src = srcs[r % nsrc];
    he = hipEventRecord(a, ctx->copy_stream);
    if (he == hipSuccess) he = hipMemcpyAsync(tmp, src, bytes, hipMemcpyHostToDevice, ctx->copy_stream);
    if (he == hipSuccess) he = hipEventRecord(b, ctx->copy_stream);
    if (he == hipSuccess) he = hipEventSynchronize(b);
    float ms = 0.f;
    if (he == hipSuccess) he = hipEventElapsedTime(&ms, a, b);
    if (he == hipSuccess && r > 0 && ms > 0.f) bps.push_back((double)bytes / (ms * 1e-3));
  }
  if (a) (void)hipEventDestroy(a);
  if (b) (void)hipEventDestroy(b);
  (void)hipFree(tmp);
  if (he != hipSuccess)
    return fail(FT_EHIP, std::string("ft_measure_bandwidth: ") + hipGetErrorString(he));
  std::vector<double> bhs;
  std::vector<uint16_t> x(d.H, 0x3f80);  // ones
  std::vector<float> y(d.H);
  for (int r = 0; r < reps + 1; ++r) {
    const uint8_t* src = srcs[(r + 1) % nsrc];
    auto t0 = clk::now();
    int rc = host_expert_ffn(ctx->pool.get(), layer->L, src, x.data(), 1, y.data());
    if (rc) return rc;
    const double s = us_since(t0) * 1e-6;
    if (r > 0 && s > 0) bhs.push_back((double)bytes / s);
  }
  layer->bp = median(bps);
  layer->bh = median(bhs);
  if (Bp) *Bp = layer->bp;
  if (Bh) *Bh = layer->bh;
  return FT_OK;
} FT_CATCH("ft_measure_bandwidth")

extern "C" FT_API int ft_probe_hbm_read(ft_ctx* ctx, const void* buf, uint64_t bytes, int reps,
                                        double* GBps) try {
  if (!ctx || !buf || !GBps || reps < 1 || bytes < (1u << 20) || bytes % 16)
    return fail(FT_EINVAL, "ft_probe_hbm_read: bad argument");
  HIP_TRY(hipSetDevice(ctx->device));
  hipDeviceProp_t prop;
  HIP_TRY(hipGetDeviceProperties(&prop, ctx->device));
  const int cus = prop.multiProcessorCount;
  uint32_t* sink = nullptr;
  if (hipMalloc(&sink, (size_t)32 * cus * 4) != hipSuccess)
    return fail(FT_ENOMEM, "ft_probe_hbm_read: sink allocation failed");
  hipEvent_t a = nullptr, b = nullptr;
  hipError_t e = hipEventCreate(&a);
  if (e == hipSuccess) e = hipEventCreate(&b);
  double best = 0.0;
  // form 0: register loads, 32 workgroups per CU; form 1: LDS copies, one workgroup per CU
  for (int form = 0; form < 2 && e == hipSuccess; ++form) {
    const int grid = form ? cus : 32 * cus;
    e = (hipError_t)ftk_read_probe(buf, bytes, sink, grid, form, ctx->copy_stream);
    if (e == hipSuccess) e = hipEventRecord(a, ctx->copy_stream);
    for (int r = 0; r < reps && e == hipSuccess; ++r)
      e = (hipError_t)ftk_read_probe(buf, bytes, sink, grid, form, ctx->copy_stream);
    if (e == hipSuccess) e = hipEventRecord(b, ctx->copy_stream);
    if (e == hipSuccess) e = hipEventSynchronize(b);
    float ms = 0.f;
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, a, b);
    if (e == hipSuccess && ms > 0.f)
      best = std::max(best, (double)bytes * reps / (ms * 1e-3) / 1e9);
  }
  if (a) hipEventDestroy(a);
  if (b) hipEventDestroy(b);
  hipFree(sink);
  if (e != hipSuccess) return fail(FT_EHIP, std::string("ft_probe_hbm_read: ") + hipGetErrorString(e));
  *GBps = best;
  return FT_OK;
} FT_CATCH("ft_probe_hbm_read")

extern "C" FT_API int ft_debug_throw(int kind) try {
  if (kind == 1) throw std::bad_alloc();
  if (kind == 2) throw std::runtime_error("planted exception");
  if (kind == 3)
    throw std::system_error(std::make_error_code(std::errc::resource_unavailable_try_again));
  if (kind != 0) return fail(FT_EINVAL, "ft_debug_throw: kind must be 0..3");
  return FT_OK;
} FT_CATCH("ft_debug_throw")

extern "C" FT_API int ft_debug_pool_stress(int threads, int jobs, int pause_us) try {
  if (threads < 1 || threads > 256 || jobs < 0 || pause_us < 0)
    return fail(FT_EINVAL, "ft_debug_pool_stress: bad argument");
  ThreadPool pool(threads);
  std::vector<std::atomic<int>> hits((size_t)threads);
  for (int j = 0; j < jobs; ++j) {
    for (auto& h : hits) h.store(0);
    pool.run([&](int i, int n) {
      if (n == threads && i >= 0 && i < n) hits[(size_t)i].fetch_add(1);
    });
    for (auto& h : hits)
      if (h.load() != 1) return fail(FT_ESTATE, "ft_debug_pool_stress: a worker missed or repeated a job");
    if (pause_us) std::this_thread::sleep_for(std::chrono::microseconds(pause_us));
  }
  return FT_OK;
} FT_CATCH("ft_debug_pool_stress")

// ---- kernel timing ------------------------------------------------------------------------
extern "C" FT_API int ft_profile_begin(ft_layer* layer, int n) try {
  if (!layer || n < 0 || n > 1000000) return fail(FT_EINVAL, "ft_profile_begin: bad argument");
  HIP_TRY(hipSetDevice(layer->ctx->device));
  const size_t need = (size_t)n * 4;
  while (layer->prof.size() < need) {
    hipEvent_t e;
    HIP_TRY(hipEventCreate(&e));
    layer->prof.push_back(e);
  }
  layer->prof_n = n;
  layer->prof_i = 0;
  return FT_OK;
} FT_CATCH("ft_profile_begin")

extern "C" FT_API int ft_profile_end(ft_layer* layer, double* gateup_us, double* down_us,
                                     int* n_recorded) try {
  if (!layer) return fail(FT_EINVAL, "ft_profile_end: null layer");
  HIP_TRY(hipSetDevice(layer->ctx->device));
  double a = 0.0, b = 0.0;
  const int n = layer->prof_i;
  for (int i = 0; i < n; ++i) {
    hipEvent_t* e = &layer->prof[(size_t)i * 4];
    HIP_TRY(hipEventSynchronize(e[3]));
    float m0 = 0.f, m1 = 0.f;
    HIP_TRY(hipEventElapsedTime(&m0, e[0], e[1]));
    HIP_TRY(hipEventElapsedTime(&m1, e[2], e[3]));
    a += m0 * 1e3;
    b += m1 * 1e3;
  }
  if (gateup_us) *gateup_us = n ? a / n : 0.0;
  if (down_us) *down_us = n ? b / n : 0.0;
  if (n_recorded) *n_recorded = n;
  layer->prof_n = layer->prof_i = 0;
  return FT_OK;
} FT_CATCH("ft_profile_end")

// ---- test hooks ---------------------------------------------------------------------------
extern "C" FT_API int ft_debug_dequant(const ft_layer* layer, int slot, int matrix, float* out,
                                       void* stream) try {
  if (!layer || !out || matrix < 0 || matrix > 2)
    return fail(FT_EINVAL, "ft_debug_dequant: bad argument");
  const ft_layer_desc& d = layer->d;
  const uint8_t* blob;
  if (slot >= 0) {
    if (slot >= d.n_slots) return fail(FT_EINVAL, "ft_debug_dequant: slot out of range");
    blob = (const uint8_t*)d.pool + (uint64_t)slot * d.blob_stride;
  } else {
    const int s = -1 - slot;
    if (s >= d.n_shared) return fail(FT_EINVAL, "ft_debug_dequant: no such shared expert");
    blob = (const uint8_t*)d.shared_blobs + (uint64_t)s * d.blob_stride;
  }
  HIP_TRY(hipSetDevice(layer->ctx->device));
  float ts = 1.0f;
  if (d.format == FT_NVFP4) {
    BlobHeader hdr;
    HIP_TRY(hipMemcpy(&hdr, blob, sizeof(hdr), hipMemcpyDeviceToHost));
    ts = hdr.tensor_scale[matrix];
  }
  HIP_TRY((hipError_t)ftk_dequant(blob, &layer->L, matrix, ts, out, (hipStream_t)stream));
  return FT_OK;
} FT_CATCH("ft_debug_dequant")

extern "C" FT_API int ft_debug_tables(const ft_layer* layer, int32_t* e2s, int32_t* s2e) try {
  if (!layer || !e2s || !s2e) return fail(FT_EINVAL, "ft_debug_tables: null argument");
  HIP_TRY(hipSetDevice(layer->ctx->device));
  HIP_TRY(hipDeviceSynchronize());
  HIP_TRY(hipMemcpy(e2s, layer->e2s_dev, (size_t)layer->d.E * 4, hipMemcpyDeviceToHost));
  HIP_TRY(hipMemcpy(s2e, layer->s2e_dev, (size_t)layer->d.n_slots * 4, hipMemcpyDeviceToHost));
  return FT_OK;
} FT_CATCH("ft_debug_tables")

extern "C" FT_API int ft_host_expert_ffn(ft_ctx* ctx, int format, int H, int I, const void* blob,
                                         const uint16_t* x, int T, float* y) try {
  if (!dims_ok(format, H, I) || !blob || !x || !y || T < 1)
    return fail(FT_EINVAL, "ft_host_expert_ffn: bad argument");
  return host_expert_ffn(ctx ? ctx->pool.get() : nullptr, blob_layout(format, H, I),
                         (const uint8_t*)blob, x, T, y);
} FT_CATCH("ft_host_expert_ffn")

// ---- prefill ------------------------------------------------------------------------------
// Workspace layout of one prefill call (every region 256-byte aligned); returns the bytes.
static size_t prefill_carve(const ft_layer* l, int T, int mode, uint8_t* base,
                            PrefillLaunch* a) {
  const ft_layer_desc& d = l->d;
  const size_t nblk = (size_t)(T + kPermBlock - 1) / kPermBlock;
  const size_t pairs = (size_t)T * d.k;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    uint8_t* r = base ? base + off : nullptr;
    off += align_up(bytes, 256);
    return r;
  };
  uint8_t* logits = take((size_t)router_splits(T, d.E, d.H) * T * d.E * 4);
  uint8_t* idx = take(pairs * 4);
  uint8_t* w = take(pairs * 4);
  uint8_t* masks = take(nblk * d.E * 8 * 4);
  uint8_t* bcnt = take(nblk * d.E * 4);
  uint8_t* counts = take((size_t)d.E * 4);
  uint8_t* offsets = take((size_t)(d.E + 1) * 4);
  uint8_t* bas = take(nblk * d.E * 4);
  uint8_t* tb_off = take((size_t)(d.E + 1) * 4);
  uint8_t* pos = take(pairs * 4);
  uint8_t* perm_tok = take(pairs * 4);
  uint8_t* perm_w = take(pairs * 4);
  const bool mx = mode == FT_PREFILL_MXFP4;
  uint8_t* xq = mx ? take((size_t)T * d.H / 2) : nullptr;
  uint8_t* xqs = mx ? take((size_t)T * d.H / 32) : nullptr;
  // tiled operands: permuted rows, each expert's padded to a multiple of pad (at most
  // T*k + (pad - 1) E rows, rounded up to pad)
  const size_t pad = mx ? 16 : 32;
  const size_t prows = (pairs + (pad - 1) * (size_t)d.E + pad - 1) / pad * pad;
  uint8_t* poff = take((size_t)(d.E + 1) * 4);
  uint8_t* xtb = mx ? nullptr : take(prows * d.H * 2);
  uint8_t* htb = mx ? nullptr : take(prows * d.I * 2);
  uint8_t* xt = mx ? take(prows * d.H / 2) : nullptr;
  uint8_t* xts = mx ? take(prows * d.H / 32) : nullptr;
  uint8_t* ht = mx ? take(prows * d.I / 2) : nullptr;
  uint8_t* hts = mx ? take(prows * d.I / 32) : nullptr;
  uint8_t* yperm = mx ? take(pairs * d.H * 3) : nullptr;   // S1: 24-bit floats
  // the expert of each token block (at most pairs / rows + E blocks of `rows` rows)
  const size_t brows = mx ? kS1Rows : kGemmM;
  uint8_t* blk_e = take(((pairs + brows - 1) / brows + d.E) * 4);
  uint8_t* tile_e = take(prows / pad * 4);   // expert of each padded row group
  if (a) {
    a->logits = (float*)logits;
    a->idx = (int32_t*)idx;
    a->w = (float*)w;
    a->masks = (uint32_t*)masks;
    a->bcnt = (int32_t*)bcnt;
    a->counts = (int32_t*)counts;
    a->offsets = (int32_t*)offsets;
    a->base = (int32_t*)bas;
    a->tb_off = (int32_t*)tb_off;
    a->pos = (int32_t*)pos;
    a->perm_tok = (int32_t*)perm_tok;
    a->perm_w = (float*)perm_w;
    a->xtb = (uint16_t*)xtb;
    a->htb = (uint16_t*)htb;
    a->pad_rows = (int)pad;
    a->xq = xq;
    a->xqs = xqs;
    a->poff = (int32_t*)poff;
    a->xt = xt;
    a->xts = xts;
    a->ht = ht;
    a->hts = hts;
    a->Yperm = (float*)yperm;
    a->blk_e = (int32_t*)blk_e;
    a->tile_e = (int32_t*)tile_e;
  }
  return off;
}

static int prefill_check(const ft_layer* layer, int T, int mode, const char* who) {
  if (!layer) return fail(FT_EINVAL, std::string(who) + ": null layer");
  if (T < 1 || (int64_t)T * layer->d.k > (int64_t)1 << 28)
    return fail(FT_EINVAL, std::string(who) + ": T out of range");
  if (mode != FT_PREFILL_EXACT && mode != FT_PREFILL_MXFP4)
    return fail(FT_EINVAL, std::string(who) + ": unknown mode");
  if (!layer->all_resident)
    return fail(FT_ESTATE, std::string(who) + ": prefill needs an all-resident layer");
  if (mode == FT_PREFILL_MXFP4 && !layer->mx_pool)
    return fail(FT_ESTATE, std::string(who) + ": FT_PREFILL_MXFP4 on an NVFP4 layer needs "
                                              "FT_LAYER_PREFILL_MXFP4 at ft_layer_create");
  if (layer->d.n_shared > 0)
    return fail(FT_EUNSUPPORTED, std::string(who) + ": prefill of layers with shared experts "
                                                    "is not built");
  return FT_OK;
}

extern "C" FT_API int ft_moe_prefill_workspace_size(const ft_layer* layer, int T, int mode,
                                                    size_t* bytes) try {
  int rc = prefill_check(layer, T, mode, "ft_moe_prefill_workspace_size");
  if (rc) return rc;
  if (!bytes) return fail(FT_EINVAL, "ft_moe_prefill_workspace_size: bytes is null");
  *bytes = prefill_carve(layer, T, mode, nullptr, nullptr);
  return FT_OK;
} FT_CATCH("ft_moe_prefill_workspace_size")

// One prefill call's launches over the workspace ws (checked by the caller).
static int prefill_launch(ft_ctx* ctx, ft_layer* layer, const uint16_t* x, int T, float* y,
                          int mode, void* ws, void* stream) {
  const ft_layer_desc& d = layer->d;
  HIP_TRY(hipSetDevice(ctx->device));
  PrefillLaunch a{};
  prefill_carve(layer, T, mode, (uint8_t*)ws, &a);
  a.x = x;
  a.T = T; a.H = d.H; a.I = d.I; a.E = d.E; a.k = d.k;
  a.wr_planes = layer->wr_planes;
  a.splits = router_splits(T, d.E, d.H);
  a.router_b = d.router_b;
  a.pool = (const uint8_t*)d.pool;
  a.stride = d.blob_stride;
  a.L = layer->L;
  a.mode = mode;
  a.mrows = mode == FT_PREFILL_MXFP4 ? kS1Rows : kGemmM;
  a.mxpool = layer->mx_pool;
  a.mxstride = layer->mx_stride;
  a.ML = blob_layout(FT_MXFP4, d.H, d.I);
  a.y = y;
  HIP_TRY((hipError_t)ftk_prefill(&a, (hipStream_t)stream, prof_events(layer)));
  return FT_OK;
}

extern "C" FT_API int ft_moe_prefill(ft_ctx* ctx, ft_layer* layer, const uint16_t* x, int T,
                                     float* y, int mode, void* ws, size_t ws_bytes,
                                     void* stream) try {
  int rc = prefill_check(layer, T, mode, "ft_moe_prefill");
  if (rc) return rc;
  if (!ctx || !x || !y || !ws) return fail(FT_EINVAL, "ft_moe_prefill: null argument");
  if (layer->ctx != ctx) return fail(FT_EINVAL, "ft_moe_prefill: layer of another context");
  if ((uintptr_t)ws % 256) return fail(FT_EINVAL, "ft_moe_prefill: ws must be 256-byte aligned");
  const size_t need = prefill_carve(layer, T, mode, nullptr, nullptr);
  if (ws_bytes < need) return fail(FT_EINVAL, "ft_moe_prefill: workspace too small");
  return prefill_launch(ctx, layer, x, T, y, mode, ws, stream);
} FT_CATCH("ft_moe_prefill")

// The workspace is the static scratch looked up at ft_ctx_create: nothing is allocated here.
extern "C" FT_API int ft_moe_prefill_noalloc(ft_ctx* ctx, ft_layer* layer, const uint16_t* x,
                                             int T, float* y, int mode, void* stream) try {
  int rc = prefill_check(layer, T, mode, "ft_moe_prefill_noalloc");
  if (rc) return rc;
  if (!ctx || !x || !y) return fail(FT_EINVAL, "ft_moe_prefill_noalloc: null argument");
  if (layer->ctx != ctx)
    return fail(FT_EINVAL, "ft_moe_prefill_noalloc: layer of another context");
  if (!ctx->scratch) return fail(FT_ESTATE, "ft_moe_prefill_noalloc: no static scratch");
  const size_t need = prefill_carve(layer, T, mode, nullptr, nullptr);
  if (need > ctx->scratch_bytes)
    return fail(FT_EINVAL, "ft_moe_prefill_noalloc: T = " + std::to_string(T) + " needs " +
                               std::to_string(need) + " workspace bytes, more than the " +
                               std::to_string(ctx->scratch_bytes) + " of the static scratch");
  return prefill_launch(ctx, layer, x, T, y, mode, ctx->scratch, stream);
} FT_CATCH("ft_moe_prefill_noalloc")

extern "C" FT_API int ft_debug_prefill_perm(const ft_layer* layer, const void* ws, int T,
                                            int32_t* counts, int32_t* offsets, int32_t* pos,
                                            void* stream) try {
  if (!layer || !ws || !counts || !offsets || !pos || T < 1)
    return fail(FT_EINVAL, "ft_debug_prefill_perm: bad argument");
  PrefillLaunch a{};
  prefill_carve(layer, T, FT_PREFILL_EXACT, (uint8_t*)ws, &a);  // same offsets in both modes
  const ft_layer_desc& d = layer->d;
  hipStream_t st = (hipStream_t)stream;
  HIP_TRY(hipSetDevice(layer->ctx->device));
  HIP_TRY(hipMemcpyAsync(counts, a.counts, (size_t)d.E * 4, hipMemcpyDeviceToDevice, st));
  HIP_TRY(hipMemcpyAsync(offsets, a.offsets, (size_t)(d.E + 1) * 4, hipMemcpyDeviceToDevice, st));
  HIP_TRY(hipMemcpyAsync(pos, a.pos, (size_t)T * d.k * 4, hipMemcpyDeviceToDevice, st));
  return FT_OK;
} FT_CATCH("ft_debug_prefill_perm")

extern "C" FT_API int ft_debug_prefill_route(const ft_layer* layer, const void* ws, int T,
                                             int32_t* idx, float* w, void* stream) try {
  if (!layer || !ws || !idx || !w || T < 1)
    return fail(FT_EINVAL, "ft_debug_prefill_route: bad argument");
  PrefillLaunch a{};
  prefill_carve(layer, T, FT_PREFILL_EXACT, (uint8_t*)ws, &a);  // same offsets in both modes
  hipStream_t st = (hipStream_t)stream;
  const size_t n = (size_t)T * layer->d.k * 4;
  HIP_TRY(hipSetDevice(layer->ctx->device));
  HIP_TRY(hipMemcpyAsync(idx, a.idx, n, hipMemcpyDeviceToDevice, st));
  HIP_TRY(hipMemcpyAsync(w, a.w, n, hipMemcpyDeviceToDevice, st));
  return FT_OK;
} FT_CATCH("ft_debug_prefill_route")

extern "C" FT_API int ft_debug_prefill_quant(const ft_layer* layer, const void* ws, int T,
                                             int which, uint8_t* codes, uint8_t* scales,
                                             void* stream) try {
  if (!layer || !ws || !codes || !scales || T < 1 || (which != 0 && which != 1))
    return fail(FT_EINVAL, "ft_debug_prefill_quant: bad argument");
  PrefillLaunch a{};
  prefill_carve(layer, T, FT_PREFILL_MXFP4, (uint8_t*)ws, &a);
  const ft_layer_desc& d = layer->d;
  hipStream_t st = (hipStream_t)stream;
  const size_t rows = which == 0 ? (size_t)T : (size_t)T * d.k;
  const size_t K = which == 0 ? (size_t)d.H : (size_t)d.I;
  HIP_TRY(hipSetDevice(layer->ctx->device));
  if (which == 0) {
    HIP_TRY(hipMemcpyAsync(codes, a.xq, rows * K / 2, hipMemcpyDeviceToDevice, st));
    HIP_TRY(hipMemcpyAsync(scales, a.xqs, rows * K / 32, hipMemcpyDeviceToDevice, st));
  } else {
    a.T = T; a.H = d.H; a.I = d.I; a.E = d.E; a.k = d.k;
    HIP_TRY((hipError_t)ftk_untile_h(&a, codes, scales, st));
  }
  return FT_OK;
} FT_CATCH("ft_debug_prefill_quant")

extern "C" FT_API int ft_debug_prefill_weights(const ft_layer* layer, int e, void* out,
                                               void* stream) try {
  if (!layer || !out || e < 0 || e >= layer->d.E)
    return fail(FT_EINVAL, "ft_debug_prefill_weights: bad argument");
  if (!layer->mx_pool) return fail(FT_ESTATE, "ft_debug_prefill_weights: no MXFP4 weights");
  HIP_TRY(hipSetDevice(layer->ctx->device));
  HIP_TRY(hipMemcpyAsync(out, layer->mx_pool + (uint64_t)e * layer->mx_stride,
                         blob_layout(FT_MXFP4, layer->d.H, layer->d.I).bytes,
                         hipMemcpyDeviceToDevice, (hipStream_t)stream));
  return FT_OK;
} FT_CATCH("ft_debug_prefill_weights")
