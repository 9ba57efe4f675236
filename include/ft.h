/*
 * ft.h — C ABI of libft, an MI355X (gfx950) sparse MoE expert layer with block-scaled FP4
 * expert weights.
 *
 * What the layer computes (FreeToken pages: mubeitech explainer, MoE paragraph — a gate
 * picks a few experts per token; smzdm explainer a825qpgl, section 二 — 6 of 256 experts
 * active, three classes of selected expert, merged by routing weight):
 *
 *   logits_t = x_t . W_r^T + b                       (fp32)
 *   S_t      = the k largest logits (ties: lower index), in rank order
 *   w_tj     = softmax over the k kept logits         (== full softmax renormalised)
 *   y_e(x)   = W_d,e . bf16(silu(W_g,e x) * (W_u,e x))   (SwiGLU; h rounded to bf16)
 *   y_t      = sum_j w_tj y_{S_tj}(x_t) + sum_s y_shared_s(x_t)
 *
 * Experts whose weights are not in the GPU slot pool (misses) are split by the rule
 * q* = m * Bp / Bh (same page, section 二): q of the m misses are copied from pinned host
 * memory into pool slots with hipMemcpyAsync and computed on the GPU, the other m - q are
 * computed on host cores at the same time.  The pool is an LRU over expert slots (smzdm
 * explainer aomxznrn, "FreeToken干的事", item 2).
 *
 * Conventions
 *   - Every function returns FT_OK (0) or a negative FT_E* code; ft_last_error() then gives
 *     a message (thread-local).  No function aborts or throws across the ABI.
 *   - "device" pointers are HIP device memory on the context's device; "host" pointers are
 *     ordinary host memory unless "pinned" is said (allocated with hipHostMalloc or
 *     torch's pin_memory).  The caller owns every buffer it passes; the library borrows
 *     layer buffers for the layer's lifetime and owns only its internal state.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Device work is enqueued on it
 *     asynchronously unless stated otherwise; outputs are valid after the stream syncs.
 *   - bf16 values are passed as uint16_t bit patterns.
 *   - Calls on one layer must be serialised by the caller.  An all-resident layer's calls
 *     also share its device scratch: issue them on one stream, or synchronise between calls
 *     made on different streams.  (A call that takes the miss path waits for the previous
 *     call's device work itself.)
 */
#ifndef FT_H
#define FT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FT_API __attribute__((visibility("default")))

enum {
  FT_OK = 0,
  FT_EINVAL = -1,        /* bad argument (null pointer, size out of range, bad layout) */
  FT_ENOMEM = -2,        /* host or device allocation failed */
  FT_EHIP = -3,          /* a HIP runtime call failed; the message names it */
  FT_EUNSUPPORTED = -4,  /* valid request this build does not implement */
  FT_ESTATE = -5,        /* call not valid in the object's current state */
  FT_EIO = -6            /* a file operation failed; the message names it and errno */
};

enum { FT_MXFP4 = 0, FT_NVFP4 = 1 };
enum { FT_PREFILL_EXACT = 0, FT_PREFILL_MXFP4 = 1 };

/* Largest token count of one ft_route / ft_moe_decode call. */
#define FT_MAX_DECODE_TOKENS 16
/* Largest k. */
#define FT_MAX_TOPK 16

typedef struct ft_ctx ft_ctx;
typedef struct ft_layer ft_layer;

/*
 * Expert blob: one expert's gate [I][H], up [I][H] and down [H][I] matrices in the
 * library's tiled FP4 layout, each sub-tensor starting on a 4096-byte boundary so that one
 * copy moves a whole expert (the FTW rule that every tensor is 4096-aligned:
 * lowalt.boxinlu2.cn article, section 三).  A 4096-byte header holds the format, sizes and
 * the three NVFP4 tensor scales.  Blobs are produced by ft_pack_expert.
 */

/* Bytes of one blob (a multiple of 4096).  H and I must be positive multiples of 128, and the
 * blob must stay under 2 GiB (FT_EINVAL otherwise; ft_layer_create applies the same rule). */
FT_API int ft_blob_bytes(int format, int H, int I, uint64_t* bytes);

/*
 * Pack one expert into `blob` (host memory, ft_blob_bytes() bytes).  Logical inputs,
 * row-major: codes uint8 [rows][K/2] with element 2i in the low nibble; scales uint8
 * [rows][K/B] (MXFP4: E8M0, B = 32; NVFP4: E4M3, B = 16) along the contraction axis K.
 * gate/up: rows = I, K = H; down: rows = H, K = I.  tensor_scales: 3 fp32 (gate, up,
 * down), used by NVFP4, may be NULL for MXFP4.  Pure host function.
 */
FT_API int ft_pack_expert(int format, int H, int I,
                          const uint8_t* gate_codes, const uint8_t* gate_scales,
                          const uint8_t* up_codes, const uint8_t* up_scales,
                          const uint8_t* down_codes, const uint8_t* down_scales,
                          const float* tensor_scales, void* blob);

/*
 * Context: device, internal copy stream, host thread pool for host-computed experts and disk
 * reads (FT_HOST_THREADS threads, default min(16, hardware threads); after a job its workers
 * spin for 0.5 ms before they sleep).  Calls that use one context (or its layers) must not run
 * concurrently from several host threads.
 */
FT_API int ft_ctx_create(int device, ft_ctx** out);
FT_API int ft_ctx_destroy(ft_ctx* ctx);

/*
 * Host placement of a context.  The host experts read the pinned blob store and the streamed
 * copies cross PCIe from it, with the CPU side's memory bandwidth setting Bh (smzdm explainer
 * a825qpgl, section 二: the CPU side's effective memory bandwidth; mubeitech explainer: the
 * CPU computes in host memory without crossing PCIe).  ft_ctx_create therefore binds the
 * pool's worker threads to the CPUs of the GPU's NUMA node (read from sysfs through the GPU's
 * PCI bus id) that the process may run on, unless FT_HOST_AFFINITY=0.  *node is that node
 * (-1 when the platform reports none), *pinned_cpus the CPUs the workers are bound to (0: not
 * bound).  A caller places the pinned blob store on the same node by allocating it from a
 * thread bound to those CPUs (the pages land on the allocating thread's node).
 */
FT_API int ft_ctx_numa(const ft_ctx* ctx, int* node, int* pinned_cpus);

typedef struct ft_layer_desc {
  int32_t H, I, E, k, n_shared;
  int32_t format;             /* FT_MXFP4 or FT_NVFP4 */
  int32_t n_slots;            /* slots in the device pool (1 .. E) */
  int32_t max_tokens;         /* largest decode T (1 .. FT_MAX_DECODE_TOKENS) */
  const float* router_w;      /* device fp32 [E][H] */
  const float* router_b;      /* device fp32 [E], or NULL for no bias */
  void* pool;                 /* device, n_slots * blob_stride bytes */
  const void* shared_blobs;   /* device, n_shared blobs at blob_stride, or NULL if none */
  const void* host_blobs;     /* pinned host, E blobs at blob_stride, or NULL; a layer that is
                                 not resident decodes from these or from a disk tier
                                 (ft_layer_set_disk_tier) */
  uint64_t blob_stride;       /* >= ft_blob_bytes(), multiple of 4096 */
  int32_t resident;           /* 1: slot e already holds expert e for every e (needs
                                 n_slots == E); 0: the pool starts empty */
  int32_t flags;              /* 0 or FT_LAYER_PREFILL_MXFP4 */
} ft_layer_desc;

/*
 * FT_LAYER_PREFILL_MXFP4: prepare the layer for ft_moe_prefill(..., FT_PREFILL_MXFP4, ...).
 * An NVFP4 layer (which must be resident) gets its experts transcoded once, here, to MXFP4
 * blobs held by the library (E * ft_blob_bytes(FT_MXFP4, H, I) device bytes, freed by
 * ft_layer_destroy): each weight's exact value E2M1 x E4M3 x tensor scale is requantised
 * per 32 along K by the OCP MX rule (see ft_moe_prefill), so the tensor scale lives inside
 * the new values.  Later writes to the pool are not seen by that copy.  MXFP4 layers need no
 * copy (requantising an MXFP4 block reproduces its values) and ignore the flag.
 */
enum { FT_LAYER_PREFILL_MXFP4 = 1 };

/* Create a layer over caller-owned buffers; allocates the library's device workspace. */
FT_API int ft_layer_create(ft_ctx* ctx, const ft_layer_desc* desc, ft_layer** out);
FT_API int ft_layer_destroy(ft_layer* layer);

/*
 * Routing (top-k softmax; smzdm explainer a825qpgl, section 二: each MoE layer's gate
 * activates a few of its experts per token, 6 of 256 in the DeepSeek-V4-Flash layer, and the
 * chosen experts' outputs are later merged by these routing weights).  logits = x W_r^T + b
 * in fp32; idx = the k largest logits in rank order (descending, ties to the lower index);
 * w = softmax over those k logits (the full softmax over E renormalised over the kept k is the
 * same number).  x: device bf16 [T][H]; idx: device int32 [T][k]; w: device fp32 [T][k].
 * 1 <= T <= max_tokens.  FT_EINVAL for a null pointer or T out of range.  Asynchronous on
 * `stream`.
 */
FT_API int ft_route(ft_ctx* ctx, const ft_layer* layer, const uint16_t* x, int T,
                    int32_t* idx, float* w, void* stream);

typedef struct ft_decode_stats {
  int32_t n_selected;   /* distinct routed experts of the call */
  int32_t n_hits;       /* of those, resident in the pool */
  int32_t n_miss;       /* m */
  int32_t q;            /* the split rule's q for m */
  int32_t n_streamed;   /* misses copied into slots this call */
  int32_t n_host;       /* misses computed on host cores */
  int32_t n_evicted;
  int32_t step;         /* decode-call counter of this layer (the LRU clock) */
  double qstar;         /* m * Bp / Bh */
  double bp, bh;        /* bandwidths used (bytes/s) */
  double host_us;       /* wall time of the host experts */
  double wait_us;       /* wall time blocked on the routing read-back */
  /* runtime measurements taken by this call (0 where there was nothing to measure):
     bp_obs from the previous call's streamed copies, bh_obs from this call's host experts
     (see ft_set_miss_policy) */
  double bp_obs, bh_obs;
  /* cross-layer prefetch (see ft_set_prefetch): experts this call admitted to and started
     copying into the linked next layer's pool, and this call's hits on slots that a prefetch
     filled and nothing has used since */
  int32_t n_prefetched, n_prefetch_hits;
  /* host-memory tier over an FTW file (see ft_layer_set_disk_tier): blobs this call read from
     disk, and the wall time of those reads */
  int32_t n_disk;
  double disk_us;
  /* GPU load (FT_SPLIT_LOAD): the previous call's GPU time for its hit and shared experts in
     microseconds (0 if none was timed) and the per-expert GPU time this call's split used,
     in seconds */
  double gpu_us_obs, t_gpu;
} ft_decode_stats;

/*
 * Decode T tokens (1 <= T <= max_tokens).  x: device bf16 [T][H]; y: device fp32 [T][H].
 * All-resident layers run fully asynchronously.  Otherwise the call blocks until the
 * routing of these tokens is read back, classifies hits and misses, streams q misses into
 * slots on the internal copy stream, enqueues the GPU experts on `stream`, computes the
 * other misses on host cores, enqueues their results and the combine, and returns; y is
 * valid after `stream` syncs.  stats may be NULL (asynchronous path: counts are filled
 * only where known on the host, i.e. in the miss path).  Both weight formats decode on the
 * GPU and on the host: an NVFP4 weight is its E2M1 value times its block's E4M3 scale, and
 * each matrix's fp32 tensor scale (blob header) multiplies that matrix's product.
 */
FT_API int ft_moe_decode(ft_ctx* ctx, ft_layer* layer, const uint16_t* x, int T, float* y,
                         ft_decode_stats* stats, void* stream);

/*
 * Prefill (large T, all experts resident; smzdm explainer aomxznrn, "FreeToken干的事", item 4:
 * prefill takes its own, compute-bound strategy).  Routing as ft_route; the (token, choice)
 * pairs are sorted by expert (stable), every expert's rows go through one grouped SwiGLU
 * FFN, and y[t] = sum_j w[t][j] * FFN_{idx[t][j]}(x[t]).  FT_PREFILL_EXACT forms the sum
 * over j by fp32 atomic adds into y as the down projection's blocks finish, in no fixed
 * order, so two calls on the same input can differ by fp32 rounding; FT_PREFILL_MXFP4 sums
 * in rank order and is deterministic.
 *   FT_PREFILL_EXACT: bf16 activations, the exact FP4 weights, bf16 MFMA, fp32 accumulate,
 *     h rounded to bf16 (as decode).
 *   FT_PREFILL_MXFP4: both operands FP4 on the scaled-FP4 MFMA.  x and h are quantised per
 *     32 along K by the OCP MX rule: scale 2^(floor(log2 max|v|) - 2), exponent clamped to
 *     [-127, 127], an all-zero block gets scale code 0; each v / scale rounds to the nearest
 *     E2M1 value, ties to the even code, saturating at 6, with v's sign bit.  The weights are
 *     the layer's MXFP4 blobs, or for NVFP4 the copy made by FT_LAYER_PREFILL_MXFP4
 *     (FT_ESTATE without it).  h is quantised from its fp32 value.
 * x: device bf16 [T][H]; y: device fp32 [T][H].  ws: device workspace of at least
 * ft_moe_prefill_workspace_size(layer, T, mode) bytes, 256-byte aligned, caller-owned; it
 * holds the routing, permutation and intermediates of the call until the next call.
 * Errors: FT_EINVAL (bad T, mode, pointers or workspace), FT_ESTATE (layer not resident, or
 * no MXFP4 weights for FT_PREFILL_MXFP4), FT_EUNSUPPORTED (shared experts).  Asynchronous.
 */
FT_API int ft_moe_prefill_workspace_size(const ft_layer* layer, int T, int mode, size_t* bytes);
FT_API int ft_moe_prefill(ft_ctx* ctx, ft_layer* layer, const uint16_t* x, int T, float* y,
                          int mode, void* ws, size_t ws_bytes, void* stream);

/*
 * ft_moe_prefill without a workspace argument, for callers that cannot allocate device memory
 * (code under HIP graph capture, serving loops or harnesses that forbid allocation).  The same
 * kernels run with their workspace in a static device array of
 * FT_PREFILL_STATIC_SCRATCH_BYTES that the library's code object holds on every GPU it runs on
 * until the process ends; the call itself allocates nothing.  The caller still passes x
 * (device bf16 [T][H]) and y (device fp32 [T][H]); results and errors are those of
 * ft_moe_prefill, plus FT_EINVAL when the call's workspace
 * (ft_moe_prefill_workspace_size(layer, T, mode)) exceeds the static array.  Every call on
 * one GPU shares that GPU's array, which keeps the last call's contents: calls that overlap
 * on one GPU (on different streams, or from different contexts or threads) race and must be
 * serialised by the caller.  Asynchronous on `stream`.
 */
#define FT_PREFILL_STATIC_SCRATCH_BYTES (64u << 20)
FT_API int ft_moe_prefill_noalloc(ft_ctx* ctx, ft_layer* layer, const uint16_t* x, int T,
                                  float* y, int mode, void* stream);

/*
 * The split rule (smzdm explainer a825qpgl, section 二; lowalt.boxinlu2.cn article,
 * section 二): qstar = m * Bp / Bh; q = floor(qstar + 1/2) clamped to [0, m] (Bh <= Bp
 * gives m).  FT_EINVAL if m < 0, Bp <= 0 or Bh <= 0.  Pure host function.
 */
FT_API int ft_qstar_split(int m, double Bp, double Bh, int* q, double* qstar);

/*
 * The split's makespan variant: both sides run at once, the copies at Bp and the host experts
 * with the bandwidth the copies leave, Bh - Bp (lowalt.boxinlu2.cn article, section 二), and
 * the q with the earlier finish wins: the integer q in [0, m] minimising
 * max(q / Bp, (m - q) / (Bh - Bp)), lowest q on ties; Bh <= Bp gives m.  FT_EINVAL as
 * ft_qstar_split.  Pure host function.
 */
enum { FT_SPLIT_ROUND = 0, FT_SPLIT_MAKESPAN = 1, FT_SPLIT_LOAD = 2 };
FT_API int ft_qstar_split_makespan(int m, double Bp, double Bh, int* q);

/*
 * The split's load variant (mubeitech explainer: the balancing watches the PCIe bandwidth, the
 * CPU's compute and the GPU's load, so that the two sides finish at the same moment): with g0
 * experts the GPU computes anyway (hits and shared experts), blob bytes per expert and t_gpu
 * seconds of GPU time per expert, the integer q in [0, m] minimising
 *   max( max(g0 t_gpu, q blob / Bp) + q t_gpu,  (m - q) blob / (Bh - Bp) )
 * (the GPU runs its g0 experts while the q copies stream and then the q streamed ones; the
 * host runs the rest with the bandwidth the copies leave), lowest q on ties; Bh <= Bp gives m;
 * t_gpu = 0 is the makespan variant.  FT_EINVAL for m < 0, g0 < 0, Bp, Bh or blob <= 0, or
 * t_gpu negative or not finite.  Pure host function.
 */
FT_API int ft_qstar_split_load(int m, int g0, double Bp, double Bh, double blob, double t_gpu,
                               int* q);

/*
 * Startup probes of the split rule's two bandwidths (smzdm explainer a825qpgl, section 二: q*
 * is computed from measured bandwidths, Bp the measured PCIe transfer rate and Bh the CPU
 * side's effective memory bandwidth):
 * Bp = median bytes/s of a pinned hipMemcpyAsync of one expert blob to the
 * device; Bh = median bytes/s of the host expert FFN over one blob on the host threads.  The
 * repetitions cycle over up to 8 distinct blobs, more than a host cache holds, as decode
 * reads them.  Needs host_blobs, or a disk tier not yet used by a decode call (the probe then
 * reads experts 0..7 into its first host-memory slots).  Blocks.  The values are stored in
 * the layer and used by decode.
 */
FT_API int ft_measure_bandwidth(ft_ctx* ctx, ft_layer* layer, double* Bp, double* Bh);
/*
 * HBM read-bandwidth probe: a plain streaming read of `bytes` (>= 1 MiB, a multiple of 16) of
 * device memory at buf in two forms, each launched reps + 1 times (the first untimed):
 * 16-byte register loads by 32 workgroups per compute unit, and direct global -> LDS copies
 * of 1 KB blocks by one workgroup per compute unit.  *GBps = bytes * reps / the timed span
 * of the faster form.  A buffer well above the 256 MB Infinity Cache measures HBM.  The
 * reference against which kernels' achieved bandwidth is also quoted.  Blocks.  FT_EINVAL
 * for bad arguments.
 */
FT_API int ft_probe_hbm_read(ft_ctx* ctx, const void* buf, uint64_t bytes, int reps,
                             double* GBps);
/* Override Bp and Bh (bytes/s, both > 0). */
FT_API int ft_set_bandwidth(ft_layer* layer, double Bp, double Bh);
/* Force q for every later decode call (q >= 0, clamped to m), or restore the rule (q < 0). */
FT_API int ft_force_q(ft_layer* layer, int q);

/*
 * Miss-path policy of a layer (the pages let q* follow the hardware as it runs: smzdm
 * explainer a825qpgl, section 二; lowalt.boxinlu2.cn article, section 二).
 *   rule: FT_SPLIT_ROUND (default: q = round(q*)), FT_SPLIT_MAKESPAN or FT_SPLIT_LOAD (see
 *     ft_qstar_split_load; t_gpu is measured on every call of the layer: the GPU time of its
 *     hit and shared experts' kernels, from events around them, per expert, read at the next
 *     call; the estimate moves toward each observation by alpha, or takes it when alpha is 0;
 *     until a first observation t_gpu is 0).
 *   alpha in [0, 1]: 0 (default) keeps Bp and Bh as measured or set.  alpha > 0 re-measures
 *     them during decode and moves each estimate toward its observation by alpha
 *     (est += alpha (obs - est)), before the next call's split:
 *       Bp_obs = bytes of the streamed blobs / their copy time on the copy stream (events
 *                around the copies, read at the next miss-path call);
 *       Bh_obs = bytes of the host-computed blobs / the host experts' wall time, plus the
 *                current Bp when copies ran at the same time (the copies take Bp of the
 *                host's memory bandwidth while they run).
 *     Calls with nothing streamed (or nothing computed on the host) leave that estimate.
 * The values a call used are in its ft_decode_stats (bp, bh), its observations in bp_obs,
 * bh_obs.  FT_EINVAL for an unknown rule or alpha outside [0, 1].
 */
FT_API int ft_set_miss_policy(ft_layer* layer, int rule, double alpha);

/*
 * Cross-layer prefetch with double buffering: while the GPU computes one layer, the experts
 * the next layer will probably need stream into VRAM in the background (mubeitech article,
 * closing section; lpnh.cn article, section 2.3, predictive prefetch).  Links `layer` to
 * `next`, both miss-path layers (partial pools) of one context with the same H.  Each later
 * ft_moe_decode of `layer`:
 *   - predicts next's routing by applying next's router (top-k softmax) to layer's own input
 *     x, in the same kernel launch as layer's own routing;
 *   - after enqueueing layer's own copies and kernels, marks the predicted experts already in
 *     next's pool as used at next's coming call, then admits up to `depth` of the others, by
 *     descending summed predicted weight (ties to the lower id), through next's slot rule
 *     (lowest empty slot, else the least recently used one not used or fetched for that call)
 *     and copies them on the copy stream, behind layer's own copies and after next's previous
 *     kernels;
 *   - reports the count in ft_decode_stats.n_prefetched.
 * next's following ft_moe_decode finds them resident; its kernels wait for those copies, and
 * its n_prefetch_hits counts its hits on them.  The two pools are separate buffers, so the
 * copies into next's never touch what layer's kernels read (the double buffer).
 * next = NULL or depth = 0 unlinks.  A layer prefetches for at most one next, and a layer
 * is the next of at most one layer; destroying either unlinks.  FT_EINVAL for a null layer,
 * depth < 0 or above next's n_slots, next == layer, another context, a resident pool, a
 * different H, or a next already linked from another layer.  FT_ENOMEM if the prediction
 * buffers cannot be allocated.
 */
FT_API int ft_set_prefetch(ft_layer* layer, ft_layer* next, int depth);

/*
 * out[i] = bf16(float(x[i]) + scale * y[i]) for 0 <= i < n: the product and the sum each
 * rounded to fp32 (no fused multiply-add), the result rounded to nearest even bf16 (NaN stays
 * NaN).  A residual step for chaining decode layers (one layer's scaled output added to its
 * input gives the next layer's input); x, y and out are device arrays (bf16 bits, fp32, bf16
 * bits), out may alias x.  n >= 0 (0 does nothing).  FT_EINVAL for a null context, n < 0 or
 * null arrays with n > 0.  Asynchronous on `stream`.
 */
FT_API int ft_residual_bf16(ft_ctx* ctx, const uint16_t* x, const float* y, float scale,
                            int64_t n, uint16_t* out, void* stream);

/*
 * FTW expert files (lowalt.boxinlu2.cn article, section 三: every tensor 4096-aligned, so a
 * blob moves from disk in a few large direct reads instead of many fragmented ones).
 * Layout: bytes [0, 4096) hold the header (magic "FTW1", version 1, format, H, I, E,
 * n_shared, blob bytes, blob stride, data offset, file bytes; little-endian); blob i sits at
 * 4096 + i * stride for i < E + n_shared (routed experts first, then shared ones), stride =
 * ft_blob_bytes(format, H, I), which is a multiple of 4096, and inside a blob every tensor
 * starts on a 4096 boundary.  The blobs are the bytes ft_pack_expert writes, unchanged.
 */
typedef struct ft_ftw ft_ftw;
typedef struct ft_ftw_info {
  int32_t format, H, I, E, n_shared;
  int32_t direct;          /* 1 if the file is read with O_DIRECT (page cache bypassed) */
  int32_t staged;          /* 1 once direct reads go through aligned host buffers and a copy
                              (the kernel refuses O_DIRECT into some memory, such as the GPU
                              driver's pinned host memory, or FT_FTW_STAGED asked for it) */
  int32_t reserved;
  uint64_t blob_bytes;     /* = blob stride in the file */
  uint64_t file_bytes;
} ft_ftw_info;

/*
 * Write an FTW file from E + n_shared packed blobs in host memory at src_stride bytes apart
 * (routed experts 0..E-1, then the shared ones).  Each blob's header must name the given
 * format, H and I.  The file is created or truncated, written and flushed to the device.
 * FT_EINVAL for bad dimensions, pointers, a stride below the blob size or a blob of other
 * dimensions; FT_EIO for a file error.  Host only, blocks.
 */
FT_API int ft_ftw_write(const char* path, int format, int H, int I, int E, int n_shared,
                        const void* blobs, uint64_t src_stride);

/*
 * Open an FTW file for reading and validate its header against its size.  flags:
 * FT_FTW_DIRECT asks for O_DIRECT reads; where the file system refuses them the file is read
 * through the page cache instead (ft_ftw_info.direct says which).  A direct read into memory
 * the kernel cannot pin for it (EFAULT) is redone through an aligned staging buffer per
 * thread and a copy, and so are all later reads of the file; FT_FTW_STAGED asks for that from
 * the start.  FT_EIO for a file error, FT_EINVAL for a file that is not a valid FTW file.
 * Host only.
 */
enum { FT_FTW_DIRECT = 1, FT_FTW_STAGED = 2 };
FT_API int ft_ftw_open(const char* path, int flags, ft_ftw** out);
FT_API int ft_ftw_get_info(const ft_ftw* f, ft_ftw_info* info);
FT_API int ft_ftw_close(ft_ftw* f);

/*
 * Read blobs ids[0..n-1] (each < E + n_shared) into dst + i * dst_stride, in requests of
 * `chunk` bytes (0: one request per blob), spread over ctx's host threads (ctx may be NULL:
 * the calling thread alone).  dst is host memory (pinned or not); with O_DIRECT, dst,
 * dst_stride and chunk must be multiples of 4096.  seconds (may be NULL) receives the wall
 * time.  FT_EINVAL for bad ids, sizes or alignment; FT_EIO for a read error or a short file.
 * Host only, blocks.
 */
FT_API int ft_ftw_read(ft_ctx* ctx, ft_ftw* f, const int32_t* ids, int n, void* dst,
                       uint64_t dst_stride, uint64_t chunk, double* seconds);

/*
 * Three-tier store for a miss-path layer (smzdm explainer aomxznrn, "FreeToken干的事", item 1:
 * disk -> system memory -> VRAM): host memory holds n_ram expert blobs in `ram` (caller-owned
 * pinned memory, n_ram * blob_stride bytes, 4096-aligned) as a second slot pool, and the rest
 * stay in the FTW file f (same format, H, I, E and n_shared as the layer; f must stay open
 * while attached).  Each later ft_moe_decode takes its VRAM misses, in miss order: those in
 * host memory are marked used at the tier's call counter, the others are read from the file
 * (1 MiB requests over the host threads) into slots taken by the pool's slot rule (lowest
 * empty, else least recently used among those not used in this call); streamed misses are then
 * copied from, and host-computed ones computed in, those slots.  ft_decode_stats.n_disk and
 * disk_us report the reads.  Attaching empties the tier; f = NULL detaches (the layer goes back
 * to host_blobs, FT_ESTATE at decode if it has none).  n_ram must be in
 * [max_tokens * k, E].  FT_EINVAL for a resident layer, a file of other dimensions, bad n_ram
 * or alignment, or a layer linked by ft_set_prefetch (prefetch copies read host_blobs).
 */
FT_API int ft_layer_set_disk_tier(ft_layer* layer, ft_ftw* f, void* ram, int n_ram);
/* Test hook: the host-memory tier's tables, expert -> slot [E] and slot -> expert [n_ram]. */
FT_API int ft_debug_host_tier(const ft_layer* layer, int32_t* e2r, int32_t* r2e);
/* Test hook (host only): run `jobs` jobs on a fresh pool of `threads` threads, pausing
 * pause_us between them (a pause past the workers' spin makes them sleep and be woken), and
 * check every job ran on every index exactly once.  FT_ESTATE if one did not. */
FT_API int ft_debug_pool_stress(int threads, int jobs, int pause_us);
/* Test hook (host only): the CPUs of a Linux cpulist string ("0-3,8,10-11"), ascending as
 * written; *n = their count (0 for a malformed list), the first cap written to cpus. */
FT_API int ft_debug_parse_cpulist(const char* text, int32_t* cpus, int cap, int* n);
/* Test hook (host only) of the no-throw rule: kind 0 returns FT_OK; kind 1 throws
 * std::bad_alloc, 2 std::runtime_error, 3 std::system_error inside an entry point, which
 * returns FT_ENOMEM, FT_ESTATE and FT_ENOMEM for them.  FT_EINVAL for another kind. */
FT_API int ft_debug_throw(int kind);

FT_API const char* ft_last_error(void);

/*
 * Kernel timing.  After ft_profile_begin(layer, n) the next n eager decode (or prefill) calls
 * launch their two expert kernels, gate/up (+SwiGLU) and down, with start/stop HIP events
 * that the dispatches record on the call's stream (so host-side gaps are not counted).
 * ft_profile_end synchronises those events and returns the mean kernel durations in
 * microseconds and the number of calls recorded.  Not for calls under graph capture.
 */
FT_API int ft_profile_begin(ft_layer* layer, int n);
FT_API int ft_profile_end(ft_layer* layer, double* gateup_us, double* down_us, int* n_recorded);

/* ---- test hooks ---------------------------------------------------------------------- */

/* Dequantise one matrix (0 gate, 1 up, 2 down) of pool slot `slot` (or, when slot < 0, of
 * shared expert -1 - slot) to device fp32 [rows][K] in logical order. */
FT_API int ft_debug_dequant(const ft_layer* layer, int slot, int matrix, float* out,
                            void* stream);
/* Host copies of the expert->slot table [E] and slot->expert table [n_slots] (-1 = none),
 * read back from the device tables the kernels use.  Blocks. */
FT_API int ft_debug_tables(const ft_layer* layer, int32_t* e2s, int32_t* s2e);
/* The library's host expert FFN on one blob (host memory): x host bf16 [T][H] -> y host
 * fp32 [T][H].  Runs on the calling thread plus the context's pool when ctx != NULL. */
FT_API int ft_host_expert_ffn(ft_ctx* ctx, int format, int H, int I, const void* blob,
                              const uint16_t* x, int T, float* y);
/* Prefill permutation of the last ft_moe_prefill call: counts [E], offsets [E+1],
 * pos [T][k] (device int32), copied from the workspace `ws` of that call. */
FT_API int ft_debug_prefill_perm(const ft_layer* layer, const void* ws, int T,
                                 int32_t* counts, int32_t* offsets, int32_t* pos,
                                 void* stream);
/* Routing of the last ft_moe_prefill call: idx [T][k] (device int32) and w [T][k] (device
 * fp32), copied from the workspace `ws` of that call. */
FT_API int ft_debug_prefill_route(const ft_layer* layer, const void* ws, int T, int32_t* idx,
                                  float* w, void* stream);
/* MXFP4 operands of the last FT_PREFILL_MXFP4 call, copied from its workspace: which = 0:
 * the quantised tokens, codes [T][H/2] (two per byte, low nibble first) and E8M0 scales
 * [T][H/32]; which = 1: the quantised h in permuted row order, codes [T*k][I/2] and scales
 * [T*k][I/32].  codes and scales are device buffers. */
FT_API int ft_debug_prefill_quant(const ft_layer* layer, const void* ws, int T, int which,
                                  uint8_t* codes, uint8_t* scales, void* stream);
/* The MXFP4 blob that FT_PREFILL_MXFP4 uses for expert e (ft_blob_bytes(FT_MXFP4, H, I)
 * bytes), copied to the device buffer out.  FT_ESTATE if the layer has none. */
FT_API int ft_debug_prefill_weights(const ft_layer* layer, int e, void* out, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* FT_H */
