// Decode kernels of libft for gfx950 (CDNA4).
//
// One decode call of T <= 16 tokens (the MoE layer of the FreeToken pages: a gate picks k
// experts per token and their outputs are merged by routing weight — smzdm explainer
// a825qpgl, section 二) runs as four kernels on the caller's stream:
//   k_logits   logits[t][e] = x_t . W_r[e] + b[e] in fp32; one workgroup per expert row.
//   k_gateup   prologue: every workgroup takes the top-k of the logits (ties to the lower
//              index), the softmax over the kept logits and the list of distinct experts
//              with their token columns, in LDS (workgroup 0 also publishes them for the
//              next kernel); then per (expert, 16-row tile): g = W_g x, u = W_u x on the
//              16x16x32 bf16 MFMA with FP4 codes converted to bf16 in registers (exact),
//              h = bf16(silu(g) * u).  Tokens are the MFMA's N columns, so every weight is
//              read once per call however many tokens share the expert.
//   k_down     per (expert, 16-row tile of W_d): y_e = W_d h into the partial buffer
//              P[t * kk + j] (j = top-k rank, k + s for shared expert s).
//   k_combine  y_t = sum_j w_tj P[t][j] + sum_s P[t][k + s], in that order.
// (k_down_combine does both of the last two in one pass where its grid fills the chip.)
// Both block-scaled formats run through the same kernels (template parameter FMT): MXFP4
// scales are powers of two and go into the hardware FP4 -> bf16 convert; an NVFP4 weight is
// E2M1 x E4M3 (at most 6 significant bits, so exact in bf16) and its fp32 tensor scale,
// read from the blob header, multiplies the fp32 result of each matrix.
// Workgroups never wait on each other inside a kernel: on this chip a device-scope fence
// writes back and invalidates the issuing XCD's L2, so data moves between workgroups only
// at kernel boundaries (except in the small routing kernel of the miss path, k_route_small,
// whose last workgroup reads what the others released).
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>

#include <map>
#include <mutex>
#include <utility>

#include "ft_device.h"

namespace ft {

constexpr int kMaxItems = FT_MAX_DECODE_TOKENS * FT_MAX_TOPK + 4;
constexpr int kRouteMaxEPerLane = 16;  // E <= 1024

// ---- router logits ----------------------------------------------------------------------
// One workgroup per expert row.  Thread tid covers H positions tid*4 + i*1024.  TB is the
// token count rounded up to a power of two; rows past T re-read row T-1 and are dropped,
// and positions past H are clamped and masked at the FMA, so no load sits behind a branch
// and a lane's weight and token loads are all in flight together.
template <int TB>
__device__ __forceinline__ void logit_row(const uint16_t* __restrict__ x,
                                          const float* __restrict__ wr,
                                          const float* __restrict__ b, int T, int H, int E,
                                          int e, float* __restrict__ logits) {
  constexpr int NI = TB >= 8 ? 2 : (TB >= 4 ? 4 : 6);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  float acc[TB];
#pragma unroll
  for (int t = 0; t < TB; ++t) acc[t] = 0.f;
  const float* wrow = wr + (uint64_t)e * H;
  for (int base = tid * 4; base < H; base += NI * 1024) {
    float4 wv[NI];
    uint2 xv[TB][NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) wv[i] = *(const float4*)(wrow + min(base + i * 1024, H - 4));
#pragma unroll
    for (int t = 0; t < TB; ++t) {
      const uint16_t* xr = x + (uint64_t)min(t, T - 1) * H;
#pragma unroll
      for (int i = 0; i < NI; ++i) xv[t][i] = *(const uint2*)(xr + min(base + i * 1024, H - 4));
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const float m = base + i * 1024 < H ? 1.f : 0.f;
      const float4 w4 = make_float4(wv[i].x * m, wv[i].y * m, wv[i].z * m, wv[i].w * m);
#pragma unroll
      for (int t = 0; t < TB; ++t) {
        acc[t] = fmaf(w4.x, bf16_lo(xv[t][i].x), acc[t]);
        acc[t] = fmaf(w4.y, bf16_hi(xv[t][i].x), acc[t]);
        acc[t] = fmaf(w4.z, bf16_lo(xv[t][i].y), acc[t]);
        acc[t] = fmaf(w4.w, bf16_hi(xv[t][i].y), acc[t]);
      }
    }
  }
  __shared__ float red[4][TB];
#pragma unroll
  for (int t = 0; t < TB; ++t) {
    const float sum = wave_sum(acc[t]);
    if (lane == 0) red[wave][t] = sum;
  }
  __syncthreads();
  if (tid < T)
    logits[(uint64_t)tid * E + e] =
        ((red[0][tid] + red[1][tid]) + (red[2][tid] + red[3][tid])) + (b ? b[e] : 0.f);
}

template <int TB>
__global__ __launch_bounds__(256) void k_logits(const uint16_t* __restrict__ x,
                                                const float* __restrict__ wr,
                                                const float* __restrict__ b, int T, int H, int E,
                                                float* __restrict__ logits) {
  logit_row<TB>(x, wr, b, T, H, E, blockIdx.x, logits);
}

// ---- top-k and the work list in LDS -------------------------------------------------------
struct TopkLds {
  int idx[kMaxCols][FT_MAX_TOPK];
  float w[kMaxCols][FT_MAX_TOPK];
};

// Order-preserving key of a float: a > b  <=>  key(a) > key(b) (NaN is mapped to -inf first).
__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Per-token top-k by a radix select: one wave per token finds the k-th largest key with a
// 32-step bitwise search whose counts are wave ballots (no cross-lane shuffles), keeps
// every key above it plus the lowest-index keys equal to it, compacts the k winners into
// LDS and ranks them (logit descending, ties to the lower index).  Weights are the softmax
// over the k kept logits.  EPL = experts per lane (E <= 64 * EPL).  Called by all 256
// threads; ends synchronised.
template <int EPL>
__device__ __forceinline__ void topk_tokens(const float* logits, int T, int E, int k, TopkLds& s,
                                            float (*c_val)[FT_MAX_TOPK],
                                            int (*c_idx)[FT_MAX_TOPK]) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int t = wave; t < T; t += 4) {
    float v[EPL];
    uint32_t key[EPL];
    // loads are unconditional (clamped to a valid index) so all are in flight together
#pragma unroll
    for (int i = 0; i < EPL; ++i) v[i] = logits[(uint64_t)t * E + min(lane + 64 * i, E - 1)];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      if (v[i] != v[i]) v[i] = -INFINITY;           // NaN logits never win
      key[i] = lane + 64 * i < E ? order_key(v[i]) : 0u;  // padding ranks below -inf
    }
    uint32_t tau = 0;
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t cand = tau | (1u << bit);
      int c = 0;
#pragma unroll
      for (int i = 0; i < EPL; ++i) c += __popcll(__ballot(key[i] >= cand));
      if (c >= k) tau = cand;
    }
    int n_gt = 0;
#pragma unroll
    for (int i = 0; i < EPL; ++i) n_gt += __popcll(__ballot(key[i] > tau));
    const int need_eq = k - n_gt;
    int eq_before = 0, sel_before = 0;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const uint64_t eqb = __ballot(key[i] == tau);
      const bool sel = key[i] > tau ||
                       (key[i] == tau && eq_before + __popcll(eqb & lt_mask) < need_eq);
      const uint64_t selb = __ballot(sel);
      if (sel) {
        const int pos = sel_before + __popcll(selb & lt_mask);
        c_val[t][pos] = v[i];
        c_idx[t][pos] = lane + 64 * i;
      }
      eq_before += __popcll(eqb);
      sel_before += __popcll(selb);
    }
  }
  __syncthreads();
  // rank the k winners of each token: thread (t, j) handles winner j of token t
  const int tid = threadIdx.x;
  if (tid < T * k) {
    const int t = tid / k, j = tid % k;
    const float vj = c_val[t][j];
    const int ej = c_idx[t][j];
    float vq[FT_MAX_TOPK];
    int eq[FT_MAX_TOPK];
#pragma unroll
    for (int q = 0; q < FT_MAX_TOPK; ++q) {
      vq[q] = c_val[t][min(q, k - 1)];
      eq[q] = c_idx[t][min(q, k - 1)];
    }
    int rank = 0;
    float vmax = vj;
#pragma unroll
    for (int q = 0; q < FT_MAX_TOPK; ++q) {
      if (q < k) {
        rank += (vq[q] > vj || (vq[q] == vj && eq[q] < ej));
        vmax = fmaxf(vmax, vq[q]);
      }
    }
    float sum = 0.f;
#pragma unroll
    for (int q = 0; q < FT_MAX_TOPK; ++q)
      if (q < k) sum += expf(vq[q] - vmax);
    s.idx[t][rank] = ej;
    s.w[t][rank] = expf(vj - vmax) / sum;
  }
  __syncthreads();
}

// Single-token top-k for E <= 256 by sorting networks on 64-bit keys: high word = the logit's
// order key, low word = (255 - expert) << 24 | (slot + 1), so among equal logits the lower
// expert ranks first and the expert's pool slot rides along as payload (the index field is
// unique, so the payload never decides a comparison).  Wave w sorts experts 64 w .. + 63 (one
// per lane) with a bitonic network of lane-pair exchanges; wave 0 then merges the four waves'
// R best (R = 8 or 16 >= k) with the bitonic merge network, which leaves the k largest
// logits in rank order in lanes 0 .. k-1.
struct SortLds {
  uint64_t key[4][FT_MAX_TOPK];
};

// Lanes of a bitonic compare-exchange step (merge size kk, distance j) that keep the larger
// key: the lower lane of a pair in descending blocks, the upper one in ascending blocks.
constexpr uint64_t keep_max_lanes(int kk, int j) {
  uint64_t m = 0;
  for (int l = 0; l < 64; ++l)
    if (((l & j) == 0) == ((l & kk) == 0)) m |= 1ull << l;
  return m;
}

template <int KK, int J>
__device__ __forceinline__ void cmpx(uint64_t& key) {
  const uint32_t ohi = xor_lane<J>((uint32_t)(key >> 32));
  const uint32_t olo = xor_lane<J>((uint32_t)key);
  const uint64_t other = ((uint64_t)ohi << 32) | olo;
  // take the partner's key where (partner larger) == (this lane keeps the max)
  const uint64_t gt = __builtin_amdgcn_ballot_w64(other > key);
  if (__builtin_amdgcn_inverse_ballot_w64(gt ^ ~keep_max_lanes(KK, J))) key = other;
}

// bitonic merge stage of size KK: distances KK/2 .. 1
template <int KK, int J = KK / 2>
__device__ __forceinline__ void bitonic_merge(uint64_t& key) {
  cmpx<KK, J>(key);
  if constexpr (J > 1) bitonic_merge<KK, J / 2>(key);
}

// sort of the 64 lanes' keys, descending from lane 0
__device__ __forceinline__ void bitonic64_desc(uint64_t& key) {
  bitonic_merge<2>(key);
  bitonic_merge<4>(key);
  bitonic_merge<8>(key);
  bitonic_merge<16>(key);
  bitonic_merge<32>(key);
  bitonic_merge<64>(key);
}

__device__ __forceinline__ float key_value(uint32_t key) {
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7fffffffu) : ~key);
}

struct ListLds;

// Top-k of one token's logits and its work list (item j = winner j, then the shared
// experts).  Called by all 256 threads; ends synchronised.
__device__ __forceinline__ void route_one_token(const float* logits, const int32_t* e2s, int E,
                                                int k, int n_shared, TopkLds& tk, ListLds& L,
                                                SortLds& sl);

struct ListLds {
  int n_items;
  int wave_tot[4];
  int expert[kMaxItems];
  int slot[kMaxItems];
  int ntok[kMaxItems];
  uint8_t tok[kMaxItems][kMaxCols];
  uint8_t jj[kMaxItems][kMaxCols];
  uint32_t tokmask[1024];   // per expert: bit t set when token t selected it
  int pos[1024];            // per expert: its item index
};

// Distinct routed experts in ascending id with their tokens ascending, then the shared
// experts (all tokens).  Per-expert token bitmasks make every step O(1) per thread: a
// token's column within its expert is the number of lower tokens in that mask.  All
// threads call; ends synchronised.
__device__ __forceinline__ void build_list(const TopkLds& tk, int T, int E, int k, int n_shared,
                                           const int32_t* e2s, ListLds& L) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  // this thread's four experts' slots, loaded first so the load overlaps the steps below
  int slot4[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) slot4[i] = e2s[min(tid * 4 + i, E - 1)];
  for (int e = tid; e < E; e += 256) L.tokmask[e] = 0u;
  __syncthreads();
  if (tid < T * k) atomicOr(&L.tokmask[tk.idx[tid / k][tid % k]], 1u << (tid / k));
  __syncthreads();
  int has[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int ee = tid * 4 + i;
    has[i] = ee < E ? (L.tokmask[ee] != 0u) : 0;
  }
  // experts of lower lanes in this wave: one ballot per position
  const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  int excl = 0, wtot = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint64_t b = __ballot(has[i]);
    excl += __popcll(b & below);
    wtot += __popcll(b);
  }
  if (lane == 0) L.wave_tot[wave] = wtot;
  __syncthreads();
  int base = excl;
  for (int w2 = 0; w2 < wave; ++w2) base += L.wave_tot[w2];
  const int n_routed = L.wave_tot[0] + L.wave_tot[1] + L.wave_tot[2] + L.wave_tot[3];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int ee = tid * 4 + i;
    if (has[i]) {
      L.pos[ee] = base;
      L.expert[base] = ee;
      L.slot[base] = slot4[i];
      L.ntok[base] = __popc(L.tokmask[ee]);
      ++base;
    }
  }
  __syncthreads();
  if (tid < T * k) {
    const int t = tid / k, j = tid % k;
    const int ee = tk.idx[t][j];
    const int it = L.pos[ee];
    const int col = __popc(L.tokmask[ee] & ((1u << t) - 1u));
    L.tok[it][col] = (uint8_t)t;
    L.jj[it][col] = (uint8_t)j;
  }
  if (tid < n_shared * kMaxCols) {
    const int sh = tid / kMaxCols, t = tid % kMaxCols;
    const int it = n_routed + sh;
    if (t == 0) { L.expert[it] = -1 - sh; L.slot[it] = -1 - sh; L.ntok[it] = T; }
    if (t < T) { L.tok[it][t] = (uint8_t)t; L.jj[it][t] = (uint8_t)(k + sh); }
  }
  if (tid == 0) L.n_items = n_routed + n_shared;
  __syncthreads();
}

__device__ __forceinline__ void route_one_token(const float* logits, const int32_t* e2s, int E,
                                                int k, int n_shared, TopkLds& tk, ListLds& L,
                                                SortLds& sl) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int e = 64 * wave + lane, ec = min(e, E - 1);
  float v = logits[ec];
  const int slot = e2s[ec];                          // issued with the logit load
  if (v != v) v = -INFINITY;                         // NaN logits never win
  uint64_t key = e < E ? ((uint64_t)order_key(v) << 32) |
                             ((uint32_t)(255 - e) << 24) | ((uint32_t)(slot + 1) & 0xFFFFFFu)
                       : 0ull;                       // padding ranks below -inf
  const bool live = 64 * wave < E;
  if (live) bitonic64_desc(key);
  if (lane < FT_MAX_TOPK) sl.key[wave][lane] = live && lane < k ? key : 0ull;
  __syncthreads();
  if (wave == 0) {
    if (E > 64) {
      // runs of R >= k: run q in lanes R q .. R q + R - 1, odd runs reversed, so every pair of
      // runs is a bitonic sequence; the merge network then sorts lanes descending
      if (k <= 8) {
        const int q = lane >> 3, i = lane & 7;
        key = q < 4 ? sl.key[q][(q & 1) ? 7 - i : i] : 0ull;
        bitonic_merge<16>(key);
        bitonic_merge<32>(key);
      } else {
        const int q = lane >> 4, i = lane & 15;
        key = sl.key[q][(q & 1) ? 15 - i : i];
        bitonic_merge<32>(key);
        bitonic_merge<64>(key);
      }
    }
    const float vl = key_value((uint32_t)(key >> 32));
    const float vmax = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(vl)));
    const float p = lane < k ? __expf(vl - vmax) : 0.f;
    // the k <= 16 terms sit in lanes 0..15: a butterfly over the row gives every lane of it
    // the same sum
    float sum = p;
    sum += __uint_as_float(xor_lane<1>(__float_as_uint(sum)));
    sum += __uint_as_float(xor_lane<2>(__float_as_uint(sum)));
    sum += __uint_as_float(xor_lane<4>(__float_as_uint(sum)));
    sum += __uint_as_float(xor_lane<8>(__float_as_uint(sum)));
    const uint32_t lo = (uint32_t)key;
    const int ew = 255 - (int)(lo >> 24);
    if (lane < k) {
      tk.idx[0][lane] = ew;
      tk.w[0][lane] = p / sum;
      L.expert[lane] = ew;
      L.slot[lane] = (int)(lo & 0xFFFFFFu) - 1;
    } else if (lane < k + n_shared) {
      L.expert[lane] = k - 1 - lane;
      L.slot[lane] = k - 1 - lane;
    }
    if (lane < k + n_shared) {
      L.ntok[lane] = 1;
      L.tok[lane][0] = 0;
      L.jj[lane][0] = (uint8_t)lane;
    }
    if (lane == 0) L.n_items = k + n_shared;
  }
  __syncthreads();
}

// Publish the routing (when write_route) and the list for the next kernel (global memory):
// entries n_items .. max_items - 1 get ntok = 0, so a reader may walk max_items entries
// without the count; every column carries its routing weight.
__device__ void store_route(const TopkLds& tk, const ListLds& L, int T, int k, int n_shared,
                            int32_t* idx_out, float* w_out, WorkItem* items, int* n_items,
                            int max_items, bool write_route) {
  const int tid = threadIdx.x, kk = k + n_shared;
  if (write_route && tid < T * k) {
    idx_out[tid] = tk.idx[tid / k][tid % k];
    w_out[tid] = tk.w[tid / k][tid % k];
  }
  for (int i = tid; i < max_items; i += 256) {
    WorkItem& it = items[i];
    const bool used = i < L.n_items;
    it.expert = used ? L.expert[i] : 0;
    it.slot = used ? L.slot[i] : 0;
    it.ntok = used ? L.ntok[i] : 0;
    it.pad = 0;
    for (int n = 0; used && n < L.ntok[i]; ++n) {
      const int t = L.tok[i][n], j = L.jj[i][n];
      it.tok[n] = t;
      it.pair[n] = t * kk + j;
      it.wt[n] = j < k ? tk.w[t][j] : 1.f;
    }
  }
  if (tid == 0) *n_items = L.n_items;
}

// Copy a host-built list (miss path) into LDS.  All threads call; ends synchronised.
__device__ void load_list(const WorkItem* items, const int* n_items, ListLds& L) {
  const int n = min(*n_items, kMaxItems);
  for (int i = threadIdx.x; i < n; i += 256) {
    L.expert[i] = items[i].expert;
    L.slot[i] = items[i].slot;
    L.ntok[i] = items[i].ntok;
    for (int c = 0; c < items[i].ntok && c < kMaxCols; ++c) L.tok[i][c] = (uint8_t)items[i].tok[c];
  }
  if (threadIdx.x == 0) L.n_items = n;
  __syncthreads();
}

// Top-k kernel (batched decode, ft_route and the miss path): one wave per token, four
// tokens per workgroup, idx/w to global.
// With the host pointers set (mapped pinned memory, miss path), the routing and the
// workgroup's token rows are also written straight to host memory, so the host reads them
// after one event wait instead of separate device-to-host copies.
template <int EPL>
__global__ __launch_bounds__(256) void k_topk(const float* logits, int T, int E, int k,
                                              int32_t* idx_out, float* w_out, int32_t* idx_host,
                                              float* w_host, const uint16_t* x, uint16_t* x_host,
                                              int H) {
  __shared__ TopkLds tk;
  __shared__ float c_val[kMaxCols][FT_MAX_TOPK];
  __shared__ int c_idx[kMaxCols][FT_MAX_TOPK];
  const int t0 = blockIdx.x * 4;
  const int nt = min(4, T - t0);
  topk_tokens<EPL>(logits + (uint64_t)t0 * E, nt, E, k, tk, c_val, c_idx);
  const int tid = threadIdx.x;
  if (tid < nt * k) {
    const int32_t e = tk.idx[tid / k][tid % k];
    const float wv = tk.w[tid / k][tid % k];
    idx_out[(uint64_t)t0 * k + tid] = e;
    w_out[(uint64_t)t0 * k + tid] = wv;
    if (idx_host) {
      idx_host[(uint64_t)t0 * k + tid] = e;
      w_host[(uint64_t)t0 * k + tid] = wv;
    }
  }
  if (x_host) {
    const uint32_t* src = (const uint32_t*)(x + (uint64_t)t0 * H);
    uint32_t* dst = (uint32_t*)(x_host + (uint64_t)t0 * H);
    for (int i = tid; i < nt * H / 2; i += 256) dst[i] = src[i];
  }
}

// ---- expert GEMVs -------------------------------------------------------------------------
__device__ __forceinline__ const uint8_t* blob_of(int expert, int slot, const uint8_t* pool,
                                                  const uint8_t* shared, uint64_t stride) {
  return expert >= 0 ? pool + (uint64_t)slot * stride : shared + (uint64_t)(-1 - expert) * stride;
}

// Tensor scale of matrix m (0 gate, 1 up, 2 down) of a blob: the header's field for NVFP4,
// 1 for MXFP4 (whose header holds 1 too, but the read is skipped).
template <int FMT>
__device__ __forceinline__ float tensor_scale(const uint8_t* blob, int m) {
  return FMT == FT_MXFP4 ? 1.f : ((const float*)(blob + offsetof(BlobHeader, tensor_scale)))[m];
}

// acc[m] += W_m[tile rows][chunks ks, ks+kstep, ...] x B for NM matrices sharing the B
// operand (gate and up share x).  Each lane owns 32 K values of one tile row per chunk: one
// 128-bit code load, one scale byte and four MFMA k-steps.  The loads of UNR chunks are all
// issued before any is consumed.  brow: this lane's B column (token row or h row) at K
// offset 32*g; bcol false makes the column zero without loading it.
// Scales: MXFP4 one E8M0 byte per lane per tile; NVFP4 two E4M3 bytes per lane per tile (the
// blocks of the lane's first and second 16 K values).
template <int NM, int UNR, int FMT>
__device__ __forceinline__ void tile_gemv(const uint8_t* const* codes, const uint8_t* const* scales,
                                          uint64_t tile0, int KC, int ks, int kstep,
                                          const uint16_t* brow, bool bcol, int lane, f32x4* acc) {
  const int NC = (KC - ks + kstep - 1) / kstep;
  for (int c0 = 0; c0 < NC; c0 += UNR) {
    uint4 cw[UNR][NM];
    uint32_t sc[UNR][NM];
    uint4 xb[UNR][4];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const bool ok = c0 + u < NC;
      const uint64_t tile = tile0 + (uint64_t)(ks + (c0 + u) * kstep);
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        cw[u][m] = ok ? ((const uint4*)codes[m])[tile * 64 + lane] : make_uint4(0u, 0u, 0u, 0u);
        if (FMT == FT_MXFP4) sc[u][m] = ok ? scales[m][tile * 64 + lane] : 127u;
        else sc[u][m] = ok ? ((const uint16_t*)scales[m])[tile * 64 + lane] : 0x3838u;
      }
    }
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const bool ok = c0 + u < NC && bcol;
      const uint4* xr = (const uint4*)(brow + (uint64_t)(ks + (c0 + u) * kstep) * kTileK);
#pragma unroll
      for (int i = 0; i < 4; ++i) xb[u][i] = ok ? xr[i] : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        const uint32_t wv[4] = {cw[u][m].x, cw[u][m].y, cw[u][m].z, cw[u][m].w};
        if (FMT == FT_MXFP4) {
          const float s = e8m0_f32(sc[u][m]);
#pragma unroll
          for (int i = 0; i < 4; ++i)
            acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fp4x8_bf16(wv[i], s),
                                                             as_bf16x8(xb[u][i]), acc[m], 0, 0, 0);
        } else {
          const float s0 = e4m3_f32_fast(sc[u][m] & 0xffu), s1 = e4m3_f32_fast(sc[u][m] >> 8);
#pragma unroll
          for (int i = 0; i < 4; ++i)
            acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fp4x8_bf16_mul(wv[i], i < 2 ? s0 : s1),
                                                             as_bf16x8(xb[u][i]), acc[m], 0, 0, 0);
        }
      }
    }
  }
}

// Workgroup = 4 waves.  KSPLIT waves share one 16-row tile and split its K chunks; the
// workgroup covers 4 / KSPLIT row tiles.  A unit is (item, group of row tiles); workgroups
// walk the units with a grid stride.
// EPL > 0: the prologue takes the top-k of the logits (E <= 64 * EPL); EPL == 0: the
// work list is read from memory (miss path); EPL < 0: the list is built from the routed
// indices a previous k_topk wrote.  Workgroup 0 publishes the list for k_down.
template <int KSPLIT, int UNR, int EPL, int FMT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void k_gateup(DecodeLaunch a) {
  constexpr int RPW = 4 / KSPLIT;
  __shared__ TopkLds tk;
  __shared__ ListLds ls;
  __shared__ f32x4 red[4][2][64];
  if (EPL > 0) {
    if (a.T == 1 && a.E <= 256) {
      route_one_token(a.logits, a.e2s, a.E, a.k, a.n_shared, tk, ls, *(SortLds*)&red[0][0][0]);
    } else {
      topk_tokens<(EPL > 0 ? EPL : 1)>(a.logits, a.T, a.E, a.k, tk,
                                       (float (*)[FT_MAX_TOPK])&red[0][0][0],
                                       (int (*)[FT_MAX_TOPK])&red[2][0][0]);
      build_list(tk, a.T, a.E, a.k, a.n_shared, a.e2s, ls);
    }
    if (blockIdx.x == 0)
      store_route(tk, ls, a.T, a.k, a.n_shared, a.idx_out, a.w_out, a.items, a.n_items,
                  a.max_items, true);
  } else if (EPL < 0) {
    if (threadIdx.x < a.T * a.k) {
      tk.idx[threadIdx.x / a.k][threadIdx.x % a.k] = a.idx_out[threadIdx.x];
      tk.w[threadIdx.x / a.k][threadIdx.x % a.k] = a.w_out[threadIdx.x];
    }
    __syncthreads();
    build_list(tk, a.T, a.E, a.k, a.n_shared, a.e2s, ls);
    if (blockIdx.x == 0)
      store_route(tk, ls, a.T, a.k, a.n_shared, a.idx_out, a.w_out, a.items, a.n_items,
                  a.max_items, false);
  } else {
    load_list(a.items, a.n_items, ls);
  }
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int rl = wave / KSPLIT, ks = wave % KSPLIT;
  const int n = lane & 15, g = lane >> 4;
  const int RT = a.I / kTileRows, KC = a.H / kTileK;
  const int groups = (RT + RPW - 1) / RPW;
  const int units = ls.n_items * groups;
  for (int u = blockIdx.x; u < units; u += gridDim.x) {
    const int iti = u / groups;
    const int rt = (u % groups) * RPW + rl;
    const int expert = ls.expert[iti], slot = ls.slot[iti], ntok = ls.ntok[iti];
    const bool active = rt < RT && (expert < 0 || slot >= 0);
    f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
    float tsg = 1.f, tsu = 1.f;
    if (active) {
      const uint8_t* blob = blob_of(expert, slot, a.pool, a.shared, a.stride);
      const uint8_t* codes[2] = {blob + a.L.off[0], blob + a.L.off[2]};
      const uint8_t* scales[2] = {blob + a.L.off[1], blob + a.L.off[3]};
      const bool col = n < ntok;
      const uint16_t* brow = a.x + (uint64_t)(col ? ls.tok[iti][n] : 0) * a.H + 32 * g;
      tile_gemv<2, UNR, FMT>(codes, scales, (uint64_t)rt * KC, KC, ks, KSPLIT, brow, col, lane,
                             acc);
      tsg = tensor_scale<FMT>(blob, 0);
      tsu = tensor_scale<FMT>(blob, 1);
    }
    if (KSPLIT > 1) {
      red[wave][0][lane] = acc[0];
      red[wave][1][lane] = acc[1];
      __syncthreads();
      if (ks == 0) {
#pragma unroll
        for (int s2 = 1; s2 < KSPLIT; ++s2) {
          acc[0] += red[wave + s2][0][lane];
          acc[1] += red[wave + s2][1][lane];
        }
      }
    }
    if (ks == 0 && active && n < ntok) {
      uint16_t hv[4];
#pragma unroll
      for (int r = 0; r < 4; ++r)
        hv[r] = f32_to_bf16_rne(silu_f32(tsg * acc[0][r]) * (tsu * acc[1][r]));
      const uint2 pk = make_uint2((uint32_t)hv[0] | ((uint32_t)hv[1] << 16),
                                  (uint32_t)hv[2] | ((uint32_t)hv[3] << 16));
      *(uint2*)(a.h + ((uint64_t)iti * kMaxCols + n) * a.I + rt * kTileRows + 4 * g) = pk;
    }
    if (KSPLIT > 1) __syncthreads();
  }
}

template <int KSPLIT, int UNR, int FMT>
__global__ __launch_bounds__(256) void k_down(DecodeLaunch a) {
  constexpr int RPW = 4 / KSPLIT;
  __shared__ f32x4 red[4][64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int rl = wave / KSPLIT, ks = wave % KSPLIT;
  const int n = lane & 15, g = lane >> 4;
  const int RT = a.H / kTileRows, KC = a.I / kTileK;
  const int groups = (RT + RPW - 1) / RPW;
  const int units = (*a.n_items) * groups;
  for (int u = blockIdx.x; u < units; u += gridDim.x) {
    const int iti = u / groups;
    const int rt = (u % groups) * RPW + rl;
    const WorkItem& it = a.items[iti];
    const bool active = rt < RT && (it.expert < 0 || it.slot >= 0);
    const int ntok = it.ntok;
    f32x4 acc[1] = {{0.f, 0.f, 0.f, 0.f}};
    float tsd = 1.f;
    if (active) {
      const uint8_t* blob = blob_of(it.expert, it.slot, a.pool, a.shared, a.stride);
      const uint8_t* codes[1] = {blob + a.L.off[4]};
      const uint8_t* scales[1] = {blob + a.L.off[5]};
      const bool col = n < ntok;
      const uint16_t* brow = a.h + ((uint64_t)iti * kMaxCols + n) * a.I + 32 * g;
      tile_gemv<1, UNR, FMT>(codes, scales, (uint64_t)rt * KC, KC, ks, KSPLIT, brow, col, lane,
                             acc);
      tsd = tensor_scale<FMT>(blob, 2);
    }
    if (KSPLIT > 1) {
      red[wave][lane] = acc[0];
      __syncthreads();
      if (ks == 0) {
#pragma unroll
        for (int s2 = 1; s2 < KSPLIT; ++s2) acc[0] += red[wave + s2][lane];
      }
    }
    if (ks == 0 && active && n < ntok) {
      float* dst = a.P + (uint64_t)it.pair[n] * a.H + rt * kTileRows + 4 * g;
      *(float4*)dst = make_float4(tsd * acc[0][0], tsd * acc[0][1], tsd * acc[0][2],
                                  tsd * acc[0][3]);
    }
    if (KSPLIT > 1) __syncthreads();
  }
}

// Down projection and weighted combine in one pass, for calls whose experts all run on the
// GPU.  A workgroup owns one 16-row tile of y for every token; wave w walks items w, w + NW,
// ... (all K chunks of an item, loads issued UNR chunks at a time) and folds each item's
// columns into its own per-token partial in LDS with the routing weight (weight 1 for shared
// experts); the waves' partials are then summed in wave order.  Every sum has a fixed order,
// so the result does not depend on timing.
template <int NW, int UNR, int FMT>
__global__ __launch_bounds__(64 * NW) void k_down_combine(DecodeLaunch a) {
  __shared__ float part[NW][kMaxCols][kTileRows];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n = lane & 15, g = lane >> 4;
  const int RT = a.H / kTileRows, KC = a.I / kTileK;
  // the list's entries past its count have ntok = 0: walking all max_items entries spares
  // every workgroup a dependent read of the count before its first item
  const int n_entries = min(a.max_items, kMaxItems);
  for (int rt = blockIdx.x; rt < RT; rt += gridDim.x) {
    for (int i = lane; i < a.T * kTileRows; i += 64) part[wave][i / kTileRows][i % kTileRows] = 0.f;
    __builtin_amdgcn_wave_barrier();
    for (int iti = wave; iti < n_entries; iti += NW) {
      const WorkItem& it = a.items[iti];
      const int ntok = it.ntok;
      const bool col = n < ntok;
      const int t = it.tok[n];
      const float wt = it.wt[n];
      if (ntok == 0) continue;
      const uint8_t* blob = blob_of(it.expert, it.slot, a.pool, a.shared, a.stride);
      const uint8_t* codes[1] = {blob + a.L.off[4]};
      const uint8_t* scales[1] = {blob + a.L.off[5]};
      const uint16_t* brow = a.h + ((uint64_t)iti * kMaxCols + n) * a.I + 32 * g;
      f32x4 acc[1] = {{0.f, 0.f, 0.f, 0.f}};
      tile_gemv<1, UNR, FMT>(codes, scales, (uint64_t)rt * KC, KC, 0, 1, brow, col, lane, acc);
      const float tsd = tensor_scale<FMT>(blob, 2);
      if (col) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          part[wave][t][4 * g + r] = fmaf(wt, tsd * acc[0][r], part[wave][t][4 * g + r]);
      }
    }
    __syncthreads();
    for (int i = threadIdx.x; i < a.T * kTileRows; i += 64 * NW) {
      const int t = i / kTileRows, r = i % kTileRows;
      float s = part[0][t][r];
#pragma unroll
      for (int w2 = 1; w2 < NW; ++w2) s += part[w2][t][r];
      a.y[(uint64_t)t * a.H + rt * kTileRows + r] = s;
    }
    __syncthreads();
  }
}

// y[t][r] = sum_{j<k} w[t][j] P[t*kk + j][r] + sum_s P[t*kk + k + s][r]; all loads of an
// output are issued together.
__global__ __launch_bounds__(256) void k_combine(const float* __restrict__ P,
                                                 const float* __restrict__ w, int T, int H,
                                                 int k, int n_shared, float* __restrict__ y) {
  constexpr int MAXKK = FT_MAX_TOPK + 4;
  const int t = blockIdx.y;
  const int r = blockIdx.x * 256 + threadIdx.x;
  if (r >= H || t >= T) return;
  const int kk = k + n_shared;
  const float* p = P + (uint64_t)t * kk * H + r;
  float v[MAXKK];
#pragma unroll
  for (int j = 0; j < MAXKK; ++j) v[j] = j < kk ? p[(uint64_t)j * H] : 0.f;
  float acc = 0.f;
#pragma unroll
  for (int j = 0; j < FT_MAX_TOPK; ++j)
    if (j < k) acc = fmaf(w[t * k + j], v[j], acc);
#pragma unroll
  for (int j = 0; j < MAXKK; ++j)
    if (j >= k && j < kk) acc += v[j];
  y[(uint64_t)t * H + r] = acc;
}

}  // namespace ft

// ---- launchers (C linkage, called by the host runtime) -----------------------------------
using namespace ft;

static int grid_for(int units_max, int cap) {
  const int g = units_max < cap ? units_max : cap;
  return g < 1 ? 1 : g;
}

// Workgroups of a kernel that the device holds at once (256 threads each), cached per kernel
// and device.  Grid-stride kernels whose workgroups start with fixed work (the routing
// prologue) launch no more than this, so no workgroup waits for another to finish before it
// can start and each pays the prologue once.
static int resident_workgroups(const void* kern) {
  static std::mutex mu;
  static std::map<std::pair<const void*, int>, int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 2048;
  std::lock_guard<std::mutex> g(mu);
  const auto key = std::make_pair(kern, dev);
  auto it = cache.find(key);
  if (it != cache.end()) return it->second;
  int per_cu = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, 256, 0) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      per_cu < 1 || cus < 1)
    return 2048;
  return cache[key] = per_cu * cus;
}

// Routing of a miss-path call in one launch: one workgroup per router row (the layer's own
// router, then optionally a second one: the linked next layer's, whose routing of the same
// tokens is the prefetch prediction); the last workgroup to finish (device-scope counter,
// reset by that workgroup; agent-scope release by every workgroup before it counts itself in,
// acquire by the last) takes the top-k of every token for each router, writes it to device
// and host memory with the token rows, and then sets a host-memory flag to the call's
// sequence number, which the host polls.  This is the one kernel where workgroups hand data
// to each other: one release per workgroup, no waiting.
template <int TB, int EPL>
__global__ __launch_bounds__(256) void k_route_small(RouteSmall a) {
  const int g = blockIdx.x, tid = threadIdx.x;
  const int r = g < a.E[0] ? 0 : 1;
  logit_row<TB>(a.x, a.wr[r], a.b[r], a.T, a.H, a.E[r], r ? g - a.E[0] : g, a.logits[r]);
  // release this workgroup's logits, count it in; the last one in acquires everyone's
  __shared__ int last;
  __syncthreads();
  if (tid == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    last = atomicAdd(a.counter, 1u) == gridDim.x - 1;
    if (last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  }
  __syncthreads();
  if (!last) return;
  __shared__ TopkLds tk;
  __shared__ float c_val[kMaxCols][FT_MAX_TOPK];
  __shared__ int c_idx[kMaxCols][FT_MAX_TOPK];
  for (int rr = 0; rr < a.n_routers; ++rr) {
    const int k = a.k[rr];
    topk_tokens<EPL>(a.logits[rr], a.T, a.E[rr], k, tk, c_val, c_idx);
    if (tid < a.T * k) {
      const int32_t e = tk.idx[tid / k][tid % k];
      const float wv = tk.w[tid / k][tid % k];
      a.idx[rr][tid] = e;
      a.w[rr][tid] = wv;
      a.idx_host[rr][tid] = e;
      a.w_host[rr][tid] = wv;
    }
    __syncthreads();
  }
  if (a.x_host) {
    if ((uintptr_t)a.x % 16 == 0) {
      const uint4* src = (const uint4*)a.x;
      uint4* dst = (uint4*)a.x_host;
      for (int i = tid; i < a.T * a.H / 8; i += 256) dst[i] = src[i];
    } else {
      for (int i = tid; i < a.T * a.H; i += 256) a.x_host[i] = a.x[i];
    }
  }
  // everything above is in host memory before the flag: each wave's stores complete (system
  // release), then one release store of the call's sequence number
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "");
  __syncthreads();
  if (tid == 0) {
    atomicExch(a.counter, 0u);
    __hip_atomic_store(a.flag_host, a.seq, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
  }
}

extern "C" int ftk_route_small(const RouteSmall* ap, hipStream_t st) {
  const RouteSmall& a = *ap;
  const int Emax = a.n_routers > 1 ? max(a.E[0], a.E[1]) : a.E[0];
  const dim3 grid(a.E[0] + (a.n_routers > 1 ? a.E[1] : 0));
#define FT_RS(TBV, EPLV) hipLaunchKernelGGL((k_route_small<TBV, EPLV>), grid, dim3(256), 0, st, a)
#define FT_RS_T(EPLV)                 \
  if (a.T <= 1) FT_RS(1, EPLV);       \
  else if (a.T <= 2) FT_RS(2, EPLV);  \
  else if (a.T <= 4) FT_RS(4, EPLV);  \
  else if (a.T <= 8) FT_RS(8, EPLV);  \
  else FT_RS(16, EPLV)
  if (Emax <= 64) { FT_RS_T(1); }
  else if (Emax <= 128) { FT_RS_T(2); }
  else if (Emax <= 256) { FT_RS_T(4); }
  else { FT_RS_T(16); }
#undef FT_RS_T
#undef FT_RS
  return (int)hipGetLastError();
}

extern "C" int ftk_logits(const uint16_t* x, const float* wr, const float* b, int T, int H, int E,
                          float* logits, hipStream_t st) {
  if (T <= 1)
    hipLaunchKernelGGL(k_logits<1>, dim3(E), dim3(256), 0, st, x, wr, b, T, H, E, logits);
  else if (T <= 2)
    hipLaunchKernelGGL(k_logits<2>, dim3(E), dim3(256), 0, st, x, wr, b, T, H, E, logits);
  else if (T <= 4)
    hipLaunchKernelGGL(k_logits<4>, dim3(E), dim3(256), 0, st, x, wr, b, T, H, E, logits);
  else if (T <= 8)
    hipLaunchKernelGGL(k_logits<8>, dim3(E), dim3(256), 0, st, x, wr, b, T, H, E, logits);
  else
    hipLaunchKernelGGL(k_logits<16>, dim3(E), dim3(256), 0, st, x, wr, b, T, H, E, logits);
  return (int)hipGetLastError();
}

extern "C" int ftk_topk(const float* logits, int T, int E, int k, int32_t* idx_out, float* w_out,
                        int32_t* idx_host, float* w_host, const uint16_t* x, uint16_t* x_host,
                        int H, hipStream_t st) {
  const dim3 grid((T + 3) / 4);
#define FT_TOPK(EPLV)                                                                     \
  hipLaunchKernelGGL(k_topk<EPLV>, grid, dim3(256), 0, st, logits, T, E, k, idx_out, w_out, \
                     idx_host, w_host, x, x_host, H)
  if (E <= 64) FT_TOPK(1);
  else if (E <= 128) FT_TOPK(2);
  else if (E <= 256) FT_TOPK(4);
  else FT_TOPK(16);
#undef FT_TOPK
  return (int)hipGetLastError();
}

// ev: null, or 4 events [gate/up start, stop, down start, stop] that the dispatches record
// themselves (hipExtLaunchKernelGGL), so host-side gaps are not counted.
#define FT_LAUNCH_NT(kern, grid, nt, evs, eve, arg)                                         \
  do {                                                                                      \
    auto* kfn_ = kern;                                                                      \
    if (evs) hipExtLaunchKernelGGL(kfn_, grid, dim3(nt), 0, st, evs, eve, 0, arg);          \
    else hipLaunchKernelGGL(kfn_, grid, dim3(nt), 0, st, arg);                              \
  } while (0)
#define FT_LAUNCH(kern, grid, evs, eve, arg) FT_LAUNCH_NT(kern, grid, 256, evs, eve, arg)

// Whether the down kernel also combines into y: for calls whose experts all run on the GPU,
// when the one-workgroup-per-row-tile grid covers the chip or the list is short (latency
// bound); otherwise down writes per-(token, choice) partials for k_combine.
extern "C" int ftk_down_combines(const DecodeLaunch* ap) {
  const DecodeLaunch& a = *ap;
  return a.fuse_combine || (a.route != 0 && (a.max_items <= 16 || a.H / kTileRows >= 256));
}

// EPL = 0: work list read from memory; EPL > 0: routing prologue for E <= 64 * EPL experts;
// EPL < 0: list built from routed indices
template <int EPL, int FMT>
static void launch_gateup(const DecodeLaunch& a, hipStream_t st, hipEvent_t e0, hipEvent_t e1) {
  const int KC = a.H / kTileK, RT = a.I / kTileRows;
#define FT_GATEUP(KS_, RPW_)                                                                \
  do {                                                                                      \
    auto* k_ = k_gateup<KS_, 2, EPL, FMT>;                                                  \
    const int cap_ = resident_workgroups((const void*)k_);                                  \
    FT_LAUNCH(k_, dim3(grid_for(a.max_items * ((RT + (RPW_) - 1) / (RPW_)), cap_)), e0, e1, a); \
  } while (0)
  if (KC >= 16) FT_GATEUP(4, 1);
  else if (KC >= 8) FT_GATEUP(2, 2);
  else FT_GATEUP(1, 4);
#undef FT_GATEUP
}

template <int FMT>
static void launch_experts(const DecodeLaunch& a, hipStream_t st, const hipEvent_t* ev) {
  hipEvent_t e0 = ev ? ev[0] : nullptr, e1 = ev ? ev[1] : nullptr;
  hipEvent_t e2 = ev ? ev[2] : nullptr, e3 = ev ? ev[3] : nullptr;
  if (a.route == 0) launch_gateup<0, FMT>(a, st, e0, e1);
  else if (a.route == 2) launch_gateup<-1, FMT>(a, st, e0, e1);
  else if (a.E <= 64) launch_gateup<1, FMT>(a, st, e0, e1);
  else if (a.E <= 128) launch_gateup<2, FMT>(a, st, e0, e1);
  else if (a.E <= 256) launch_gateup<4, FMT>(a, st, e0, e1);
  else launch_gateup<16, FMT>(a, st, e0, e1);
  const int KC = a.I / kTileK, RT = a.H / kTileRows;
  if (ftk_down_combines(&a)) {
    // down and combine in one kernel, one workgroup per row tile
    const dim3 grid(RT);
    if (a.max_items <= 16) {
      if (KC >= 8) FT_LAUNCH_NT((k_down_combine<8, 8, FMT>), grid, 512, e2, e3, a);
      else FT_LAUNCH_NT((k_down_combine<8, 4, FMT>), grid, 512, e2, e3, a);
    } else {
      FT_LAUNCH_NT((k_down_combine<16, 4, FMT>), grid, 1024, e2, e3, a);
    }
  } else if (KC >= 8) {
    auto* k = k_down<2, 4, FMT>;
    FT_LAUNCH(k, dim3(grid_for(a.max_items * ((RT + 1) / 2), resident_workgroups((const void*)k))),
              e2, e3, a);
  } else {
    auto* k = k_down<1, 4, FMT>;
    FT_LAUNCH(k, dim3(grid_for(a.max_items * ((RT + 3) / 4), resident_workgroups((const void*)k))),
              e2, e3, a);
  }
}

extern "C" int ftk_decode_experts(const DecodeLaunch* ap, hipStream_t st, const hipEvent_t* ev) {
  if (ap->L.fmt == FT_MXFP4) launch_experts<FT_MXFP4>(*ap, st, ev);
  else launch_experts<FT_NVFP4>(*ap, st, ev);
  return (int)hipGetLastError();
}

// out = bf16(float(x) + s*y): the product and the sum each rounded to fp32 (no fused
// multiply-add), then rounded to nearest even bf16, a NaN kept quiet.  Eight
// elements per thread per round (16-byte bf16 and 2 x 16-byte fp32 accesses when vec, which
// the host sets for 16-byte aligned arrays), grid-stride; out may alias x.
__device__ __forceinline__ uint16_t bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

__global__ __launch_bounds__(256) void k_residual(const uint16_t* x, const float* y, float sc,
                                                  int64_t n, uint16_t* out, int vec) {
  const int64_t stride = (int64_t)gridDim.x * 256 * 8;
  for (int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8; i < n; i += stride) {
    if (vec && i + 8 <= n) {
      const uint4 xv = *(const uint4*)(x + i);
      const float4 y0 = *(const float4*)(y + i), y1 = *(const float4*)(y + i + 4);
      const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
      const float yv[8] = {y0.x, y0.y, y0.z, y0.w, y1.x, y1.y, y1.z, y1.w};
      uint32_t o[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float lo = __fadd_rn(__uint_as_float(xw[q] << 16), __fmul_rn(sc, yv[2 * q]));
        const float hi = __fadd_rn(__uint_as_float(xw[q] & 0xffff0000u), __fmul_rn(sc, yv[2 * q + 1]));
        o[q] = (uint32_t)bf16_rne(lo) | ((uint32_t)bf16_rne(hi) << 16);
      }
      *(uint4*)(out + i) = make_uint4(o[0], o[1], o[2], o[3]);
    } else {
      for (int64_t j = i; j < n && j < i + 8; ++j)
        out[j] = bf16_rne(__fadd_rn(__uint_as_float((uint32_t)x[j] << 16), __fmul_rn(sc, y[j])));
    }
  }
}

extern "C" int ftk_residual(const uint16_t* x, const float* y, float sc, int64_t n, uint16_t* out,
                            hipStream_t st) {
  if (n <= 0) return 0;
  const int vec = ((uintptr_t)x % 16 == 0 && (uintptr_t)y % 16 == 0 && (uintptr_t)out % 16 == 0);
  const int64_t want = (n + 2047) / 2048;
  const int grid = (int)(want < 2048 ? want : 2048);
  hipLaunchKernelGGL(k_residual, dim3(grid), dim3(256), 0, st, x, y, sc, n, out, vec);
  return (int)hipGetLastError();
}

extern "C" int ftk_combine(const float* P, const float* w, int T, int H, int k, int n_shared,
                           float* y, hipStream_t st) {
  hipLaunchKernelGGL(k_combine, dim3((H + 255) / 256, T), dim3(256), 0, st, P, w, T, H, k,
                     n_shared, y);
  return (int)hipGetLastError();
}
