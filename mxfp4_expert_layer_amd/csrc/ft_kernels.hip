// HIP kernels of libft for gfx950 (CDNA4): decode routing, FP4 GEMVs on MFMA, combine.
//
// Decode path for one call of T <= 16 tokens (the MoE layer of the FreeToken pages: a gate
// picks k experts per token and their outputs are merged by routing weight — smzdm
// explainer a825qpgl, section 二):
//   k_route_decode   logits = x W_r^T + b (fp32 FMA), then the last workgroup to finish
//                    (atomic ticket) runs top-k + softmax per token and builds the work
//                    list: one item per distinct expert with its token columns.
//   k_gateup         per item and 16-row tile: g = W_g x, u = W_u x on the 16x16x32 bf16
//                    MFMA (FP4 codes converted to bf16 in registers, exact), then
//                    h = bf16(silu(g) * u).  Tokens are the MFMA's N columns.
//   k_down           per item and 16-row tile of W_d: y_e = W_d h into the per-(token,
//                    choice) partial buffer P.
//   k_combine        y_t = sum_j w_tj P[t][j] + sum_s P[t][k + s].
// Weights are read once per call however many tokens share an expert; every kernel loops
// over its work units with a grid stride, so the launch size is fixed and no workgroup
// waits on another.
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>

#include "ft_internal.h"

namespace ft {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// ---- FP4 decode --------------------------------------------------------------------------
// E8M0 code -> fp32 scale 2^(e - 127): e = 0 is 2^-127 (an fp32 subnormal), e = 255 NaN.
__device__ __forceinline__ float e8m0_f32(uint32_t e) {
  uint32_t bits = (e == 0u) ? 0x00400000u : ((e == 255u) ? 0x7fc00000u : (e << 23));
  return __uint_as_float(bits);
}

// Eight E2M1 codes (one dword, element 0 in the low nibble) times a power-of-two scale ->
// eight bf16 (exact: an E2M1 value has at most 2 significant bits).
__device__ __forceinline__ bf16x8 fp4x8_bf16(uint32_t w, float scale) {
  bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 0);
  bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 1);
  bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 2);
  bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 3);
  auto lo = __builtin_shufflevector(p0, p1, 0, 1, 2, 3);
  auto hi = __builtin_shufflevector(p2, p3, 0, 1, 2, 3);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) {
  return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t b = __float_as_uint(f);
  if ((b & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;  // NaN
  b += 0x7fffu + ((b >> 16) & 1u);
  return (uint16_t)(b >> 16);
}

__device__ __forceinline__ float silu_f32(float z) { return z / (1.0f + expf(-z)); }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ const uint8_t* item_blob(const WorkItem& it, const uint8_t* pool,
                                                    const uint8_t* shared, uint64_t stride) {
  return it.expert >= 0 ? pool + (uint64_t)it.slot * stride
                        : shared + (uint64_t)(-1 - it.expert) * stride;
}

// ---- routing -----------------------------------------------------------------------------
// Grid: ceil(E / 4) workgroups of 4 waves; wave w computes the logits of expert 4*b + w for
// all T tokens.  The last workgroup to finish does the per-token top-k (one wave per token,
// k rounds of a wave-wide argmax with ties to the lower index) and the work list.
constexpr int kRouteMaxEPerLane = 16;  // E <= 1024

struct RouteArgs {
  const uint16_t* x; const float* wr; const float* b;
  int T, H, E, k, n_shared;
  float* logits; int* ticket;
  int32_t* idx_out; float* w_out;      // [T][k]
  const int32_t* e2s;
  WorkItem* items; int* n_items;       // may be null (routing only)
};

__global__ __launch_bounds__(256) void k_route_decode(RouteArgs a) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int e = blockIdx.x * 4 + wave;
  if (e < a.E) {
    float acc[kMaxCols];
#pragma unroll
    for (int t = 0; t < kMaxCols; ++t) acc[t] = 0.f;
    const float* wrow = a.wr + (uint64_t)e * a.H;
    for (int h0 = lane * 4; h0 < a.H; h0 += 256) {
      float4 wv = *(const float4*)(wrow + h0);
#pragma unroll
      for (int t = 0; t < kMaxCols; ++t) {
        if (t < a.T) {
          uint2 xv = *(const uint2*)(a.x + (uint64_t)t * a.H + h0);
          acc[t] = fmaf(wv.x, __uint_as_float(xv.x << 16), acc[t]);
          acc[t] = fmaf(wv.y, __uint_as_float(xv.x & 0xffff0000u), acc[t]);
          acc[t] = fmaf(wv.z, __uint_as_float(xv.y << 16), acc[t]);
          acc[t] = fmaf(wv.w, __uint_as_float(xv.y & 0xffff0000u), acc[t]);
        }
      }
    }
    const float bias = a.b ? a.b[e] : 0.f;
#pragma unroll
    for (int t = 0; t < kMaxCols; ++t) {
      if (t < a.T) {
        float s = wave_sum(acc[t]);
        if (lane == 0) a.logits[(uint64_t)t * a.E + e] = s + bias;
      }
    }
  }
  // last-arriving workgroup finishes the call
  __shared__ int s_last;
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    int prev = atomicAdd(a.ticket, 1);
    s_last = (prev == (int)gridDim.x - 1);
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  if (threadIdx.x == 0) *a.ticket = 0;  // re-armed for the next launch

  __shared__ int s_idx[kMaxCols][FT_MAX_TOPK];
  __shared__ float s_w[kMaxCols][FT_MAX_TOPK];
  const volatile float* lg = a.logits;
  for (int t = wave; t < a.T; t += 4) {
    float v[kRouteMaxEPerLane];
#pragma unroll
    for (int i = 0; i < kRouteMaxEPerLane; ++i) {
      const int ee = lane + 64 * i;
      v[i] = (ee < a.E) ? lg[(uint64_t)t * a.E + ee] : -INFINITY;
      if (v[i] != v[i]) v[i] = -INFINITY;  // NaN logits never win
    }
    float sel_v[FT_MAX_TOPK];
    int sel_i[FT_MAX_TOPK];
    uint32_t taken = 0;
    for (int j = 0; j < a.k; ++j) {
      float bv = -INFINITY; int bi = 0x7fffffff;
#pragma unroll
      for (int i = 0; i < kRouteMaxEPerLane; ++i) {
        const int ee = lane + 64 * i;
        if (ee < a.E && !((taken >> i) & 1u) && (v[i] > bv || (v[i] == bv && ee < bi))) {
          bv = v[i]; bi = ee;
        }
      }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        float ov = __shfl_xor(bv, o, 64);
        int oi = __shfl_xor(bi, o, 64);
        if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
      }
      sel_v[j] = bv; sel_i[j] = bi;
      if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
    }
    // softmax over the kept logits (rank 0 is the maximum)
    float sum = 0.f;
    for (int j = 0; j < a.k; ++j) sum += expf(sel_v[j] - sel_v[0]);
    if (lane == 0) {
      for (int j = 0; j < a.k; ++j) {
        const float wj = expf(sel_v[j] - sel_v[0]) / sum;
        a.idx_out[t * a.k + j] = sel_i[j];
        a.w_out[t * a.k + j] = wj;
        s_idx[t][j] = sel_i[j];
        s_w[t][j] = wj;
      }
    }
  }
  if (!a.items) return;
  __syncthreads();

  // work list: distinct experts in ascending id, tokens ascending within an expert
  const int kk = a.k + a.n_shared;
  __shared__ int s_wave_tot[4];
  int cnt[4] = {0, 0, 0, 0};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int ee = threadIdx.x * 4 + i;
    if (ee < a.E)
      for (int t = 0; t < a.T; ++t)
        for (int j = 0; j < a.k; ++j) cnt[i] += (s_idx[t][j] == ee);
  }
  const int mine = (cnt[0] > 0) + (cnt[1] > 0) + (cnt[2] > 0) + (cnt[3] > 0);
  int incl = mine;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int n = __shfl_up(incl, o, 64);
    if (lane >= o) incl += n;
  }
  if (lane == 63) s_wave_tot[wave] = incl;
  __syncthreads();
  int base = incl - mine;
  for (int w2 = 0; w2 < wave; ++w2) base += s_wave_tot[w2];
  const int n_routed = s_wave_tot[0] + s_wave_tot[1] + s_wave_tot[2] + s_wave_tot[3];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int ee = threadIdx.x * 4 + i;
    if (ee < a.E && cnt[i] > 0) {
      WorkItem& it = a.items[base];
      it.expert = ee;
      it.slot = a.e2s[ee];
      int n = 0;
      for (int t = 0; t < a.T; ++t)
        for (int j = 0; j < a.k; ++j)
          if (s_idx[t][j] == ee) { it.tok[n] = t; it.pair[n] = t * kk + j; ++n; }
      it.ntok = n;
      ++base;
    }
  }
  if (threadIdx.x < a.n_shared) {
    const int s = threadIdx.x;
    WorkItem& it = a.items[n_routed + s];
    it.expert = -1 - s;
    it.slot = -1 - s;
    it.ntok = a.T;
    for (int t = 0; t < a.T; ++t) { it.tok[t] = t; it.pair[t] = t * kk + a.k + s; }
  }
  if (threadIdx.x == 0) *a.n_items = n_routed + a.n_shared;
}

// ---- gate/up GEMV + SwiGLU ---------------------------------------------------------------
// Workgroup = 4 waves.  KSPLIT waves share one 16-row tile and split its K chunks (strided);
// the workgroup covers 4 / KSPLIT row tiles.  A unit is (item, group of row tiles).
struct FfnArgs {
  const uint16_t* x;            // gate/up: tokens [T][H]; down: h buffer [items][16][I]
  int H, I;
  const WorkItem* items; const int* n_items;
  const uint8_t* pool; const uint8_t* shared; uint64_t stride;
  BlobLayout L;
  uint16_t* h;                  // gate/up output [items][16][I]
  float* P;                     // down output [T * kk][H]
};

template <int KSPLIT>
__global__ __launch_bounds__(256) void k_gateup(FfnArgs a) {
  constexpr int RPW = 4 / KSPLIT;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int rl = wave / KSPLIT, ks = wave % KSPLIT;
  const int n = lane & 15, g = lane >> 4;
  const int RT = a.I / kTileRows, KC = a.H / kTileK;
  const int groups = (RT + RPW - 1) / RPW;
  const int units = (*a.n_items) * groups;
  __shared__ f32x4 red[4][2][64];
  for (int u = blockIdx.x; u < units; u += gridDim.x) {
    const int iti = u / groups;
    const int rt = (u % groups) * RPW + rl;
    const WorkItem& it = a.items[iti];
    const bool active = rt < RT && (it.expert < 0 || it.slot >= 0);
    const int ntok = it.ntok;
    f32x4 ag = {0.f, 0.f, 0.f, 0.f}, au = {0.f, 0.f, 0.f, 0.f};
    if (active) {
      const uint8_t* blob = item_blob(it, a.pool, a.shared, a.stride);
      const uint64_t tile0 = (uint64_t)rt * KC;
      const uint4* gc = (const uint4*)(blob + a.L.off[0]) + tile0 * 64 + lane;
      const uint8_t* gs = blob + a.L.off[1] + tile0 * 64 + lane;
      const uint4* uc = (const uint4*)(blob + a.L.off[2]) + tile0 * 64 + lane;
      const uint8_t* us = blob + a.L.off[3] + tile0 * 64 + lane;
      const int tok = (n < ntok) ? it.tok[n] : -1;
      const uint4* xr = (const uint4*)(a.x + (uint64_t)(tok < 0 ? 0 : tok) * a.H + 32 * g);
      int kc = ks;
      for (; kc + KSPLIT < KC; kc += 2 * KSPLIT) {
        const int k2 = kc + KSPLIT;
        uint4 cg0 = gc[(uint64_t)kc * 64], cu0 = uc[(uint64_t)kc * 64];
        uint4 cg1 = gc[(uint64_t)k2 * 64], cu1 = uc[(uint64_t)k2 * 64];
        float sg0 = e8m0_f32(gs[(uint64_t)kc * 64]), su0 = e8m0_f32(us[(uint64_t)kc * 64]);
        float sg1 = e8m0_f32(gs[(uint64_t)k2 * 64]), su1 = e8m0_f32(us[(uint64_t)k2 * 64]);
        uint4 xb0[4], xb1[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          xb0[i] = tok >= 0 ? xr[kc * 16 + i] : make_uint4(0, 0, 0, 0);
          xb1[i] = tok >= 0 ? xr[k2 * 16 + i] : make_uint4(0, 0, 0, 0);
        }
        const uint32_t wg0[4] = {cg0.x, cg0.y, cg0.z, cg0.w}, wu0[4] = {cu0.x, cu0.y, cu0.z, cu0.w};
        const uint32_t wg1[4] = {cg1.x, cg1.y, cg1.z, cg1.w}, wu1[4] = {cu1.x, cu1.y, cu1.z, cu1.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          ag = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fp4x8_bf16(wg0[i], sg0), as_bf16x8(xb0[i]), ag, 0, 0, 0);
          au = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fp4x8_bf16(wu0[i], su0), as_bf16x8(xb0[i]), au, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          ag = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fp4x8_bf16(wg1[i], sg1), as_bf16x8(xb1[i]), ag, 0, 0, 0);
          au = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fp4x8_bf16(wu1[i], su1), as_bf16x8(xb1[i]), au, 0, 0, 0);
        }
      }
      for (; kc < KC; kc += KSPLIT) {
        uint4 cg0 = gc[(uint64_t)kc * 64], cu0 = uc[(uint64_t)kc * 64];
        float sg0 = e8m0_f32(gs[(uint64_t)kc * 64]), su0 = e8m0_f32(us[(uint64_t)kc * 64]);
        uint4 xb0[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) xb0[i] = tok >= 0 ? xr[kc * 16 + i] : make_uint4(0, 0, 0, 0);
        const uint32_t wg0[4] = {cg0.x, cg0.y, cg0.z, cg0.w}, wu0[4] = {cu0.x, cu0.y, cu0.z, cu0.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          ag = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fp4x8_bf16(wg0[i], sg0), as_bf16x8(xb0[i]), ag, 0, 0, 0);
          au = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fp4x8_bf16(wu0[i], su0), as_bf16x8(xb0[i]), au, 0, 0, 0);
        }
      }
    }
    if (KSPLIT > 1) {
      red[wave][0][lane] = ag;
      red[wave][1][lane] = au;
      __syncthreads();
      if (ks == 0) {
#pragma unroll
        for (int s = 1; s < KSPLIT; ++s) {
          ag += red[wave + s][0][lane];
          au += red[wave + s][1][lane];
        }
      }
    }
    if (ks == 0 && active && n < ntok) {
      uint16_t hv[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) hv[r] = f32_to_bf16_rne(silu_f32(ag[r]) * au[r]);
      uint2 pk = make_uint2((uint32_t)hv[0] | ((uint32_t)hv[1] << 16),
                            (uint32_t)hv[2] | ((uint32_t)hv[3] << 16));
      *(uint2*)(a.h + ((uint64_t)iti * kMaxCols + n) * a.I + rt * kTileRows + 4 * g) = pk;
    }
    if (KSPLIT > 1) __syncthreads();
  }
}

// ---- down GEMV ---------------------------------------------------------------------------
template <int KSPLIT>
__global__ __launch_bounds__(256) void k_down(FfnArgs a) {
  constexpr int RPW = 4 / KSPLIT;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int rl = wave / KSPLIT, ks = wave % KSPLIT;
  const int n = lane & 15, g = lane >> 4;
  const int RT = a.H / kTileRows, KC = a.I / kTileK;
  const int groups = (RT + RPW - 1) / RPW;
  const int units = (*a.n_items) * groups;
  __shared__ f32x4 red[4][64];
  for (int u = blockIdx.x; u < units; u += gridDim.x) {
    const int iti = u / groups;
    const int rt = (u % groups) * RPW + rl;
    const WorkItem& it = a.items[iti];
    const bool active = rt < RT && (it.expert < 0 || it.slot >= 0);
    const int ntok = it.ntok;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if (active) {
      const uint8_t* blob = item_blob(it, a.pool, a.shared, a.stride);
      const uint64_t tile0 = (uint64_t)rt * KC;
      const uint4* dc = (const uint4*)(blob + a.L.off[4]) + tile0 * 64 + lane;
      const uint8_t* ds = blob + a.L.off[5] + tile0 * 64 + lane;
      const bool col = n < ntok;
      const uint4* hr = (const uint4*)(a.x + ((uint64_t)iti * kMaxCols + n) * a.I + 32 * g);
      int kc = ks;
      for (; kc + KSPLIT < KC; kc += 2 * KSPLIT) {
        const int k2 = kc + KSPLIT;
        uint4 c0 = dc[(uint64_t)kc * 64], c1 = dc[(uint64_t)k2 * 64];
        float s0 = e8m0_f32(ds[(uint64_t)kc * 64]), s1 = e8m0_f32(ds[(uint64_t)k2 * 64]);
        uint4 hb0[4], hb1[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          hb0[i] = col ? hr[kc * 16 + i] : make_uint4(0, 0, 0, 0);
          hb1[i] = col ? hr[k2 * 16 + i] : make_uint4(0, 0, 0, 0);
        }
        const uint32_t w0[4] = {c0.x, c0.y, c0.z, c0.w}, w1[4] = {c1.x, c1.y, c1.z, c1.w};
#pragma unroll
        for (int i = 0; i < 4; ++i)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fp4x8_bf16(w0[i], s0), as_bf16x8(hb0[i]), acc, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fp4x8_bf16(w1[i], s1), as_bf16x8(hb1[i]), acc, 0, 0, 0);
      }
      for (; kc < KC; kc += KSPLIT) {
        uint4 c0 = dc[(uint64_t)kc * 64];
        float s0 = e8m0_f32(ds[(uint64_t)kc * 64]);
        uint4 hb0[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) hb0[i] = col ? hr[kc * 16 + i] : make_uint4(0, 0, 0, 0);
        const uint32_t w0[4] = {c0.x, c0.y, c0.z, c0.w};
#pragma unroll
        for (int i = 0; i < 4; ++i)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fp4x8_bf16(w0[i], s0), as_bf16x8(hb0[i]), acc, 0, 0, 0);
      }
    }
    if (KSPLIT > 1) {
      red[wave][lane] = acc;
      __syncthreads();
      if (ks == 0) {
#pragma unroll
        for (int s = 1; s < KSPLIT; ++s) acc += red[wave + s][lane];
      }
    }
    if (ks == 0 && active && n < ntok) {
      float* dst = a.P + (uint64_t)it.pair[n] * a.H + rt * kTileRows + 4 * g;
      *(float4*)dst = make_float4(acc[0], acc[1], acc[2], acc[3]);
    }
    if (KSPLIT > 1) __syncthreads();
  }
}

// ---- combine -----------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_combine(const float* P, const float* w, int T, int H,
                                                 int k, int n_shared, float* y) {
  const int kk = k + n_shared;
  const int h4 = blockIdx.x * 256 + threadIdx.x;  // float4 index
  const int t = blockIdx.y;
  if (h4 * 4 >= H || t >= T) return;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j = 0; j < k; ++j) {
    const float wj = w[t * k + j];
    const float4 p = *(const float4*)(P + ((uint64_t)t * kk + j) * H + h4 * 4);
    acc.x = fmaf(wj, p.x, acc.x); acc.y = fmaf(wj, p.y, acc.y);
    acc.z = fmaf(wj, p.z, acc.z); acc.w = fmaf(wj, p.w, acc.w);
  }
  for (int s = 0; s < n_shared; ++s) {
    const float4 p = *(const float4*)(P + ((uint64_t)t * kk + k + s) * H + h4 * 4);
    acc.x += p.x; acc.y += p.y; acc.z += p.z; acc.w += p.w;
  }
  *(float4*)(y + (uint64_t)t * H + h4 * 4) = acc;
}

// ---- debug dequant -----------------------------------------------------------------------
// One wave per tile; the MXFP4 path decodes with the same conversion the GEMVs use.
__global__ __launch_bounds__(64) void k_dequant_mx(const uint8_t* codes, const uint8_t* scales,
                                                   int R, int K, float* out) {
  const int KC = K / kTileK;
  const int tile = blockIdx.x, lane = threadIdx.x;
  const int rt = tile / KC, kc = tile % KC;
  const int row = rt * kTileRows + (lane & 15);
  const int k0 = kc * kTileK + 32 * (lane >> 4);
  const uint4 c = ((const uint4*)codes)[(uint64_t)tile * 64 + lane];
  const float s = e8m0_f32(scales[(uint64_t)tile * 64 + lane]);
  const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    bf16x8 v = fp4x8_bf16(w[i], s);
#pragma unroll
    for (int q = 0; q < 8; ++q) out[(uint64_t)row * K + k0 + 8 * i + q] = (float)v[q];
  }
}

// NVFP4 reference-grade decode (E2M1 table value * E4M3 value * tensor scale, fp32).
__device__ __forceinline__ float e2m1_f32(uint32_t c) {
  const float mag[8] = {0.f, 0.5f, 1.f, 1.5f, 2.f, 3.f, 4.f, 6.f};
  const float m = mag[c & 7];
  return (c & 8) ? -m : m;
}
__device__ __forceinline__ float e4m3_f32(uint32_t c) {
  const uint32_t e = (c >> 3) & 15, m = c & 7;
  float v;
  if (e == 15 && m == 7) v = __uint_as_float(0x7fc00000u);
  else if (e == 0) v = ldexpf((float)m / 8.f, -6);
  else v = ldexpf(1.f + (float)m / 8.f, (int)e - 7);
  return (c & 0x80) ? -v : v;
}

__global__ __launch_bounds__(64) void k_dequant_nv(const uint8_t* codes, const uint8_t* scales,
                                                   int R, int K, float ts, float* out) {
  const int KC = K / kTileK;
  const int tile = blockIdx.x, lane = threadIdx.x;
  const int rt = tile / KC, kc = tile % KC;
  const int row = rt * kTileRows + (lane & 15);
  const int k0 = kc * kTileK + 32 * (lane >> 4);
  const uint4 c = ((const uint4*)codes)[(uint64_t)tile * 64 + lane];
  const float s0 = e4m3_f32(scales[(uint64_t)tile * 128 + 2 * lane]);
  const float s1 = e4m3_f32(scales[(uint64_t)tile * 128 + 2 * lane + 1]);
  const uint32_t w[4] = {c.x, c.y, c.z, c.w};
  for (int q = 0; q < 32; ++q) {
    const uint32_t code = (w[q >> 3] >> (4 * (q & 7))) & 15;
    out[(uint64_t)row * K + k0 + q] = e2m1_f32(code) * (q < 16 ? s0 : s1) * ts;
  }
}

}  // namespace ft

// ---- launchers (C linkage, called by the host runtime) -----------------------------------
using namespace ft;

static int grid_for(int units_max, int cap) {
  int g = units_max < cap ? units_max : cap;
  return g < 1 ? 1 : g;
}

extern "C" int ftk_route_decode(const uint16_t* x, const float* wr, const float* b, int T, int H,
                                int E, int k, int n_shared, float* logits, int* ticket,
                                int32_t* idx_out, float* w_out, const int32_t* e2s,
                                WorkItem* items, int* n_items, hipStream_t st) {
  RouteArgs a{x, wr, b, T, H, E, k, n_shared, logits, ticket, idx_out, w_out, e2s, items, n_items};
  hipLaunchKernelGGL(k_route_decode, dim3((E + 3) / 4), dim3(256), 0, st, a);
  return (int)hipGetLastError();
}

// ev: null, or 4 events [gate/up start, gate/up stop, down start, down stop] that the
// dispatches themselves record (hipExtLaunchKernelGGL), so host gaps are not counted.
#define FT_LAUNCH(kern, grid, evs, eve, args)                                               \
  do {                                                                                      \
    if (evs) hipExtLaunchKernelGGL(kern, grid, dim3(256), 0, st, evs, eve, 0, args);        \
    else hipLaunchKernelGGL(kern, grid, dim3(256), 0, st, args);                            \
  } while (0)

extern "C" int ftk_ffn_decode(const uint16_t* x, int H, int I, const WorkItem* items,
                              const int* n_items, int max_items, const uint8_t* pool,
                              const uint8_t* shared, uint64_t stride, const BlobLayout* L,
                              uint16_t* h, float* P, hipStream_t st, const hipEvent_t* ev) {
  FfnArgs a{x, H, I, items, n_items, pool, shared, stride, *L, h, P};
  const int cap = 2048;
  hipEvent_t e0 = ev ? ev[0] : nullptr, e1 = ev ? ev[1] : nullptr;
  hipEvent_t e2 = ev ? ev[2] : nullptr, e3 = ev ? ev[3] : nullptr;
  // gate/up: split K over 4 waves when K is long, else give each wave its own row tile
  {
    const int KC = H / kTileK, RT = I / kTileRows;
    if (KC >= 8) {
      FT_LAUNCH(k_gateup<4>, dim3(grid_for(max_items * RT, cap)), e0, e1, a);
    } else if (KC >= 4) {
      FT_LAUNCH(k_gateup<2>, dim3(grid_for(max_items * ((RT + 1) / 2), cap)), e0, e1, a);
    } else {
      FT_LAUNCH(k_gateup<1>, dim3(grid_for(max_items * ((RT + 3) / 4), cap)), e0, e1, a);
    }
  }
  FfnArgs d = a;
  d.x = h;
  {
    const int KC = I / kTileK, RT = H / kTileRows;
    if (KC >= 16) {
      FT_LAUNCH(k_down<2>, dim3(grid_for(max_items * ((RT + 1) / 2), cap)), e2, e3, d);
    } else {
      FT_LAUNCH(k_down<1>, dim3(grid_for(max_items * ((RT + 3) / 4), cap)), e2, e3, d);
    }
  }
  return (int)hipGetLastError();
}

extern "C" int ftk_combine(const float* P, const float* w, int T, int H, int k, int n_shared,
                           float* y, hipStream_t st) {
  dim3 grid((H / 4 + 255) / 256, T);
  hipLaunchKernelGGL(k_combine, grid, dim3(256), 0, st, P, w, T, H, k, n_shared, y);
  return (int)hipGetLastError();
}

extern "C" int ftk_dequant(const uint8_t* blob, const BlobLayout* L, int matrix, float ts,
                           float* out, hipStream_t st) {
  const int R = matrix == 2 ? L->H : L->I;
  const int K = matrix == 2 ? L->I : L->H;
  const uint8_t* codes = blob + L->off[2 * matrix];
  const uint8_t* scales = blob + L->off[2 * matrix + 1];
  const int tiles = (R / kTileRows) * (K / kTileK);
  if (L->fmt == FT_MXFP4)
    hipLaunchKernelGGL(k_dequant_mx, dim3(tiles), dim3(64), 0, st, codes, scales, R, K, out);
  else
    hipLaunchKernelGGL(k_dequant_nv, dim3(tiles), dim3(64), 0, st, codes, scales, R, K, ts, out);
  return (int)hipGetLastError();
}
