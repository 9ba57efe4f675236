// Prefill kernels of libft for gfx950 (CDNA4).
//
// Prefill and decode get separate strategies (smzdm explainer aomxznrn, "FreeToken干的事",
// item 4): prefill is compute-bound, so the (token, expert) pairs are sorted by expert and
// each expert's tokens go through one grouped GEMM on the matrix cores.  One call of T
// tokens through an all-resident layer runs, on the caller's stream:
//   k_router_prefill  partial logits x W_r^T over `splits` ranges of H: the fp32 router
//                     weights are held as three bf16 planes whose sum is exactly W_r (24 =
//                     3 x 8 significant bits), so the 32x32x16 bf16 MFMA forms exact products
//                     with fp32 accumulation.
//   k_topk_many       logits = sum of the partials in order + b; per-token top-k + softmax
//                     (the decode routine, one token per wave).
//   k_perm_masks      per 256-token block: a token bitmask per expert (LDS atomics).
//   k_perm_scan       counts, offsets (exclusive scan), per-block bases, the row-block map.
//   k_perm_place      pos[t][j] = base + (tokens below t in the block's mask); the row of
//                     every pair, expert ascending then token ascending (stable).
//   k_tile_x          the permuted x rows, each expert's padded to a multiple of 32, into
//                     the token tiles of the gate/up GEMM (MFMA operand order).
//   k_zero            y = 0 (the down GEMM adds into it).
//   k_xgemm<0>        per (expert, 256-row block, 128 gate + 128 up features): G, U on the
//                     32x32x16 bf16 MFMA with the FP4 weights decoded to bf16 in registers
//                     (E2M1 x E4M3 has at most 6 significant bits, so the decode is exact; the
//                     fp32 tensor scale is applied in the epilogue), h = bf16(silu(ts_g G) *
//                     (ts_u U)), silu on the hardware exp and reciprocal.
//   k_xgemm<1>        per (expert, 256-row block, 256 rows of W_d): y[t] += w ts_d (W_d h) for
//                     each row's token t and routing weight w (the combine, as atomic adds).
// The scaled-FP4 mode replaces the two GEMMs (both operands FP4) and combines separately:
//   k_quant_x         x -> MXFP4 per 32 along H (OCP MX rule), once per token.
//   k_tile_xq         the quantised rows, in permuted order with every expert padded to a
//                     multiple of 16 rows, into the tile format of the GEMM operand.
//   k_s1_gemm<0>      per (expert, 256-row block, 128 gate + 128 up features): G, U on the
//                     32x32x64 scaled-FP4 MFMA; h = silu(G) * U quantised to MXFP4 per 32
//                     features in the epilogue.
//   k_s1_gemm<1>      per (expert, row block, 256 rows of W_d): Y_perm = W_d h.
//   k_unpermute       y[t] = sum_j w[t][j] Y_perm[pos[t][j]].
// and its NVFP4 weights come from k_nv_to_mx, run once when the layer is created.
// Workgroups of one kernel never wait on each other.
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>

#include <algorithm>
#include <type_traits>

#include "ft_device.h"

namespace ft {

// A 16-byte buffer copy into LDS with the nontemporal bit: for weight streams read once per
// block, so they do not displace the token tiles that other blocks re-read from L2 (measured:
// the exact-mode down GEMM 925 -> 915 us, the scaled-FP4 down 430 -> 418 us; the scaled-FP4
// gate/up got slower with it and keeps plain copies).
__device__ __forceinline__ void bdma16_nt(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff,
                                          void* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 16, voff, soff, 0, 2);
}

// ---- router ------------------------------------------------------------------------------
// planes (bf16, tiled, see PrefillLaunch::wr_planes): w = plane0 + plane1 + plane2 exactly
// (each plane takes the next 8 significant bits by truncation; the remainders are exact in
// fp32).  One thread per (expert tile, K-step, lane): 8 weights -> 16 bytes in each plane.
__global__ __launch_bounds__(256) void k_split_router(const float* __restrict__ wr, int E, int H,
                                                      uint16_t* __restrict__ planes) {
  const int NTe = router_expert_tiles(E), KS = H / 16;
  const uint64_t u = (uint64_t)blockIdx.x * 256 + threadIdx.x;
  const uint64_t per_plane = (uint64_t)NTe * KS * 64;
  if (u >= per_plane) return;
  const int l = (int)(u & 63);
  const uint64_t op = u >> 6;   // et * KS + ks
  const int et = (int)(op / KS), ks = (int)(op % KS);
  const int e = et * 32 + (l & 31);
  const int k0 = ks * 16 + 8 * (l >> 5);
  uint32_t pw[3][4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t lo[3], hi[3];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      const float w = e < E ? wr[(uint64_t)e * H + k0 + 2 * i + h2] : 0.f;
      const uint32_t p0 = __float_as_uint(w) & 0xffff0000u;
      const float r1 = w - __uint_as_float(p0);
      const uint32_t p1 = __float_as_uint(r1) & 0xffff0000u;
      const float r2 = r1 - __uint_as_float(p1);
      const uint32_t p2 = __float_as_uint(r2) & 0xffff0000u;
      const uint32_t ps[3] = {p0 >> 16, p1 >> 16, p2 >> 16};
#pragma unroll
      for (int p = 0; p < 3; ++p) (h2 ? hi : lo)[p] = ps[p];
    }
#pragma unroll
    for (int p = 0; p < 3; ++p) pw[p][i] = lo[p] | (hi[p] << 16);
  }
#pragma unroll
  for (int p = 0; p < 3; ++p)
    *(uint4*)(planes + ((uint64_t)p * per_plane + u) * 8) = make_uint4(pw[p][0], pw[p][1], pw[p][2], pw[p][3]);
}

// D (32 rows x 32 columns) += A (32 x 16 bf16) * B (16 x 32 bf16): lane l holds row / column
// l % 32, K elements 8 (l / 32) .. + 7; D element (8 (r / 4) + 4 (l / 32) + r % 4, l % 32) in
// register r of lane l (the same result layout as the FP4 32x32 MFMA).
__device__ __forceinline__ f32x16 mfma_bf16_32(const uint4& a, const uint4& b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// Two fp32 values -> two bf16 rounded to nearest even by one hardware convert (low half
// first; a NaN stays a NaN).
__device__ __forceinline__ uint32_t bf16x2_bits(float lo, float hi) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2));
}

// Grid (ceil(T/128), splits, expert groups of up to 6 tiles).  Wave w takes tokens 32 w ..
// + 31 of the block (the MFMA columns, loaded from x per lane, two chunks ahead); the NT
// expert tiles x 3 planes x 2 K-steps of each 32-K chunk (one 1 KB operand each) are copied
// global -> LDS through four stages, shared by the four waves.  Each wave issues the same
// number of copies per chunk (slots past the last operand get a duplicate, never read).
template <int NT, bool FAST>
__global__ __launch_bounds__(256) void k_router_prefill(PrefillLaunch a) {
  constexpr int NOP = 6 * NT;               // operands per chunk: tile j, plane p, K-step ks
  constexpr int NDMA = (NOP + 3) / 4;       // copies per wave per chunk
  constexpr int SLOTS = 4 * NDMA * 64;      // uint4 per stage
  __shared__ uint4 r0[SLOTS], r1[SLOTS], r2[SLOTS], r3[SLOTS];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tb = blockIdx.x, sp = blockIdx.y, grp = blockIdx.z;
  const int KS = a.H / a.splits, k0 = sp * KS, NC = KS / 32;
  const int NTe = router_expert_tiles(a.E), et0 = grp * kRouterGroupTiles;
  const uint64_t per_plane = (uint64_t)NTe * (a.H / 16) * 64;   // uint4 per plane
  const uint4* planes = (const uint4*)a.wr_planes;
  // this wave's copies: operand slots wave + 4 i
  const uint4* osrc[NDMA];
#pragma unroll
  for (int i = 0; i < NDMA; ++i) {
    const int q = min(wave + 4 * i, NOP - 1);
    const int j = q / 6, pl = (q / 2) % 3, ks = q % 2;
    const int et = min(et0 + j, NTe - 1);
    osrc[i] = planes + (uint64_t)pl * per_plane + ((uint64_t)et * (a.H / 16) + k0 / 16 + ks) * 64 + lane;
  }
  const int t = min(tb * kRouterTokens + 32 * wave + (lane & 31), a.T - 1);
  const uint16_t* xsrc = a.x + (uint64_t)t * a.H + k0 + 8 * (lane >> 5);

  f32x16 acc[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0.f;

  uint4 b0[2], b1[2], b2[2], b3[2];
#define FT_RT_ISSUE(c_, ST_)                                                               \
  do {                                                                                     \
    const int cc_ = min((c_), NC - 1);                                                     \
    _Pragma("unroll") for (int i_ = 0; i_ < NDMA; ++i_)                                    \
      dma16(osrc[i_] + (uint64_t)cc_ * 2 * 64, &ST_[(wave + 4 * i_) * 64]);                \
  } while (0)
#define FT_RT_XLOAD(c_, B_)                                                                \
  do {                                                                                     \
    const int cc_ = min((c_), NC - 1);                                                     \
    B_[0] = *(const uint4*)(xsrc + cc_ * 32);                                              \
    B_[1] = *(const uint4*)(xsrc + cc_ * 32 + 16);                                         \
  } while (0)
#define FT_RT_SYNC()                                                                       \
  do {                                                                                     \
    __builtin_amdgcn_s_waitcnt(FT_VMCNT(NDMA + 2) & ~(15 << 8));                           \
    asm volatile("" ::: "memory");                                                         \
    __builtin_amdgcn_s_barrier();                                                          \
    asm volatile("" ::: "memory");                                                         \
  } while (0)
  // chunk c: its copies (issued three chunks earlier) and tokens (two chunks earlier) have
  // landed once at most the next chunk's copies and tokens are in flight
#define FT_RT_STEP(c_, ST_, STN_, B_, BN_)                                                 \
  do {                                                                                     \
    FT_RT_SYNC();                                                                          \
    FT_RT_ISSUE((c_) + 3, STN_);                                                           \
    FT_RT_XLOAD((c_) + 2, BN_);                                                            \
    if (FAST || (c_) < NC) {                                                               \
      _Pragma("unroll") for (int ks_ = 0; ks_ < 2; ++ks_)                                  \
        _Pragma("unroll") for (int j_ = 0; j_ < NT; ++j_)                                  \
          _Pragma("unroll") for (int p_ = 0; p_ < 3; ++p_)                                 \
            acc[j_] = mfma_bf16_32(ST_[(j_ * 6 + p_ * 2 + ks_) * 64 + lane], B_[ks_], acc[j_]); \
    }                                                                                      \
  } while (0)

  FT_RT_ISSUE(0, r0);
  FT_RT_ISSUE(1, r1);
  FT_RT_XLOAD(0, b0);
  FT_RT_ISSUE(2, r2);
  FT_RT_XLOAD(1, b1);
  for (int c = 0; c < NC; c += 4) {
    FT_RT_STEP(c, r0, r3, b0, b2);
    if (FAST || c + 1 < NC) FT_RT_STEP(c + 1, r1, r0, b1, b3);
    if (FAST || c + 2 < NC) FT_RT_STEP(c + 2, r2, r1, b2, b0);
    if (FAST || c + 3 < NC) FT_RT_STEP(c + 3, r3, r2, b3, b1);
  }
#undef FT_RT_STEP
#undef FT_RT_SYNC
#undef FT_RT_XLOAD
#undef FT_RT_ISSUE
  __builtin_amdgcn_s_waitcnt(FT_VMCNT(0));

  // partial logits [sp][t][e]: register 4q + r of lane l is expert 32 et + 8q + 4 (l / 32) + r,
  // token 32 wave + l % 32 of the block
  const int tok = tb * kRouterTokens + 32 * wave + (lane & 31);
  if (tok < a.T) {
    float* out = a.logits + ((uint64_t)sp * a.T + tok) * a.E;
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const int et = et0 + j;
      if (et >= NTe) break;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int e = et * 32 + 8 * q + 4 * (lane >> 5);
        if (e + 3 < a.E && (a.E & 3) == 0) {
          *(float4*)(out + e) = make_float4(acc[j][4 * q], acc[j][4 * q + 1], acc[j][4 * q + 2],
                                            acc[j][4 * q + 3]);
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (e + r < a.E) out[e + r] = acc[j][4 * q + r];
        }
      }
    }
  }
}

// ---- top-k for many tokens ------------------------------------------------------------------
// Same radix select as decode (see ft_decode.hip), four tokens per workgroup.
__device__ __forceinline__ uint32_t order_key_p(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Four tokens per workgroup, one per wave, so the waves' partial-logit loads are all in flight
// together (more workgroups per CU rather than tokens taken one after another by a wave).
constexpr int kTopkTokens = 4;
template <int EPL>
__global__ __launch_bounds__(256) void k_topk_many(const float* __restrict__ logits, int splits,
                                                   const float* __restrict__ bias, int T, int E,
                                                   int k, int32_t* __restrict__ idx,
                                                   float* __restrict__ w) {
  __shared__ float c_val[kTopkTokens][FT_MAX_TOPK];
  __shared__ int c_idx[kTopkTokens][FT_MAX_TOPK];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int tb = blockIdx.x * kTopkTokens;
  const int nt = min(kTopkTokens, T - tb);
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int tl = wave; tl < nt; tl += 4) {
    const int t = tb + tl;
    float v[EPL];
    uint32_t key[EPL];
    // logit = (partial 0 + partial 1 + ...) + b, in that order; every partial is loaded
    // before the sum (unconditional loads of a clamped split index, unused ones ignored)
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int e = min(lane + 64 * i, E - 1);
      float part[kRouterMaxSplits];
#pragma unroll
      for (int sp = 0; sp < kRouterMaxSplits; ++sp)
        part[sp] = logits[((uint64_t)min(sp, splits - 1) * T + t) * E + e];
      float acc = part[0];
#pragma unroll
      for (int sp = 1; sp < kRouterMaxSplits; ++sp)
        if (sp < splits) acc += part[sp];
      v[i] = acc + (bias ? bias[e] : 0.f);
    }
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      if (v[i] != v[i]) v[i] = -INFINITY;
      key[i] = lane + 64 * i < E ? order_key_p(v[i]) : 0u;
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
        const int p = sel_before + __popcll(selb & lt_mask);
        c_val[tl][p] = v[i];
        c_idx[tl][p] = lane + 64 * i;
      }
      eq_before += __popcll(eqb);
      sel_before += __popcll(selb);
    }
  }
  __syncthreads();
  const int tid = threadIdx.x;
  if (tid < nt * k) {
    const int tl = tid / k, j = tid % k;
    const float vj = c_val[tl][j];
    const int ej = c_idx[tl][j];
    int rank = 0;
    float vmax = vj;
    for (int q = 0; q < k; ++q) {
      const float vq = c_val[tl][q];
      rank += (vq > vj || (vq == vj && c_idx[tl][q] < ej));
      vmax = fmaxf(vmax, vq);
    }
    float sum = 0.f;
    for (int q = 0; q < k; ++q) sum += expf(c_val[tl][q] - vmax);
    idx[(uint64_t)(tb + tl) * k + rank] = ej;
    w[(uint64_t)(tb + tl) * k + rank] = expf(vj - vmax) / sum;
  }
}

// ---- permutation ----------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_perm_masks(PrefillLaunch a) {
  __shared__ uint32_t m[1024][8];
  const int b = blockIdx.x, tid = threadIdx.x;
  for (int i = tid; i < a.E * 8; i += 256) m[i >> 3][i & 7] = 0u;
  __syncthreads();
  const int t = b * kPermBlock + tid;
  if (t < a.T)
    for (int j = 0; j < a.k; ++j) {
      const int e = a.idx[(uint64_t)t * a.k + j];
      atomicOr(&m[e][tid >> 5], 1u << (tid & 31));
    }
  __syncthreads();
  for (int e = tid; e < a.E; e += 256) {
    int c = 0;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      a.masks[((uint64_t)b * a.E + e) * 8 + q] = m[e][q];
      c += __popc(m[e][q]);
    }
    a.bcnt[(uint64_t)b * a.E + e] = c;
  }
}

// One workgroup: counts, offsets, bases and the map of mrows-row token blocks.
__global__ __launch_bounds__(256) void k_perm_scan(PrefillLaunch a) {
  __shared__ int s_wave[4];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int NBk = (a.T + kPermBlock - 1) / kPermBlock;
  int cnt[4] = {0, 0, 0, 0}, blk[4], pad[4];
  // the per-block counts of this thread's four experts, eight blocks at a time with every
  // load of a round in flight together (clamped addresses, masked sums)
  for (int b0 = 0; b0 < NBk; b0 += 8) {
    int v[8][4];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int b = min(b0 + u, NBk - 1);
#pragma unroll
      for (int i = 0; i < 4; ++i) v[u][i] = a.bcnt[(uint64_t)b * a.E + min(tid * 4 + i, a.E - 1)];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (b0 + u < NBk && tid * 4 + i < a.E) cnt[i] += v[u][i];
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    blk[i] = (cnt[i] + a.mrows - 1) / a.mrows;
    pad[i] = (cnt[i] + a.pad_rows - 1) / a.pad_rows * a.pad_rows;
  }
  // exclusive scans over experts (pairs, row blocks and, in the MXFP4 mode, 16-padded rows),
  // four experts per thread
  const int npass = a.poff ? 3 : 2;
  for (int pass = 0; pass < npass; ++pass) {
    int v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = pass == 0 ? cnt[i] : pass == 1 ? blk[i] : pad[i];
    const int mine = v[0] + v[1] + v[2] + v[3];
    int incl = mine;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int nb = __shfl_up(incl, o, 64);
      if (lane >= o) incl += nb;
    }
    __syncthreads();
    if (lane == 63) s_wave[wave] = incl;
    __syncthreads();
    int base = incl - mine;
    for (int w2 = 0; w2 < wave; ++w2) base += s_wave[w2];
    const int total = s_wave[0] + s_wave[1] + s_wave[2] + s_wave[3];
    int* out = pass == 0 ? a.offsets : pass == 1 ? a.tb_off : a.poff;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = tid * 4 + i;
      if (e < a.E) {
        out[e] = base;
        if (pass == 1 && a.blk_e)   // the expert of every row block
          for (int j = 0; j < v[i]; ++j) a.blk_e[base + j] = e;
        if (pass == 2 && a.tile_e)  // the expert of every padded row group
          for (int j = 0; j < v[i] / a.pad_rows; ++j) a.tile_e[base / a.pad_rows + j] = e;
        if (pass == 0) {
          a.counts[e] = cnt[i];
          int run = base;
          for (int b0 = 0; b0 < NBk; b0 += 8) {
            int v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = a.bcnt[(uint64_t)min(b0 + u, NBk - 1) * a.E + e];
#pragma unroll
            for (int u = 0; u < 8; ++u)
              if (b0 + u < NBk) {
                a.base[(uint64_t)(b0 + u) * a.E + e] = run;
                run += v[u];
              }
          }
        }
      }
      base += v[i];
    }
    if (tid == 0) out[a.E] = total;
  }
}

// One thread per token.  KMAX (>= k) bounds the choices: all of a token's index and weight
// loads are issued together, then all of its mask-row and base loads (clamped addresses,
// results past k unused), so the kernel waits on two rounds of loads rather than two per
// choice.
template <int KMAX>
__global__ __launch_bounds__(256) void k_perm_place(PrefillLaunch a) {
  const int b = blockIdx.x, tl = threadIdx.x;
  const int t = b * kPermBlock + tl;
  if (t >= a.T) return;
  int e[KMAX];
  float wv[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    const uint64_t q = (uint64_t)t * a.k + min(j, a.k - 1);
    e[j] = a.idx[q];
    wv[j] = a.w[q];
  }
  uint4 m0[KMAX], m1[KMAX];
  int bs[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    const uint64_t row = (uint64_t)b * a.E + e[j];
    m0[j] = *(const uint4*)(a.masks + row * 8);
    m1[j] = *(const uint4*)(a.masks + row * 8 + 4);
    bs[j] = a.base[row];
  }
  const int wq = tl >> 5;
  const uint32_t below = (1u << (tl & 31)) - 1u;
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    if (j >= a.k) break;
    const uint32_t m[8] = {m0[j].x, m0[j].y, m0[j].z, m0[j].w, m1[j].x, m1[j].y, m1[j].z, m1[j].w};
    // tokens of this block below t that chose e[j]: whole words below t's word, then the
    // bits below t in its own word
    int r = 0;
#pragma unroll
    for (int q = 0; q < 8; ++q) r += q < wq ? __popc(m[q]) : (q == wq ? __popc(m[q] & below) : 0);
    const int p = bs[j] + r;
    a.pos[(uint64_t)t * a.k + j] = p;
    a.perm_tok[p] = t;
    a.perm_w[p] = wv[j];
  }
}

__device__ __forceinline__ float blob_tscale(const uint8_t* blob, int m) {
  return ((const BlobHeader*)blob)->tensor_scale[m];
}

// ---- grouped GEMM, exact mode: weights decoded in registers, tokens through LDS -----------
// A workgroup owns one block of up to 256 permuted rows of one expert and one feature block:
//   MODE 0 (gate/up + SwiGLU): 128 features, i.e. 128 gate rows and the same 128 up rows;
//   MODE 1 (down + combine):   256 rows of W_d (outputs).
// Eight waves, two per SIMD: wave w owns one 32-row weight operand (MODE 0: gate rows of 16
// features in lanes 0..15 and the up rows of the same features in lanes 16..31, so one lane
// holds a feature's gate and up sums; MODE 1: two 16-row tiles of W_d) and multiplies it by
// all of the block's 32-row token operands on the 32x32x16 bf16 MFMA with fp32 accumulators.
// Each weight is decoded once per block, and the second wave on a SIMD issues while the
// first waits; the token operands are read from LDS by every wave (the LDS has the bandwidth).
// The K axis runs in chunks of 64.  Per chunk the waves copy global -> LDS (buffer loads
// that land every lane's 16 bytes in lane order) their weight operands' code slots and scale
// dwords and four of the 32 token tiles (8 operands x 4 steps), all in MFMA operand order, so
// the reads are one conflict-free 16-byte LDS read per lane.  Three LDS stages keep two
// chunks of copies in flight while one is multiplied.
// A weight lane (row r, K half h) reads the tile slot r % 16 + 16 (2 c + h) of chunk half c:
// 32 K values, of which step ks takes values 8 ks .. 8 ks + 7; the token lane (row t, half h)
// supplies the same K (64 chunk + 32 h + 8 ks + i), since a dot product needs both operands in
// the same K order and no other.  The weights are decoded to bf16 in registers (exact: an
// E2M1 value times an E8M0 scale, or times an E4M3 scale, has at most 6 significant bits).
// MODE 1 uses the token operand as the MFMA's A and the weights as B, so a result register
// holds 32 consecutive outputs of one row across a lane half: the routing-weighted combine
// is then a coalesced fp32 atomic add of w x ts_d x y into y[token] (y zeroed first), and no
// per-pair output is stored.  Blocks (token block g, feature block fb) sit on XCD g % 8, so
// the feature blocks of one token block share that XCD's L2 for the token rows.
constexpr int kXRows = kGemmM;                // token rows per block
constexpr int kXJ = kXRows / 32;              // 32-row token operands per block
constexpr int kXWaves = 8;                    // waves per workgroup
constexpr int kXThreads = 64 * kXWaves;
constexpr int kXOps = 8 / kXWaves;            // 32-row weight operands per wave
constexpr int kXTok = 4 * kXJ / kXWaves;      // token tiles each wave copies per chunk
constexpr int kXCopies = kXTok + 2 * kXOps;   // copies per wave per chunk (tokens, codes, scales)

template <int MODE, int FMT>
__global__ __launch_bounds__(kXThreads) void k_xgemm(PrefillLaunch a, int NB) {
  // stage s: token operands [ks 4][j kXJ][64 lanes] (tk), then in wk the weight code slots
  // [operand 8][64 lanes] followed by the weight scale dwords [operand 8][64 lanes] (one
  // array per kind and stage: six copy targets, few enough for the compiler to keep apart)
  __shared__ uint4 tk0[4 * kXJ * 64], tk1[4 * kXJ * 64], tk2[4 * kXJ * 64];
  __shared__ uint4 wk0[640], wk1[640], wk2[640];
  __shared__ int s_tok[kXRows];
  __shared__ float s_w[kXRows];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int Lb = blockIdx.x, jj = Lb >> 3;
  const int gblk = (Lb & 7) + 8 * (jj / NB), fb = jj % NB;
  if (gblk >= a.tb_off[a.E]) return;
  const int e = a.blk_e[gblk];
  const int row0 = a.offsets[e] + (gblk - a.tb_off[e]) * kXRows;
  const int nrows = min(kXRows, a.offsets[e + 1] - row0);
  const int nj = (nrows + 31) >> 5;
  const int K = MODE == 0 ? a.H : a.I;
  const int KC = K / kTileK;
  const int nrt = (MODE == 0 ? a.I : a.H) / kTileRows;
  const uint8_t* blob = a.pool + (uint64_t)e * a.stride;
  const int h = lane >> 5, r32 = lane & 31;

  // copy sources: buffer resources over the weight codes, the weight scales and the block's
  // token tiles, a fixed lane offset per copy in a vector register and the chunk's offset in
  // a scalar one, so a chunk step is scalar arithmetic.  Weight operand o of this wave, lane
  // (r32, h): tile rt of matrix m, slot (r32 % 16) + 16 h of chunk 0 (chunk ch adds (ch / 2)
  // tiles and 32 (ch % 2) slots).  MODE 0 reads gate (lanes 0..15) and up (16..31) rows, so
  // the code resource starts at the gate codes and spans to the end of the blob.
  const int m0 = MODE == 0 ? 0 : 2;
  const __amdgpu_buffer_rsrc_t wres = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(blob + a.L.off[2 * m0]), (short)0, (int)(a.L.bytes - a.L.off[2 * m0]), kBufFlags);
  const __amdgpu_buffer_rsrc_t sres = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(blob + a.L.off[2 * m0 + 1]), (short)0, (int)(a.L.bytes - a.L.off[2 * m0 + 1]),
      kBufFlags);
  uint32_t wvo[kXOps], svo[kXOps];
#pragma unroll
  for (int o = 0; o < kXOps; ++o) {
    const int go = wave * kXOps + o;   // the workgroup's operand index, 0..7
    int m, rt;
    if (MODE == 0) { m = r32 >> 4; rt = fb * 8 + go; }
    else { m = 2; rt = min(fb * 16 + 2 * go + (r32 >> 4), nrt - 1); }
    const int slot = (r32 & 15) + 16 * h;
    wvo[o] = (uint32_t)(a.L.off[2 * m] - a.L.off[2 * m0] + ((uint64_t)rt * KC * 64 + slot) * 16);
    const uint64_t sb = FMT == FT_MXFP4 ? (uint64_t)rt * KC * 64 + slot
                                        : (uint64_t)rt * KC * 128 + 2 * slot;
    svo[o] = (uint32_t)(a.L.off[2 * m + 1] - a.L.off[2 * m0 + 1] + (sb & ~(uint64_t)3));
  }
  // this wave's token copies: tiles (step ks, operand j) with ks * kXJ + j in
  // [kXTok wave, kXTok (wave + 1)), each from a row group of the tiled operand (a group past
  // the block re-reads the block's last group; its results are never used)
  const int prow0 = a.poff[e] + (gblk - a.tb_off[e]) * kXRows;   // padded row of the block
  const uint32_t gbytes = (uint32_t)(K / 64) * 4096;              // one row group's tiles
  const __amdgpu_buffer_rsrc_t tres = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const uint8_t*)(MODE == 0 ? a.xtb : a.htb) + (uint64_t)(prow0 >> 5) * gbytes),
      (short)0, (int)(nj * gbytes), kBufFlags);
  uint32_t tvo[kXTok];
#pragma unroll
  for (int q = 0; q < kXTok; ++q) {
    const int tile = kXTok * wave + q, ks = tile / kXJ, j = tile % kXJ;
    tvo[q] = (uint32_t)min(j, nj - 1) * gbytes + ks * 1024 + 16 * lane;
  }
  if (MODE == 1) {   // visible to the epilogue through the main loop's barriers
    const float tsd = blob_tscale(blob, 2);
    for (int i = tid; i < nrows; i += kXThreads) {
      s_tok[i] = a.perm_tok[row0 + i];
      s_w[i] = a.perm_w[row0 + i] * tsd;
    }
  }
  // The main loop and epilogue with NJ (= ceil(rows / 32)) token operands, a compile-time
  // count so that every step is straight-line code.  The LDS arrays are named directly (they
  // are static, not captured), which lets the compiler see that the reads of one stage do not
  // wait on the copies into another.
  auto block = [&](auto njc) {
    constexpr int NJ = decltype(njc)::value;
    const int NC = K / 64;

#define FT_X_ISSUE(ch_, TK_, WK_)                                                          \
    do {                                                                                     \
      const int c_ = min((ch_), NC - 1);                                                     \
      const uint32_t wo_ = (c_ >> 1) * 1024 + (c_ & 1) * 512;                                \
      const uint32_t so_ = FMT == FT_MXFP4 ? (c_ >> 1) * 64 + (c_ & 1) * 32                  \
                                           : (c_ >> 1) * 128 + (c_ & 1) * 64;                \
      _Pragma("unroll") for (int o_ = 0; o_ < kXOps; ++o_) {                                 \
        bdma16_nt(wres, wvo[o_], wo_, &WK_[(wave * kXOps + o_) * 64]);                       \
        bdma4(sres, svo[o_], so_, (uint32_t*)&WK_[512] + (wave * kXOps + o_) * 64);          \
      }                                                                                      \
      _Pragma("unroll") for (int q_ = 0; q_ < kXTok; ++q_)                                   \
        bdma16(tres, tvo[q_], (uint32_t)c_ * 4096, &TK_[(kXTok * wave + q_) * 64]);          \
    } while (0)

    f32x16 acc[kXOps][NJ];
#pragma unroll
    for (int o = 0; o < kXOps; ++o)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[o][j][r] = 0.f;

    // Software pipeline over the four 16-K steps of a chunk: while the MFMAs of step ks run,
    // the token operands of step ks + 1 are read from LDS and its weights decoded.  Between
    // steps 2 and 3 every wave's reads of the chunk are done, so after a count wait and a
    // barrier that stage is refilled with the chunk three ahead; step 3's MFMAs then cover the
    // reads and decode of the next chunk's first step.  Scheduling groups fix the interleave,
    // which the compiler would otherwise undo: the LDS reads go out one or two per MFMA in
    // the first half of a step (so they land before the next step needs them), the decode
    // VALU work between the MFMAs of the second half.
    uint4 cw[kXOps], Bc[NJ], Bn[NJ], Ac[kXOps], An[kXOps];
    float s0[kXOps], s1[kXOps];
#define FT_X_READW(WK_, CW_, SW_)                                                           \
    do {                                                                                    \
      _Pragma("unroll") for (int o_ = 0; o_ < kXOps; ++o_) {                                \
        CW_[o_] = WK_[(wave * kXOps + o_) * 64 + lane];                                     \
        SW_[o_] = ((const uint32_t*)&WK_[512])[(wave * kXOps + o_) * 64 + lane];           \
      }                                                                                     \
    } while (0)
#define FT_X_SCALES(SW_, S0_, S1_)                                                          \
    do {                                                                                    \
      _Pragma("unroll") for (int o_ = 0; o_ < kXOps; ++o_) {                                \
        if (FMT == FT_MXFP4) {                                                              \
          S0_[o_] = S1_[o_] = e8m0_f32((SW_[o_] >> (8 * (lane & 3))) & 0xffu);              \
        } else {                                                                            \
          const uint32_t p_ = (SW_[o_] >> (16 * (lane & 1))) & 0xffffu;                     \
          S0_[o_] = e4m3_f32_fast(p_ & 0xffu);                                              \
          S1_[o_] = e4m3_f32_fast(p_ >> 8);                                                 \
        }                                                                                   \
      }                                                                                     \
    } while (0)
#define FT_X_DEC(KS_, CW_, S0_, S1_, A_)                                                    \
    do {                                                                                    \
      _Pragma("unroll") for (int o_ = 0; o_ < kXOps; ++o_) {                                \
        const uint32_t w_ = (KS_) == 0 ? CW_[o_].x : (KS_) == 1 ? CW_[o_].y                 \
                          : (KS_) == 2 ? CW_[o_].z : CW_[o_].w;                             \
        A_[o_] = FMT == FT_MXFP4                                                            \
                     ? __builtin_bit_cast(uint4, fp4x8_bf16(w_, S0_[o_]))                   \
                     : __builtin_bit_cast(uint4, fp4x8_bf16_mul(w_, (KS_) < 2 ? S0_[o_]     \
                                                                           : S1_[o_]));     \
      }                                                                                     \
    } while (0)
#define FT_X_READB(TK_, KS_, B_)                                                            \
    _Pragma("unroll") for (int j_ = 0; j_ < NJ; ++j_) B_[j_] = TK_[((KS_) * kXJ + j_) * 64 + lane]
#define FT_X_MMA()                                                                          \
    _Pragma("unroll") for (int j_ = 0; j_ < NJ; ++j_)                                       \
      _Pragma("unroll") for (int o_ = 0; o_ < kXOps; ++o_)                                  \
        acc[o_][j_] = MODE == 0 ? mfma_bf16_32(Ac[o_], Bc[j_], acc[o_][j_])                 \
                                : mfma_bf16_32(Bc[j_], Ac[o_], acc[o_][j_])
#define FT_X_SCHED(NR_, NV_)                                                                \
    do {                                                                                    \
      _Pragma("unroll") for (int i_ = 0; i_ < NJ * kXOps / 2; ++i_) {                       \
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                  \
        __builtin_amdgcn_sched_group_barrier(0x100, (NR_) * 2 / kXOps, 0);                  \
      }                                                                                     \
      _Pragma("unroll") for (int i_ = 0; i_ < NJ * kXOps / 2; ++i_) {                       \
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                  \
        __builtin_amdgcn_sched_group_barrier(0x002, 2 * (NV_), 0);                          \
      }                                                                                     \
      __builtin_amdgcn_sched_barrier(0);                                                    \
    } while (0)
    // the step after the barrier: its first MFMAs also carry the wave's copies of the chunk
    // three ahead, two each, so the matrix core starts right after the barrier
#define FT_X_SCHED_COPIES()                                                                 \
    do {                                                                                    \
      _Pragma("unroll") for (int i_ = 0; i_ < kXCopies / 2; ++i_) {                         \
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                  \
        __builtin_amdgcn_sched_group_barrier(0x020, 2, 0);                                  \
        __builtin_amdgcn_sched_group_barrier(0x100, 2 / kXOps, 0);                          \
      }                                                                                     \
      _Pragma("unroll") for (int i_ = kXCopies / 2; i_ < NJ * kXOps / 2; ++i_) {            \
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                  \
        __builtin_amdgcn_sched_group_barrier(0x100, 2 / kXOps, 0);                          \
      }                                                                                     \
      _Pragma("unroll") for (int i_ = 0; i_ < NJ * kXOps / 2; ++i_) {                       \
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                  \
        __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);                                  \
      }                                                                                     \
      __builtin_amdgcn_sched_barrier(0);                                                    \
    } while (0)
#define FT_X_NEXT()                                                                         \
    do {                                                                                    \
      _Pragma("unroll") for (int j_ = 0; j_ < NJ; ++j_) Bc[j_] = Bn[j_];                    \
      _Pragma("unroll") for (int o_ = 0; o_ < kXOps; ++o_) Ac[o_] = An[o_];                 \
    } while (0)
    // one chunk, read from stage (TK_, WK_); (TKN_, WKN_) holds the next chunk.  A wave reads
    // only its own weight slots, so it may read the next chunk's weights (in step 2) after
    // its own count wait; the token operands are shared, so they wait for the barrier.
#define FT_X_CHUNK(ch_, TK_, WK_, TKN_, WKN_)                                               \
    do {                                                                                    \
      FT_X_READB(TK_, 1, Bn);                                                               \
      FT_X_DEC(1, cw, s0, s1, An);                                                          \
      FT_X_MMA();                                                                           \
      FT_X_SCHED(1, 4);                                                                     \
      FT_X_NEXT();                                                                          \
      /* this wave's copies of the next chunk have landed: its weights can be read */       \
      __builtin_amdgcn_s_waitcnt(FT_VMCNT(kXCopies));                                       \
      asm volatile("" ::: "memory");                                                        \
      uint4 cwn_[kXOps];                                                                    \
      uint32_t swn_[kXOps];                                                                 \
      float s0n_[kXOps], s1n_[kXOps];                                                       \
      FT_X_READB(TK_, 2, Bn);                                                               \
      FT_X_READW(WKN_, cwn_, swn_);                                                         \
      FT_X_DEC(2, cw, s0, s1, An);                                                          \
      FT_X_MMA();                                                                           \
      FT_X_SCHED(2, 4);                                                                     \
      FT_X_NEXT();                                                                          \
      FT_X_READB(TK_, 3, Bn);                                                               \
      FT_X_SCALES(swn_, s0n_, s1n_);                                                        \
      FT_X_DEC(3, cw, s0, s1, An);                                                          \
      FT_X_MMA();                                                                           \
      FT_X_SCHED(1, 10);                                                                    \
      FT_X_NEXT();                                                                          \
      /* this wave's reads of the stage are done (LDS count 0); after the barrier, every */ \
      /* wave's are, and every wave's copies of the next chunk have landed */               \
      __builtin_amdgcn_s_waitcnt(FT_VMCNT(kXCopies) & ~(15 << 8));                          \
      asm volatile("" ::: "memory");                                                        \
      __builtin_amdgcn_s_barrier();                                                         \
      asm volatile("" ::: "memory");                                                        \
      FT_X_ISSUE((ch_) + 3, TK_, WK_);                                                      \
      FT_X_READB(TKN_, 0, Bn);                                                              \
      FT_X_DEC(0, cwn_, s0n_, s1n_, An);                                                    \
      FT_X_MMA();                                                                           \
      FT_X_SCHED_COPIES();                                                                  \
      FT_X_NEXT();                                                                          \
      _Pragma("unroll") for (int o_ = 0; o_ < kXOps; ++o_) {                                \
        cw[o_] = cwn_[o_]; s0[o_] = s0n_[o_]; s1[o_] = s1n_[o_];                            \
      }                                                                                     \
    } while (0)

    FT_X_ISSUE(0, tk0, wk0);
    FT_X_ISSUE(1, tk1, wk1);
    __builtin_amdgcn_s_waitcnt(FT_VMCNT(kXCopies) & ~(15 << 8));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    FT_X_ISSUE(2, tk2, wk2);
    {
      uint32_t sw0[kXOps];
      FT_X_READW(wk0, cw, sw0);
      FT_X_SCALES(sw0, s0, s1);
    }
    FT_X_READB(tk0, 0, Bc);
    FT_X_DEC(0, cw, s0, s1, Ac);
    // whole rounds of three chunks with no branch inside (a branch there makes the compiler
    // wait for every copy in flight before the next LDS read), then the remaining one or two
    int ch = 0;
    for (; ch + 3 <= NC; ch += 3) {
      FT_X_CHUNK(ch, tk0, wk0, tk1, wk1);
      FT_X_CHUNK(ch + 1, tk1, wk1, tk2, wk2);
      FT_X_CHUNK(ch + 2, tk2, wk2, tk0, wk0);
    }
    if (ch < NC) FT_X_CHUNK(ch, tk0, wk0, tk1, wk1);
    if (ch + 1 < NC) FT_X_CHUNK(ch + 1, tk1, wk1, tk2, wk2);
#undef FT_X_CHUNK
#undef FT_X_NEXT
#undef FT_X_SCHED
#undef FT_X_SCHED_COPIES
#undef FT_X_MMA
#undef FT_X_READB
#undef FT_X_DEC
#undef FT_X_SCALES
#undef FT_X_READW
    // the trailing copies (clamped re-reads) land before the workgroup's LDS is released
    __builtin_amdgcn_s_waitcnt(FT_VMCNT(0));
#undef FT_X_ISSUE

    if (MODE == 0) {
      // lane (r32, h) holds token row 32 j + r32 and, in registers 8 (r / 4) + 4 h + r % 4 for
      // r < 8, gate features f0 + 8 (r / 4) + 4 h + r % 4 of operand o, with the up sums of the
      // same features in registers r + 8
      const float tsg = blob_tscale(blob, 0), tsu = blob_tscale(blob, 1);
      // into the down GEMM's token tiles: feature f = 64 c + 32 h' + 8 s + i of padded row
      // 32 g + t sits in tile (g, c, s), lane t + 32 h', element i; a lane's four consecutive
      // features are one 8-byte piece
      const int NCI = a.I / 64;
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int tl = 32 * j + r32;
        if (tl < nrows) {
          const int prow = prow0 + tl, g = prow >> 5, t = prow & 31;
#pragma unroll
          for (int o = 0; o < kXOps; ++o) {
#pragma unroll
            for (int q = 0; q < 2; ++q) {
              const int f = fb * 128 + (wave * kXOps + o) * 16 + 8 * q + 4 * h;
              float hf[4];
#pragma unroll
              for (int r = 0; r < 4; ++r)
                hf[r] = silu_fast(acc[o][j][4 * q + r] * tsg) * (acc[o][j][8 + 4 * q + r] * tsu);
              const int c = f >> 6, kk = f & 63;
              const uint64_t slot = (((uint64_t)g * NCI + c) * 4 + ((kk >> 3) & 3)) * 64 + t +
                                    32 * (kk >> 5);
              *(uint2*)(a.htb + slot * 8 + (kk & 7)) =
                  make_uint2(bf16x2_bits(hf[0], hf[1]), bf16x2_bits(hf[2], hf[3]));
            }
          }
        }
      }
    } else {
      // lane (r32, h) holds output fb * 256 + 32 (wave kXOps + o) + r32 of token rows
      // 32 j + 8 (r / 4) + 4 h + r % 4 in register r
#pragma unroll
      for (int o = 0; o < kXOps; ++o) {
        const int out = fb * 256 + (wave * kXOps + o) * 32 + r32;
        if (out < a.H) {
#pragma unroll
          for (int j = 0; j < NJ; ++j) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int tl = 32 * j + 8 * (r >> 2) + 4 * h + (r & 3);
              if (tl < nrows)
                unsafeAtomicAdd(a.y + (uint64_t)s_tok[tl] * a.H + out, s_w[tl] * acc[o][j][r]);
            }
          }
        }
      }
    }
  };
#define FT_X_BLOCK(N)                                                                       \
  case N:                                                                                  \
    block(std::integral_constant<int, N>{});                                               \
    break
  if constexpr (kXJ == 8) {
    switch (nj) {
      FT_X_BLOCK(1); FT_X_BLOCK(2); FT_X_BLOCK(3); FT_X_BLOCK(4);
      FT_X_BLOCK(5); FT_X_BLOCK(6); FT_X_BLOCK(7); default: FT_X_BLOCK(8);
    }
  } else {
    static_assert(kXJ == 4, "blocks of 128 or 256 rows");
    switch (nj) {
      FT_X_BLOCK(1); FT_X_BLOCK(2); FT_X_BLOCK(3); default: FT_X_BLOCK(4);
    }
  }
#undef FT_X_BLOCK
}

// Nontemporal stores (the nt bit), for large outputs that the caches cannot keep until their
// reader, a later kernel, runs: the lines are not retained on the way to memory.  Used where
// each store instruction fills whole 128-byte lines; Y_perm's stores (24 bytes per row per
// instruction) ran three times slower with it.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x3 __attribute__((ext_vector_type(3)));
__device__ __forceinline__ void st_nt(void* p, uint4 v) {
  __builtin_nontemporal_store((u32x4){v.x, v.y, v.z, v.w}, (u32x4*)p);
}

// Exact mode: the permuted x rows into the gate/up GEMM's token tiles (xtb).  One workgroup
// per 32-row group of padded permuted rows (its expert from the group map k_perm_scan wrote)
// and 8 chunks of 64 K: thread (t, p) reads 16 bytes, K 64 c + 8 p .. + 7 of the group's row t
// (eight threads read a row's 128-byte chunk contiguously) and writes them to tile
// (g, c, p % 4), lane t + 32 (p / 4); padding rows get zeros.  The grid covers the largest
// padded row count.
constexpr int kTileXChunks = 8;
__global__ __launch_bounds__(256) void k_tile_x(PrefillLaunch a) {
  const int g = blockIdx.x;
  if (g >= (a.poff[a.E] >> 5)) return;
  const int NC = a.H / 64;
  const int t = threadIdx.x >> 3, p = threadIdx.x & 7;
  const int e = a.tile_e[g];
  const int r = 32 * g + t - a.poff[e];
  const bool valid = r < a.counts[e];
  const uint16_t* xr =
      a.x + (uint64_t)a.perm_tok[a.offsets[e] + min(r, a.counts[e] - 1)] * a.H + 8 * p;
  const int c0 = blockIdx.y * kTileXChunks;
  uint4 v[kTileXChunks];
#pragma unroll
  for (int u = 0; u < kTileXChunks; ++u)
    v[u] = *(const uint4*)(xr + (uint64_t)min(c0 + u, NC - 1) * 64);
#pragma unroll
  for (int u = 0; u < kTileXChunks; ++u) {
    const int c = c0 + u;
    if (c < NC) {
      const uint64_t slot = (((uint64_t)g * NC + c) * 4 + (p & 3)) * 64 + t + 32 * (p >> 2);
      st_nt(a.xtb + slot * 8, valid ? v[u] : make_uint4(0u, 0u, 0u, 0u));
    }
  }
}

// y = 0 before the down GEMM's atomic combine (a kernel, not a memset node, so that the call
// can be captured into a graph).
__global__ __launch_bounds__(256) void k_zero(float* __restrict__ y, uint64_t n4) {
  const uint64_t i = (uint64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n4) st_nt((uint4*)y + i, make_uint4(0u, 0u, 0u, 0u));
}

// ---- scaled-FP4 mode (both MFMA operands FP4) ------------------------------------------------

// D (16 weight rows x 16 tokens) += A (16 x 128 E2M1, E8M0 scale sa per lane) * B (128 x 16
// E2M1, scale sb per lane).  Lane l holds row / column l % 16, K elements 32 (l / 16) .. +31:
// exactly one 16-byte slice of the tile layout and one MX block, so each lane's scale is the
// scale of its block.  The scale operands use their low byte.
__device__ __forceinline__ f32x4 mfma_fp4(const uint4& a, const uint4& b, f32x4 c, uint32_t sa,
                                          uint32_t sb) {
  const i32x8 av = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
  const i32x8 bv = {(int)b.x, (int)b.y, (int)b.z, (int)b.w, 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, c, 4, 4, 0, (int)sa, 0, (int)sb);
}

// D (32 weight rows x 32 tokens) += A (32 x 64 E2M1) * B (64 x 32 E2M1), scales per lane.
// Lane l holds row / column l % 32, K elements 32 (l / 32) .. +31 (one MX block, one scale);
// D element (8 (r / 4) + 4 (l / 32) + r % 4, l % 32) is in register r of lane l.  This shape
// runs at twice the rate of the 16x16x128 one on gfx950 (measured: 8.4 vs 4.3 PFLOP/s).
__device__ __forceinline__ f32x16 mfma_fp4_32(const uint4& a, const uint4& b, f32x16 c, uint32_t sa,
                                              uint32_t sb) {
  const i32x8 av = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
  const i32x8 bv = {(int)b.x, (int)b.y, (int)b.z, (int)b.w, 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, c, 4, 4, 0, (int)sa, 0, (int)sb);
}

// x (bf16 [T][H]) -> codes [T][H/2] + scales [T][H/32]; one thread per 32-value block.
__global__ __launch_bounds__(256) void k_quant_x(PrefillLaunch a) {
  const uint64_t nblk = (uint64_t)a.T * (a.H / 32);
  const uint64_t b = (uint64_t)blockIdx.x * 256 + threadIdx.x;
  if (b >= nblk) return;
  const uint4* src = (const uint4*)(a.x + b * 32);
  uint32_t w[16];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 v = src[i];
    w[4 * i] = v.x; w[4 * i + 1] = v.y; w[4 * i + 2] = v.z; w[4 * i + 3] = v.w;
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fmaxf(fabsf(bf16_lo(w[i])), fabsf(bf16_hi(w[i]))));
  const uint32_t sc = mx_scale_code(amax);
  const float inv = mx_inv_scale(sc);
  uint32_t out[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint32_t o = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t wi = w[4 * q + i];
      o |= mx_code(bf16_lo(wi), inv) << (8 * i);
      o |= mx_code(bf16_hi(wi), inv) << (8 * i + 4);
    }
    out[q] = o;
  }
  *(uint4*)(a.xq + b * 16) = make_uint4(out[0], out[1], out[2], out[3]);
  a.xqs[b] = (uint8_t)sc;
}

// Expert of padded permuted row p: poff[e] <= p < poff[e + 1] (wave-uniform callers).
__device__ __forceinline__ int expert_of(const int32_t* off, int E, int p) {
  int lo = 0, hi = E - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (off[mid] <= p) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Quantised token rows -> the GEMM's token operand in tile format, rows in permuted order
// padded per expert to a multiple of 16.  One workgroup per 16-row tile row (every such row
// belongs to one expert, from the tile map the scan wrote): the 16 rows' tokens are read
// once, then wave w writes K tiles w, w + 4, ... of the row (lane l: row l % 16, 32-K block
// 4 kc + l / 16), four tiles' loads in flight at a time.  Padding rows get zero codes and
// scales.  The grid covers the largest padded row count.
__global__ __launch_bounds__(256) void k_tile_xq(PrefillLaunch a) {
  const int KC = a.H / kTileK;
  const int trow = blockIdx.x;                    // 16-row tile row
  if (trow >= (a.poff[a.E] >> 4)) return;
  const int wave = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int e = a.tile_e[trow];
  const int r = trow * 16 + (l & 15) - a.poff[e];
  const bool valid = r < a.counts[e];
  const uint64_t t = valid ? (uint64_t)a.perm_tok[min(a.offsets[e] + r, a.T * a.k - 1)] : 0;
  for (int kc0 = wave; kc0 < KC; kc0 += 16) {
    uint4 c[4];
    uint8_t sc[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int kc = min(kc0 + 4 * u, KC - 1);
      const int blk = kc * 4 + (l >> 4);
      c[u] = *(const uint4*)(a.xq + t * (a.H / 2) + blk * 16);
      sc[u] = a.xqs[t * (a.H / 32) + blk];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int kc = kc0 + 4 * u;
      if (kc < KC) {
        const uint64_t tile = (uint64_t)trow * KC + kc;
        st_nt(a.xt + tile * 1024 + l * 16, valid ? c[u] : make_uint4(0u, 0u, 0u, 0u));
        a.xts[tile * 64 + l] = valid ? sc[u] : (uint8_t)0;
      }
    }
  }
}

// Test hook: the tiled h back to permuted row order, codes [T*k][I/2] and scales [T*k][I/32].
// One thread per (row, 32-value block).
__global__ __launch_bounds__(256) void k_untile_h(PrefillLaunch a, uint8_t* codes, uint8_t* scales) {
  const int nb = a.I / 32, KC = a.I / kTileK;
  const uint64_t gid = (uint64_t)blockIdx.x * 256 + threadIdx.x;
  if (gid >= (uint64_t)a.T * a.k * nb) return;
  const int p = (int)(gid / nb), u = (int)(gid % nb);
  const int e = expert_of(a.offsets, a.E, p);
  const int prow = a.poff[e] + p - a.offsets[e];
  const uint64_t tile = (uint64_t)(prow / 16) * KC + u / 4;
  const int slotl = (prow % 16) + 16 * (u % 4);
  *(uint4*)(codes + gid * 16) = *(const uint4*)(a.ht + tile * 1024 + slotl * 16);
  scales[gid] = a.hts[tile * 64 + slotl];
}

// NVFP4 blob -> MXFP4 blob of the same expert: every weight's exact value E2M1 x E4M3 x tensor
// scale (fp64: at most 8 + 24 significant bits) requantised by the OCP MX rule per 32 along K.
// A tile lane holds one 32-value K run of one row (two NVFP4 blocks), which is one MX block in
// the same lane of the same tile.  One thread per (matrix, tile, lane).
__device__ __forceinline__ double e2m1_f64(uint32_t c) {
  const double m = (c & 4) ? ((c & 2) ? ((c & 1) ? 6.0 : 4.0) : ((c & 1) ? 3.0 : 2.0))
                           : ((c & 2) ? ((c & 1) ? 1.5 : 1.0) : ((c & 1) ? 0.5 : 0.0));
  return (c & 8) ? -m : m;
}

__global__ __launch_bounds__(256) void k_nv_to_mx(const uint8_t* __restrict__ src,
                                                  uint8_t* __restrict__ dst, BlobLayout S,
                                                  BlobLayout D, uint64_t lanes_per_matrix) {
  const uint64_t gid = (uint64_t)blockIdx.x * 256 + threadIdx.x;
  if (gid == 0) {
    BlobHeader* h = (BlobHeader*)dst;
    h->magic = kBlobMagic;
    h->fmt = FT_MXFP4;
    h->H = D.H;
    h->I = D.I;
    for (int i = 0; i < 3; ++i) h->tensor_scale[i] = 1.0f;
    for (int i = 0; i < 9; ++i) h->reserved[i] = 0;
  }
  if (gid >= 3 * lanes_per_matrix) return;
  const int m = (int)(gid / lanes_per_matrix);
  const uint64_t tl = gid % lanes_per_matrix;     // tile * 64 + lane
  const double ts = (double)((const BlobHeader*)src)->tensor_scale[m];
  const uint4 c = *(const uint4*)(src + S.off[2 * m] + tl * 16);
  const uint8_t* sp = src + S.off[2 * m + 1] + (tl >> 6) * 128 + 2 * (tl & 63);
  const double s0 = (double)e4m3_f32(sp[0]) * ts, s1 = (double)e4m3_f32(sp[1]) * ts;
  const uint32_t cw[4] = {c.x, c.y, c.z, c.w};
  double v[32];
  double amax = 0.0;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    v[i] = e2m1_f64((cw[i >> 3] >> (4 * (i & 7))) & 15u) * (i < 16 ? s0 : s1);
    amax = fmax(amax, fabs(v[i]));
  }
  int sc = 0;
  if (amax > 0.0) {
    int ex;
    frexp(amax, &ex);                                 // amax = f 2^ex, f in [0.5, 1)
    sc = min(max(ex - 3, -127), 127) + 127;           // exponent floor(log2 amax) - 2
  }
  const double inv = ldexp(1.0, 127 - sc);
  uint32_t out[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const double r = fabs(v[i]) * inv;
    uint32_t q = (uint32_t)(r > 0.25) + (uint32_t)(r >= 0.75) + (uint32_t)(r > 1.25) +
                 (uint32_t)(r >= 1.75) + (uint32_t)(r > 2.5) + (uint32_t)(r >= 3.5) +
                 (uint32_t)(r > 5.0);
    if (signbit(v[i])) q |= 8u;
    out[i >> 3] |= q << (4 * (i & 7));
  }
  *(uint4*)(dst + D.off[2 * m] + tl * 16) = make_uint4(out[0], out[1], out[2], out[3]);
  dst[D.off[2 * m + 1] + tl] = (uint8_t)sc;
}

// Grouped GEMM on the scaled-FP4 MFMA.  MODE 0: gate/up + SwiGLU + MXFP4 quantise of h;
// MODE 1: down -> Y_perm.
//
// A workgroup owns 16 weight row tiles (MODE 0: 8 gate + the same 8 up tiles, 128 features;
// MODE 1: 16 row tiles of W_d, 256 outputs) and a block of up to 256 rows of one expert.  Its
// four waves split that 256 x 256 tile 2 x 2: wave (wm, wn) multiplies 128 weight rows (four
// 32-row operands) by the 32-token tiles wn, wn + 2, wn + 4, wn + 6 on the 32x32x64 MFMA
// (fp32 accumulators in the AGPRs); a 32-row operand is two 16-row tiles, read from LDS at
// the lane slots that hold its K half.  Per 128-K chunk,
// the 16 weight tiles (1 KB each, one per 16-row tile of the blob) and the 16 token tiles
// (1 KB each, 16 rows x 64 B in the tile layout k_tile_xq wrote) are copied global -> LDS by
// the DMA form of the buffer load, straight
// into MFMA operand order, so no register holds data in flight: four LDS stages give three
// chunks of loads in flight while the fourth is multiplied.  Each stage is its own LDS array,
// which lets the compiler see that reading one stage does not wait on the copies into
// another; each wave issues the same ten copies per chunk, so an explicit count wait
// followed by a barrier (no fence, which would drain every copy in flight) makes a stage
// visible to the whole workgroup.  Block (token block g, feature block fb) sits on XCD g % 8.

// The lane index, computed where it is used: volatile, so the compiler neither merges it with
// an earlier copy nor keeps one live across a loop.
__device__ __forceinline__ int lane_index_here() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

constexpr int kS1Stages = 4;
constexpr int kS1Copies = 10;   // copies per wave per chunk: 4 weight + 1 scale + 4 token + 1 scale

template <int MODE, bool FAST>
__global__ __launch_bounds__(256) void k_s1_gemm(PrefillLaunch a, int NB) {
  // stage s: weight and token codes [16 tiles][64 lanes], weight and token scales
  // [16 tiles][64 B]: the tile format throughout
  __shared__ uint4 wc0[1024], wc1[1024], wc2[1024], wc3[1024];
  __shared__ uint4 tc0[1024], tc1[1024], tc2[1024], tc3[1024];
  __shared__ uint32_t ws0[256], ws1[256], ws2[256], ws3[256];
  __shared__ uint32_t ts0[256], ts1[256], ts2[256], ts3[256];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int n = lane & 15, g = lane >> 4;
  const int KC = (MODE == 0 ? a.H : a.I) / kTileK;
  const int nrt = (MODE == 0 ? a.I : a.H) / kTileRows;   // row tiles of each matrix
  const uint8_t* tcodes = MODE == 0 ? a.xt : a.ht;
  const uint8_t* tscales = MODE == 0 ? a.xts : a.hts;
  const int tb_total = a.tb_off[a.E];
  // A block (token block gblk, feature block fb) has index Lb = 8 (NB (gblk / 8) + fb) +
  // gblk % 8, so its workgroup, and all of the token block's, sits on XCD gblk % 8 (the
  // token tiles stay in that L2).  The down GEMM's fast path is persistent: workgroup b takes
  // blocks b, b + grid, b + 2 grid, ... (grid a multiple of 8), whose token blocks only grow,
  // and the next block's first copies run during this block's epilogue.  (The gate/up GEMM
  // keeps one block per workgroup: carrying the next block's state through its epilogue
  // spills registers, and every reload there waits for the copies in flight.)
  constexpr bool PERSIST = FAST && MODE == 1;
#define FT_S1_BLOCK(Lb_, gblk_, fb_)                                                      \
  do {                                                                                    \
    const int jj_ = (Lb_) >> 3;                                                           \
    gblk_ = ((Lb_) & 7) + 8 * (jj_ / NB);                                                 \
    fb_ = jj_ % NB;                                                                       \
  } while (0)
  // the per-block scalars (expert from the block map k_perm_scan wrote; all uniform)
#define FT_S1_SCALARS(gblk_, fb_, e_, row0_, nrows_, nj_, ntile16_, ptile0_, wvalid_)        \
  do {                                                                                    \
    e_ = a.blk_e[gblk_];                                                                  \
    row0_ = a.offsets[e_] + ((gblk_) - a.tb_off[e_]) * kS1Rows;                           \
    nrows_ = min(kS1Rows, a.offsets[(e_) + 1] - (row0_));                                 \
    nj_ = max(0, ((((nrows_) + 31) >> 5) - wn + 1) >> 1);                                 \
    ntile16_ = ((nrows_) + 15) >> 4;                                                      \
    ptile0_ = (a.poff[e_] >> 4) + ((gblk_) - a.tb_off[e_]) * (kS1Rows / 16);              \
    wvalid_ = MODE == 0 || (fb_) * 16 + wm * 8 < nrt;                                     \
  } while (0)
  // this wave's copy sources, as buffer resources (base and extent) with scalar offsets per
  // copy, the chunk's offset added to them at issue: weight tiles wave + 4i of the expert's
  // blob and the scale dwords of tiles 4 wave .. + 3 (a lane offset); token tiles wave + 4i
  // and the scale dwords of rows 64 wave .. + 63 from resources spanning exactly the block's
  // tiles (rows past the block re-read its last row; MODE 1 row tiles past the matrix are
  // clamped, their results never stored).  Only the lane offsets (16 lane and the two scale
  // offsets) sit in vector registers.
#define FT_S1_SOURCES(e_, fb_, ntile16_, ptile0_)                                         \
  do {                                                                                    \
    wres = __builtin_amdgcn_make_buffer_rsrc((void*)(a.mxpool + (uint64_t)(e_) * a.mxstride), \
                                             (short)0, (int)a.ML.bytes, kBufFlags);       \
    _Pragma("unroll") for (int i_ = 0; i_ < 4; ++i_) {                                    \
      const int q_ = wave + 4 * i_;                                                       \
      const int m_ = MODE == 0 ? (q_ < 8 ? 0 : 1) : 2;                                    \
      const int rt_ = min(MODE == 0 ? (fb_) * 8 + (q_ & 7) : (fb_) * 16 + q_, nrt - 1);   \
      wso[i_] = __builtin_amdgcn_readfirstlane(                                           \
          (uint32_t)(a.ML.off[2 * m_] + (uint64_t)rt_ * KC * kTileCodeBytes));            \
    }                                                                                     \
    {                                                                                     \
      const int q_ = 4 * wave + (lane >> 4);                                              \
      const int m_ = MODE == 0 ? (q_ < 8 ? 0 : 1) : 2;                                    \
      const int rt_ = min(MODE == 0 ? (fb_) * 8 + (q_ & 7) : (fb_) * 16 + q_, nrt - 1);   \
      wsv = (uint32_t)(a.ML.off[2 * m_ + 1] + (uint64_t)rt_ * KC * 64) + 4 * (lane & 15); \
    }                                                                                     \
    const uint64_t tb_ = (uint64_t)(ptile0_) * KC;                                        \
    tres = __builtin_amdgcn_make_buffer_rsrc((void*)(tcodes + tb_ * kTileCodeBytes),      \
                                             (short)0, (ntile16_) * KC * kTileCodeBytes,  \
                                             kBufFlags);                                  \
    tsres = __builtin_amdgcn_make_buffer_rsrc((void*)(tscales + tb_ * 64), (short)0,      \
                                              (ntile16_) * KC * 64, kBufFlags);           \
    _Pragma("unroll") for (int i_ = 0; i_ < 4; ++i_)                                      \
      tso[i_] = __builtin_amdgcn_readfirstlane(                                           \
          (uint32_t)(min(wave + 4 * i_, (ntile16_) - 1) * KC * kTileCodeBytes));          \
    tsv = (uint32_t)(min(4 * wave + (lane >> 4), (ntile16_) - 1) * KC * 64) + 4 * (lane & 15); \
  } while (0)

  int Lb = blockIdx.x, gblk, fb;
  FT_S1_BLOCK(Lb, gblk, fb);
  if (gblk >= tb_total) return;
  int e, row0, nrows, nj, ntile16, ptile0;
  bool wvalid;
  FT_S1_SCALARS(gblk, fb, e, row0, nrows, nj, ntile16, ptile0, wvalid);
  __amdgpu_buffer_rsrc_t wres, tres, tsres;
  uint32_t wso[4], tso[4], wsv, tsv;
  const uint32_t lo16 = 16 * lane;
  FT_S1_SOURCES(e, fb, ntile16, ptile0);

  f32x16 acc[4][4];

  // first stage tile of this wave's 32-row operand o: MODE 0 gate features wm * 64 + 32 o
  // (o = 0, 1) and the same up features (o = 2, 3); MODE 1 rows wm * 128 + 32 o
  auto otile = [&](int o) {
    return MODE == 0 ? (o < 2 ? 4 * wm + 2 * o : 8 + 4 * wm + 2 * (o - 2)) : 8 * wm + 2 * o;
  };
  // lane slot of a 16-row tile holding this lane's 32 K values of K half kh: row lane % 16
  // of tile (lane / 16) % 2 of the pair, K group 2 kh + lane / 32
  const int hi = (lane >> 4) & 1, h = lane >> 5;
  auto slot = [&](int kh) { return (lane & 15) + 16 * (2 * kh + h); };

#define FT_S1_ISSUE(kc_, WC_, TC_, WS_, TS_)                                              \
  do {                                                                                    \
    const uint32_t c_ = (uint32_t)((kc_) < KC ? (kc_) : (nxt ? (kc_) - KC : KC - 1));     \
    _Pragma("unroll") for (int i_ = 0; i_ < 4; ++i_)                                      \
      if (MODE == 1)                                                                      \
        bdma16_nt(wres, lo16, __builtin_amdgcn_readfirstlane(wso[i_] + c_ * kTileCodeBytes), \
                  &WC_[(wave + 4 * i_) * 64]);                                            \
      else                                                                                \
        bdma16(wres, lo16, __builtin_amdgcn_readfirstlane(wso[i_] + c_ * kTileCodeBytes), \
               &WC_[(wave + 4 * i_) * 64]);                                               \
    bdma4(wres, wsv, c_ * 64, &WS_[64 * wave]);                                           \
    _Pragma("unroll") for (int i_ = 0; i_ < 4; ++i_)                                      \
      bdma16(tres, lo16, __builtin_amdgcn_readfirstlane(tso[i_] + c_ * kTileCodeBytes),   \
             &TC_[(wave + 4 * i_) * 64]);                                                 \
    bdma4(tsres, tsv, c_ * 64, &TS_[64 * wave]);                                          \
  } while (0)

  // Operands are double-buffered in registers: step kc reads chunk kc's operands from its
  // stage while the MFMAs of chunk kc - 1 (read one step earlier) run, so the LDS reads hide
  // behind the matrix cores.
  uint4 PA0[4][2], PB0[4][2], PA1[4][2], PB1[4][2];
  uint32_t pa0[4][2], pb0[4][2], pa1[4][2], pb1[4][2];

#define FT_S1_READ(WC_, TC_, WS_, TS_, A_, B_, SA_, SB_)                                   \
  do {                                                                                    \
    const uint8_t* wsb_ = (const uint8_t*)WS_;                                            \
    const uint8_t* tsb_ = (const uint8_t*)TS_;                                            \
    _Pragma("unroll") for (int kh_ = 0; kh_ < 2; ++kh_) {                                 \
      _Pragma("unroll") for (int o_ = 0; o_ < 4; ++o_) {                                  \
        const int t_ = otile(o_) + hi;                                                    \
        A_[o_][kh_] = WC_[t_ * 64 + slot(kh_)];                                           \
        SA_[o_][kh_] = wsb_[t_ * 64 + slot(kh_)];                                         \
      }                                                                                   \
      _Pragma("unroll") for (int i_ = 0; i_ < 4; ++i_) {                                  \
        const int J_ = wn + 2 * i_;                                                       \
        B_[i_][kh_] = TC_[(2 * J_ + hi) * 64 + slot(kh_)];                                \
        SB_[i_][kh_] = tsb_[(2 * J_ + hi) * 64 + slot(kh_)];                              \
      }                                                                                   \
    }                                                                                     \
  } while (0)
#define FT_S1_MFMA(A_, B_, SA_, SB_)                                                      \
  do {                                                                                    \
    _Pragma("unroll") for (int kh_ = 0; kh_ < 2; ++kh_)                                   \
      _Pragma("unroll") for (int i_ = 0; i_ < 4; ++i_) {                                  \
        if (FAST || i_ < nj) {                                                            \
          _Pragma("unroll") for (int o_ = 0; o_ < 4; ++o_)                                \
            acc[o_][i_] = mfma_fp4_32(A_[o_][kh_], B_[i_][kh_], acc[o_][i_],              \
                                      SA_[o_][kh_], SB_[i_][kh_]);                        \
        }                                                                                 \
      }                                                                                   \
  } while (0)
#define FT_S1_SYNC()                                                                      \
  do {                                                                                    \
    __builtin_amdgcn_s_waitcnt(FT_VMCNT(kS1Copies * (kS1Stages - 2)) & ~(15 << 8));       \
    asm volatile("" ::: "memory");                                                        \
    __builtin_amdgcn_s_barrier();                                                         \
    asm volatile("" ::: "memory");                                                        \
  } while (0)

  // step kc: this wave's LDS reads of every earlier stage have completed (lgkmcnt 0) and at
  // most the copies of the two later chunks are in flight, so its copies for chunk kc have
  // landed; the barrier extends both to all waves.  Then the stage of chunk kc - 1 (no longer
  // read by anyone) is refilled with chunk kc + 3, chunk kc's operands are read and chunk
  // kc - 1 is multiplied.
#define FT_S1_STEP(kc_, WC_, TC_, WS_, TS_, WCN_, TCN_, WSN_, TSN_, RA_, RB_, RSA_, RSB_,     \
                   CA_, CB_, CSA_, CSB_)                                                  \
  do {                                                                                    \
    __builtin_amdgcn_s_waitcnt(FT_VMCNT(kS1Copies * (kS1Stages - 2)) & ~(15 << 8));       \
    asm volatile("" ::: "memory");                                                        \
    __builtin_amdgcn_s_barrier();                                                         \
    asm volatile("" ::: "memory");                                                        \
    FT_S1_ISSUE((kc_) + kS1Stages - 1, WCN_, TCN_, WSN_, TSN_);                           \
    if ((kc_) < KC && wvalid) FT_S1_READ(WC_, TC_, WS_, TS_, RA_, RB_, RSA_, RSB_);       \
    if ((kc_) >= 1 && (kc_) - 1 < KC && wvalid) FT_S1_MFMA(CA_, CB_, CSA_, CSB_);         \
  } while (0)

  bool nxt = false;   // the next block's first chunks go out in the last four steps
  FT_S1_ISSUE(0, wc0, tc0, ws0, ts0);
  FT_S1_ISSUE(1, wc1, tc1, ws1, ts1);
  FT_S1_ISSUE(2, wc2, tc2, ws2, ts2);
  if (FAST) {
    FT_S1_SYNC();
    FT_S1_ISSUE(3, wc3, tc3, ws3, ts3);
    FT_S1_READ(wc0, tc0, ws0, ts0, PA0, PB0, pa0, pb0);
  }
  for (;;) {
#pragma unroll
    for (int o = 0; o < 4; ++o)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[o][i][r] = 0.f;
    int n_gblk = 0, n_fb = 0, n_e = 0, n_row0 = 0, n_nrows = 0, n_nj = 0, n_ntile16 = 0;
    int n_ptile0 = 0;
    bool n_wvalid = false;
    if (FAST) {
      // KC % 4 == 0: steps 1 .. KC each read one chunk and multiply the one before, on all
      // four token tiles (tiles past the block hold valid rows whose results are never
      // stored; the barrier makes every wave wait for the busiest one anyway).  No step has a
      // branch, so the accumulators never pass through a control-flow join.  The next
      // block's scalars are loaded here (scalar loads, long before they are needed); its
      // copy sources replace this block's in the last iteration, whose four steps issue its
      // chunks 0 .. 3 into stages 0 .. 3, just as this block's chunks KC .. KC + 3 would go.
      if (PERSIST) {
        const int Lb2 = Lb + (int)gridDim.x;
        FT_S1_BLOCK(Lb2, n_gblk, n_fb);
        nxt = n_gblk < tb_total;
        if (nxt)
          FT_S1_SCALARS(n_gblk, n_fb, n_e, n_row0, n_nrows, n_nj, n_ntile16, n_ptile0, n_wvalid);
      }
      // after the barrier the matrix core starts at once: the first 16 of this chunk's 32
      // MFMAs each carry one of the wave's copies (the first kS1Copies) and two of its LDS
      // reads of the next chunk's operands into the other register set (scheduling groups),
      // so the copy and read issue hides behind the MFMAs instead of preceding them
#define FT_S1_FAST_STEP(kcn_, WCN_, TCN_, WSN_, TSN_, WC_, TC_, WS_, TS_, RA_, RB_, RSA_, RSB_, \
                        CA_, CB_, CSA_, CSB_)                                               \
      do {                                                                                \
        FT_S1_SYNC();                                                                     \
        FT_S1_ISSUE(kcn_, WCN_, TCN_, WSN_, TSN_);                                        \
        FT_S1_READ(WC_, TC_, WS_, TS_, RA_, RB_, RSA_, RSB_);                             \
        FT_S1_MFMA(CA_, CB_, CSA_, CSB_);                                                 \
        _Pragma("unroll") for (int g_ = 0; g_ < kS1Copies; ++g_) {                        \
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                              \
          __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);                              \
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);                              \
        }                                                                                 \
        _Pragma("unroll") for (int g_ = 0; g_ < 16 - kS1Copies; ++g_) {                   \
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                              \
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);                              \
        }                                                                                 \
        __builtin_amdgcn_sched_barrier(0);                                                \
      } while (0)
      for (int kc = 1; kc <= KC; kc += kS1Stages) {
        if (PERSIST && nxt && kc + kS1Stages - 1 >= KC) {
          // an opaque zero keeps the address arithmetic here instead of hoisted out of the
          // loop, where its registers would stay live through every step
          int z_;
          asm volatile("s_mov_b32 %0, 0" : "=s"(z_));
          FT_S1_SOURCES(n_e + z_, n_fb + z_, n_ntile16, n_ptile0 + z_);
        }
        FT_S1_FAST_STEP(kc + 3, wc0, tc0, ws0, ts0, wc1, tc1, ws1, ts1, PA1, PB1, pa1, pb1, PA0, PB0, pa0, pb0);
        FT_S1_FAST_STEP(kc + 4, wc1, tc1, ws1, ts1, wc2, tc2, ws2, ts2, PA0, PB0, pa0, pb0, PA1, PB1, pa1, pb1);
        FT_S1_FAST_STEP(kc + 5, wc2, tc2, ws2, ts2, wc3, tc3, ws3, ts3, PA1, PB1, pa1, pb1, PA0, PB0, pa0, pb0);
        FT_S1_FAST_STEP(kc + 6, wc3, tc3, ws3, ts3, wc0, tc0, ws0, ts0, PA0, PB0, pa0, pb0, PA1, PB1, pa1, pb1);
      }
#undef FT_S1_FAST_STEP
    } else {
      for (int kc = 0; kc < KC; kc += kS1Stages) {
        FT_S1_STEP(kc, wc0, tc0, ws0, ts0, wc3, tc3, ws3, ts3, PA0, PB0, pa0, pb0, PA1, PB1, pa1, pb1);
        FT_S1_STEP(kc + 1, wc1, tc1, ws1, ts1, wc0, tc0, ws0, ts0, PA1, PB1, pa1, pb1, PA0, PB0, pa0, pb0);
        FT_S1_STEP(kc + 2, wc2, tc2, ws2, ts2, wc1, tc1, ws1, ts1, PA0, PB0, pa0, pb0, PA1, PB1, pa1, pb1);
        FT_S1_STEP(kc + 3, wc3, tc3, ws3, ts3, wc2, tc2, ws2, ts2, PA1, PB1, pa1, pb1, PA0, PB0, pa0, pb0);
      }
      // the last chunk's MFMAs: when KC % 4 == 0 its operands (odd chunk) are in set 1;
      // otherwise the loop's padding steps already ran them
      if (KC % kS1Stages == 0 && wvalid) FT_S1_MFMA(PA1, PB1, pa1, pb1);
    }
    // without a next block, the trailing copies (clamped re-reads) land before the
    // workgroup's LDS is released; with one, they are its first chunks, left in flight
    if (!nxt) __builtin_amdgcn_s_waitcnt(FT_VMCNT(0));

    if (wvalid) {
  if (MODE == 0) {
    // h = silu(G) * U for the 32 features of operand pair (o, o + 2) and token lane % 32: one MX
    // block, held by lanes l and l ^ 32 (features 8q + 4h + r in register 4q + r).  The lane
    // index is recomputed rather than kept across the main loop.
    const int lane_e = lane_index_here();
    const int h = lane_e >> 5;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (i >= nj) continue;
      const int row = 32 * (wn + 2 * i) + (lane_e & 31);
#pragma unroll
      for (int o = 0; o < 2; ++o) {
        float hv[16];
        float amax = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          hv[r] = silu_fast(acc[o][i][r]) * acc[o + 2][i][r];
          amax = fmaxf(amax, fabsf(hv[r]));
        }
        amax = fmaxf(amax, __uint_as_float(xor_lane<32>(__float_as_uint(amax))));
        const uint32_t sc = mx_scale_code(amax);
        // the hardware convert rounds v / 2^(sc - 127) to E2M1 exactly as the OCP rule does
        // (nearest, ties to the even code, saturating, sign kept; checked on gfx950 over every
        // rounding midpoint and its neighbours, zeros of both signs and subnormal scales).
        // w01 holds features 4h + {0..3, 8..11} (regs 0..7), w23 regs 8..15: as 16-bit pieces
        // p[q] = features 8q + 4h .. + 3 = block bytes 4q + 2h, 4q + 2h + 1
        const float scl = e8m0_f32(sc);
        uint32_t w01 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, hv[0], hv[1], scl, 0);
        w01 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w01, hv[2], hv[3], scl, 1);
        w01 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w01, hv[4], hv[5], scl, 2);
        w01 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w01, hv[6], hv[7], scl, 3);
        uint32_t w23 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, hv[8], hv[9], scl, 0);
        w23 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w23, hv[10], hv[11], scl, 1);
        w23 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w23, hv[12], hv[13], scl, 2);
        w23 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w23, hv[14], hv[15], scl, 3);
        // lane half 0 writes block bytes 0..7, half 1 bytes 8..15; each sends the pieces the
        // other half writes
        const uint32_t send = h == 0 ? w23 : w01;
        const uint32_t recv = xor_lane<32>(send);
        const uint2 out = h == 0 ? make_uint2((w01 & 0xffffu) | (recv << 16),
                                              (w01 >> 16) | (recv & 0xffff0000u))
                                 : make_uint2((recv & 0xffffu) | (w23 << 16),
                                              (recv >> 16) | (w23 & 0xffff0000u));
        // into the tiled h: padded row ptile0 * 16 + row, 32-K block 4 fb + 2 wm + o of the
        // down projection's K = I (rows past nrows hold h of zero tokens: zero codes)
        if (row < 16 * ntile16) {
          const int prow = ptile0 * 16 + row;
          const uint64_t tile = (uint64_t)(prow >> 4) * (a.I / kTileK) + fb;
          const int sl = (prow & 15) + 16 * (2 * wm + o);
          *(uint2*)(a.ht + tile * kTileCodeBytes + sl * 16 + 8 * h) = out;
          if (h == 0) a.hts[tile * 64 + sl] = (uint8_t)sc;
        }
      }
    }
  } else {
    // the lane index recomputed here, so no lane value is kept live (or spilled) across the
    // main loop
    const int lane_e = lane_index_here();
    const int h_e = lane_e >> 5;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (i >= nj) continue;
      const int row = 32 * (wn + 2 * i) + (lane_e & 31);
      if (row < nrows) {
#pragma unroll
        for (int o = 0; o < 4; ++o)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int col = fb * 256 + wm * 128 + 32 * o + 8 * q + 4 * h_e;
            *(uint3*)((uint8_t*)a.Yperm + ((uint64_t)(row0 + row) * a.H + col) * 3) =
                pack_f24x4(acc[o][i][4 * q], acc[o][i][4 * q + 1], acc[o][i][4 * q + 2],
                           acc[o][i][4 * q + 3]);
          }
      }
    }
  }
    }   // wvalid
    if (!nxt) break;
    Lb += (int)gridDim.x;
    gblk = n_gblk; fb = n_fb; e = n_e; row0 = n_row0; nrows = n_nrows; nj = n_nj;
    ntile16 = n_ntile16; ptile0 = n_ptile0; wvalid = n_wvalid;
    // recomputed rather than carried through the epilogue (registers)
    FT_S1_SOURCES(e, fb, ntile16, ptile0);
    // the epilogue's stores and the next block's copies share the count, and loads and
    // stores need not complete in issue order: wait for all of them, then read chunk 0 (it
    // landed, for every wave, at the last step's barrier)
    __builtin_amdgcn_s_waitcnt(FT_VMCNT(0));
    asm volatile("" ::: "memory");
    FT_S1_READ(wc0, tc0, ws0, ts0, PA0, PB0, pa0, pb0);
  }
#undef FT_S1_STEP
#undef FT_S1_SYNC
#undef FT_S1_MFMA
#undef FT_S1_READ
#undef FT_S1_ISSUE
#undef FT_S1_SOURCES
#undef FT_S1_SCALARS
#undef FT_S1_BLOCK
}

// y[t][h] = sum_j w[t][j] Y_perm[pos[t][j]][h], j in rank order; four h per thread.  KMAX
// (>= k) bounds the rows loaded, all issued before the first is used.  F24: Y_perm holds
// 24-bit floats (the scaled-FP4 mode), else fp32.
template <int KMAX, bool F24>
__global__ __launch_bounds__(256) void k_unpermute(PrefillLaunch a) {
  const int t = blockIdx.y;
  const int h = (blockIdx.x * 256 + threadIdx.x) * 4;
  if (h >= a.H) return;
  float4 v[KMAX];
  float wj[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    const int jc = min(j, a.k - 1);
    const int p = a.pos[(uint64_t)t * a.k + jc];
    wj[j] = a.w[(uint64_t)t * a.k + jc];
    if (F24) {
      // read once: nontemporal loads
      const u32x3 q = __builtin_nontemporal_load(
          (const u32x3*)((const uint8_t*)a.Yperm + ((uint64_t)p * a.H + h) * 3));
      v[j] = unpack_f24x4(make_uint3(q.x, q.y, q.z));
    } else {
      v[j] = *(const float4*)(a.Yperm + (uint64_t)p * a.H + h);
    }
  }
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    if (j < a.k) {
      acc.x = fmaf(wj[j], v[j].x, acc.x);
      acc.y = fmaf(wj[j], v[j].y, acc.y);
      acc.z = fmaf(wj[j], v[j].z, acc.z);
      acc.w = fmaf(wj[j], v[j].w, acc.w);
    }
  }
  *(float4*)(a.y + (uint64_t)t * a.H + h) = acc;
}

}  // namespace ft

// ---- launchers ----------------------------------------------------------------------------
using namespace ft;

extern "C" int ftk_split_router(const float* wr, int E, int H, uint16_t* planes, hipStream_t st) {
  const uint64_t n = (uint64_t)router_expert_tiles(E) * (H / 16) * 64;
  hipLaunchKernelGGL(k_split_router, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, wr, E,
                     H, planes);
  return (int)hipGetLastError();
}

#define FT_PLAUNCH_NT(kern, grid, nt, evs, eve, ...)                                       \
  do {                                                                                     \
    auto* kfn_ = kern;                                                                     \
    if (evs) hipExtLaunchKernelGGL(kfn_, grid, dim3(nt), 0, st, evs, eve, 0, __VA_ARGS__);  \
    else hipLaunchKernelGGL(kfn_, grid, dim3(nt), 0, st, __VA_ARGS__);                     \
  } while (0)
#define FT_PLAUNCH(kern, grid, evs, eve, ...) FT_PLAUNCH_NT(kern, grid, 256, evs, eve, __VA_ARGS__)

// ev: null or 4 events (gate/up start, stop, down start, stop).
// Workgroups of a persistent S1 kernel: the device's resident count, rounded down to a
// multiple of 8 (at least 8).
static int s1_slots(const void* kern) {
  int dev = 0, per_cu = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, 256, 0) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 256;
  return std::max(8, per_cu * cus / 8 * 8);
}

extern "C" int ftk_prefill(const PrefillLaunch* ap, hipStream_t st, const hipEvent_t* ev) {
  const PrefillLaunch& a = *ap;
  const int nblk = (a.T + kPermBlock - 1) / kPermBlock;
  {
    const int NTe = router_expert_tiles(a.E);
    const int NT = min(NTe, kRouterGroupTiles);
    const dim3 rg((a.T + kRouterTokens - 1) / kRouterTokens, a.splits,
                  (NTe + kRouterGroupTiles - 1) / kRouterGroupTiles);
    const bool fast = ((a.H / a.splits) / 32) % 4 == 0;
#define FT_RT_LAUNCH(N)                                                                      \
  if (fast) hipLaunchKernelGGL((k_router_prefill<N, true>), rg, dim3(256), 0, st, a);        \
  else hipLaunchKernelGGL((k_router_prefill<N, false>), rg, dim3(256), 0, st, a)
    switch (NT) {
      case 1: FT_RT_LAUNCH(1); break;
      case 2: FT_RT_LAUNCH(2); break;
      case 3: FT_RT_LAUNCH(3); break;
      case 4: FT_RT_LAUNCH(4); break;
      case 5: FT_RT_LAUNCH(5); break;
      default: FT_RT_LAUNCH(6); break;
    }
#undef FT_RT_LAUNCH
  }
  const dim3 tg((a.T + kTopkTokens - 1) / kTopkTokens);
#define FT_TK_ARGS a.logits, a.splits, a.router_b, a.T, a.E, a.k, a.idx, a.w
  if (a.E <= 64) hipLaunchKernelGGL(k_topk_many<1>, tg, dim3(256), 0, st, FT_TK_ARGS);
  else if (a.E <= 128) hipLaunchKernelGGL(k_topk_many<2>, tg, dim3(256), 0, st, FT_TK_ARGS);
  else if (a.E <= 256) hipLaunchKernelGGL(k_topk_many<4>, tg, dim3(256), 0, st, FT_TK_ARGS);
  else hipLaunchKernelGGL(k_topk_many<16>, tg, dim3(256), 0, st, FT_TK_ARGS);
#undef FT_TK_ARGS
  if (a.mode == FT_PREFILL_MXFP4) {
    const uint64_t nq = (uint64_t)a.T * (a.H / 32);
    hipLaunchKernelGGL(k_quant_x, dim3((unsigned)((nq + 255) / 256)), dim3(256), 0, st, a);
  }
  hipLaunchKernelGGL(k_perm_masks, dim3(nblk), dim3(256), 0, st, a);
  hipLaunchKernelGGL(k_perm_scan, dim3(1), dim3(256), 0, st, a);
  if (a.k <= 8) hipLaunchKernelGGL(k_perm_place<8>, dim3(nblk), dim3(256), 0, st, a);
  else hipLaunchKernelGGL(k_perm_place<FT_MAX_TOPK>, dim3(nblk), dim3(256), 0, st, a);
  if (a.mode == FT_PREFILL_MXFP4) {
    // tiles of the padded permuted tokens: at most T*k + 15 E rows
    const unsigned maxtrows = (unsigned)((a.T * a.k + 15 * a.E + 15) / 16);
    hipLaunchKernelGGL(k_tile_xq, dim3(maxtrows), dim3(256), 0, st, a);
  } else {
    // at most T*k + 31 E padded rows, 32 per group
    const unsigned groups = (unsigned)((a.T * a.k + 31 * a.E + 31) / 32);
    const unsigned cg = (unsigned)((a.H / 64 + kTileXChunks - 1) / kTileXChunks);
    hipLaunchKernelGGL(k_tile_x, dim3(groups, cg), dim3(256), 0, st, a);
  }
  // upper bound on mrows-row token blocks: sum_e ceil(c_e / mrows) <= T*k/mrows + E
  const int gmax = (a.T * a.k + a.mrows - 1) / a.mrows + a.E;
  const int g8 = (gmax + 7) / 8 * 8;
  hipEvent_t e0 = ev ? ev[0] : nullptr, e1 = ev ? ev[1] : nullptr;
  hipEvent_t e2 = ev ? ev[2] : nullptr, e3 = ev ? ev[3] : nullptr;
  if (a.mode == FT_PREFILL_MXFP4) {
    const int sb0 = a.I / 128, sb1 = (a.H + 255) / 256;   // feature blocks
    // The branch-free main loop needs the chunk count to be a multiple of the stage count.
    // The down GEMM's is persistent, one workgroup per resident slot (a multiple of 8, so
    // every workgroup keeps to one XCD); the others take one block per workgroup.
    if ((a.H / kTileK) % kS1Stages == 0)
      FT_PLAUNCH((k_s1_gemm<0, true>), dim3(g8 * sb0), e0, e1, a, sb0);
    else FT_PLAUNCH((k_s1_gemm<0, false>), dim3(g8 * sb0), e0, e1, a, sb0);
    const int slots = s1_slots((const void*)k_s1_gemm<1, true>);
    if ((a.I / kTileK) % kS1Stages == 0)
      FT_PLAUNCH((k_s1_gemm<1, true>), dim3(std::min(g8 * sb1, slots)), e2, e3, a, sb1);
    else FT_PLAUNCH((k_s1_gemm<1, false>), dim3(g8 * sb1), e2, e3, a, sb1);
    const dim3 ug((a.H / 4 + 255) / 256, a.T);
    if (a.k <= 8) hipLaunchKernelGGL((k_unpermute<8, true>), ug, dim3(256), 0, st, a);
    else hipLaunchKernelGGL((k_unpermute<FT_MAX_TOPK, true>), ug, dim3(256), 0, st, a);
  } else {
    // exact mode: gate/up + SwiGLU into h, then down with the combine folded into its
    // epilogue (atomic adds into y, zeroed first)
    const uint64_t n4 = (uint64_t)a.T * a.H / 4;
    hipLaunchKernelGGL(k_zero, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, st, a.y, n4);
    const int nb0 = a.I / 128, nb1 = (a.H + 255) / 256;
    if (a.L.fmt == FT_MXFP4) {
      FT_PLAUNCH_NT((k_xgemm<0, FT_MXFP4>), dim3(g8 * nb0), kXThreads, e0, e1, a, nb0);
      FT_PLAUNCH_NT((k_xgemm<1, FT_MXFP4>), dim3(g8 * nb1), kXThreads, e2, e3, a, nb1);
    } else {
      FT_PLAUNCH_NT((k_xgemm<0, FT_NVFP4>), dim3(g8 * nb0), kXThreads, e0, e1, a, nb0);
      FT_PLAUNCH_NT((k_xgemm<1, FT_NVFP4>), dim3(g8 * nb1), kXThreads, e2, e3, a, nb1);
    }
  }
  return (int)hipGetLastError();
}

// NVFP4 blob -> MXFP4 blob (layouts S and D of the same H, I).
extern "C" int ftk_nv_to_mx(const uint8_t* src, uint8_t* dst, const BlobLayout* S,
                            const BlobLayout* D, hipStream_t st) {
  const uint64_t lanes = (uint64_t)(S->I / kTileRows) * (S->H / kTileK) * 64;  // per matrix
  const uint64_t n = 3 * lanes;
  hipLaunchKernelGGL(k_nv_to_mx, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, src, dst,
                     *S, *D, lanes);
  return (int)hipGetLastError();
}

// Test hook: the last MXFP4-mode call's h in permuted row order.
extern "C" int ftk_untile_h(const PrefillLaunch* ap, uint8_t* codes, uint8_t* scales, hipStream_t st) {
  const PrefillLaunch& a = *ap;
  const uint64_t n = (uint64_t)a.T * a.k * (a.I / 32);
  hipLaunchKernelGGL(k_untile_h, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, a, codes, scales);
  return (int)hipGetLastError();
}
