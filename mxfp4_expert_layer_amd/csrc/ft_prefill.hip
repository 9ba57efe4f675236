// Prefill kernels of libft for gfx950 (CDNA4).
//
// Prefill and decode get separate strategies (smzdm explainer aomxznrn, "FreeToken干的事",
// item 4): prefill is compute-bound, so the (token, expert) pairs are sorted by expert and
// each expert's tokens go through one grouped GEMM on the matrix cores.  One call of T
// tokens through an all-resident layer runs, on the caller's stream:
//   k_router_prefill  logits = x W_r^T + b: the fp32 router weights are held as three bf16
//                     planes whose sum is exactly W_r (24 = 3 x 8 significant bits), so the
//                     16x16x32 bf16 MFMA forms exact products with fp32 accumulation.
//   k_topk_many       per-token top-k + softmax (the decode routine, 16 tokens a workgroup).
//   k_perm_masks      per 256-token block: a token bitmask per expert (LDS atomics).
//   k_perm_scan       counts, offsets (exclusive scan), per-block bases, 128-row block map.
//   k_perm_place      pos[t][j] = base + (tokens below t in the block's mask); the row of
//                     every pair, expert ascending then token ascending (stable).
//   k_ggemm<0>        per (expert, 128-token block, 64 gate + 64 up features): G, U on the
//                     bf16 MFMA with NVFP4 weights decoded to bf16 in LDS (E2M1 x E4M3 has at
//                     most 6 significant bits, so the decode is exact; the fp32 tensor scale
//                     is applied in the epilogue), h = bf16(silu(ts_g G) * (ts_u U)).
//   k_ggemm<1>        per (expert, token block, 128 rows of W_d): Y_perm = ts_d (W_d h).
//   k_unpermute       y[t] = sum_j w[t][j] Y_perm[pos[t][j]].
// The scaled-FP4 mode replaces the two GEMMs (both operands FP4):
//   k_quant_x         x -> MXFP4 per 32 along H (OCP MX rule), once per token.
//   k_s1_gemm<0>      per (expert, 256-row block, 64 gate + 64 up features): G, U on the
//                     16x16x128 scaled-FP4 MFMA; h = silu(G) * U quantised to MXFP4 per 32
//                     features in the epilogue.
//   k_s1_gemm<1>      per (expert, row block, 128 rows of W_d): Y_perm = W_d h.
// and its NVFP4 weights come from k_nv_to_mx, run once when the layer is created.
// Workgroups of one kernel never wait on each other.
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>

#include "ft_device.h"

namespace ft {

constexpr int kRouterTokens = 64;    // tokens per router workgroup (16 per wave)
constexpr int kRouterExperts = 32;   // experts per router workgroup (two 16-row tiles)

// ---- router ------------------------------------------------------------------------------
// planes[p][i] (bf16): w = planes0 + planes1 + planes2 exactly (each plane takes the next 8
// significant bits by truncation; the remainders are exact in fp32).
__global__ __launch_bounds__(256) void k_split_router(const float* __restrict__ wr, int n,
                                                      uint16_t* __restrict__ planes) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const float w = wr[i];
  const uint32_t p0 = __float_as_uint(w) & 0xffff0000u;
  const float r1 = w - __uint_as_float(p0);
  const uint32_t p1 = __float_as_uint(r1) & 0xffff0000u;
  const float r2 = r1 - __uint_as_float(p1);
  const uint32_t p2 = __float_as_uint(r2) & 0xffff0000u;
  planes[i] = (uint16_t)(p0 >> 16);
  planes[(uint64_t)n + i] = (uint16_t)(p1 >> 16);
  planes[2 * (uint64_t)n + i] = (uint16_t)(p2 >> 16);
}

// Grid (ceil(T/64), ceil(E/32)).  Experts are the MFMA rows (A, staged in LDS per 128-K
// chunk in operand order), tokens the columns (B, loaded per lane from x).
__global__ __launch_bounds__(256) void k_router_prefill(PrefillLaunch a) {
  __shared__ uint4 wl[3][2][4][64];  // [plane][expert tile][k-step][lane]  24 KB
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int n = lane & 15, g = lane >> 4;
  const int t0 = blockIdx.x * kRouterTokens + wave * 16;
  const int e0 = blockIdx.y * kRouterExperts;
  const int tok = min(t0 + n, a.T - 1);
  const uint16_t* xr = a.x + (uint64_t)tok * a.H + 32 * g;
  const uint64_t plane = (uint64_t)a.E * a.H;
  f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
  const int KC = a.H / kTileK;
  for (int kc = 0; kc < KC; ++kc) {
    // stage: 3 planes x 2 tiles x 4 k-steps x 64 lanes = 1536 uint4, 6 per thread
#pragma unroll
    for (int q = 0; q < 6; ++q) {
      const int slotq = q * 256 + tid;
      const int p = slotq / 512, j = (slotq / 256) & 1, i = (slotq / 64) & 3, l = slotq & 63;
      const int e = e0 + j * 16 + (l & 15);
      const int kk = kc * kTileK + 32 * (l >> 4) + 8 * i;
      uint4 v = *(const uint4*)(a.wr_planes + p * plane + (uint64_t)min(e, a.E - 1) * a.H + kk);
      if (e >= a.E) v = make_uint4(0u, 0u, 0u, 0u);
      wl[p][j][i][l] = v;
    }
    uint4 xb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) xb[i] = *(const uint4*)(xr + kc * kTileK + 8 * i);
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int p = 0; p < 3; ++p)
          acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(wl[p][j][i][lane]),
                                                           as_bf16x8(xb[i]), acc[j], 0, 0, 0);
    __syncthreads();
  }
  if (t0 + n < a.T) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int e = e0 + j * 16 + 4 * g + r;
        if (e < a.E)
          a.logits[(uint64_t)(t0 + n) * a.E + e] = acc[j][r] + (a.router_b ? a.router_b[e] : 0.f);
      }
  }
}

// ---- top-k for many tokens ------------------------------------------------------------------
// Same radix select as decode (see ft_decode.hip), 16 tokens per workgroup.
__device__ __forceinline__ uint32_t order_key_p(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

template <int EPL>
__global__ __launch_bounds__(256) void k_topk_many(const float* __restrict__ logits, int T, int E,
                                                   int k, int32_t* __restrict__ idx,
                                                   float* __restrict__ w) {
  __shared__ float c_val[16][FT_MAX_TOPK];
  __shared__ int c_idx[16][FT_MAX_TOPK];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int tb = blockIdx.x * 16;
  const int nt = min(16, T - tb);
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int tl = wave; tl < nt; tl += 4) {
    const int t = tb + tl;
    float v[EPL];
    uint32_t key[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) v[i] = logits[(uint64_t)t * E + min(lane + 64 * i, E - 1)];
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
  int cnt[4], blk[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = tid * 4 + i;
    int c = 0;
    if (e < a.E)
      for (int b = 0; b < NBk; ++b) c += a.bcnt[(uint64_t)b * a.E + e];
    cnt[i] = c;
    blk[i] = (c + a.mrows - 1) / a.mrows;
  }
  // two exclusive scans over experts (pairs and 128-row blocks), four experts per thread
  for (int pass = 0; pass < 2; ++pass) {
    int v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = pass == 0 ? cnt[i] : blk[i];
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
    int* out = pass == 0 ? a.offsets : a.tb_off;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = tid * 4 + i;
      if (e < a.E) {
        out[e] = base;
        if (pass == 0) {
          a.counts[e] = cnt[i];
          int run = base;
          for (int b = 0; b < NBk; ++b) {
            a.base[(uint64_t)b * a.E + e] = run;
            run += a.bcnt[(uint64_t)b * a.E + e];
          }
        }
      }
      base += v[i];
    }
    if (tid == 0) out[a.E] = total;
  }
}

__global__ __launch_bounds__(256) void k_perm_place(PrefillLaunch a) {
  const int b = blockIdx.x, tl = threadIdx.x;
  const int t = b * kPermBlock + tl;
  if (t >= a.T) return;
  for (int j = 0; j < a.k; ++j) {
    const int e = a.idx[(uint64_t)t * a.k + j];
    const uint32_t* m = a.masks + ((uint64_t)b * a.E + e) * 8;
    int r = __popc(m[tl >> 5] & ((1u << (tl & 31)) - 1u));
    for (int q = 0; q < (tl >> 5); ++q) r += __popc(m[q]);
    const int p = a.base[(uint64_t)b * a.E + e] + r;
    a.pos[(uint64_t)t * a.k + j] = p;
    a.perm_tok[p] = t;
  }
}

// ---- grouped GEMM (S0: exact bf16 operands) ------------------------------------------------
// Two E2M1 codes (byte B of w) times a non-power-of-two scale s -> packed bf16 pair.  The
// scaled convert uses only the exponent of its scale, so it runs with 1.0 and the fp32
// product (exact) is truncated to bf16 (exact: at most 6 significant bits).
template <int B>
__device__ __forceinline__ uint32_t nv_pair_c(uint32_t w, float s) {
  const auto f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, B);
  return (__float_as_uint(f[0] * s) >> 16) | (__float_as_uint(f[1] * s) & 0xffff0000u);
}
__device__ __forceinline__ uint32_t nv_pair(uint32_t w, float s, int b) {
  return b == 0 ? nv_pair_c<0>(w, s) : b == 1 ? nv_pair_c<1>(w, s) : b == 2 ? nv_pair_c<2>(w, s)
                                                                             : nv_pair_c<3>(w, s);
}

// Decode one 16-row x 128-K weight tile lane (16 code bytes + its scales) into four 16 B
// MFMA operands (k-steps i = 0..3, eight K values each).
__device__ __forceinline__ void decode_tile_lane(int fmt, const uint8_t* codes, const uint8_t* scales,
                                                 uint64_t tile, int lane, uint4 out[4]) {
  const uint4 c = ((const uint4*)codes)[tile * 64 + lane];
  const uint32_t wv[4] = {c.x, c.y, c.z, c.w};
  if (fmt == FT_MXFP4) {
    const float s = e8m0_f32(scales[tile * 64 + lane]);
#pragma unroll
    for (int i = 0; i < 4; ++i) out[i] = __builtin_bit_cast(uint4, fp4x8_bf16(wv[i], s));
  } else {
    // E2M1 -> fp32 (exact), times the E4M3 block scale (exact: <= 6 significant bits), then
    // the top half of each fp32 is the bf16 value
    const float s0 = e4m3_f32(scales[tile * 128 + 2 * lane]);
    const float s1 = e4m3_f32(scales[tile * 128 + 2 * lane + 1]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float s = i < 2 ? s0 : s1;
      out[i] = make_uint4(nv_pair(wv[i], s, 0), nv_pair(wv[i], s, 1), nv_pair(wv[i], s, 2),
                          nv_pair(wv[i], s, 3));
    }
  }
}

__device__ __forceinline__ void decode_tile_regs(int fmt, uint4 c, uint32_t sc0, uint32_t sc1,
                                                 uint4 out[4]) {
  const uint32_t wv[4] = {c.x, c.y, c.z, c.w};
  if (fmt == FT_MXFP4) {
    const float s = e8m0_f32(sc0);
#pragma unroll
    for (int i = 0; i < 4; ++i) out[i] = __builtin_bit_cast(uint4, fp4x8_bf16(wv[i], s));
  } else {
    const float s0 = e4m3_f32(sc0), s1 = e4m3_f32(sc1);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float s = i < 2 ? s0 : s1;
      out[i] = make_uint4(nv_pair(wv[i], s, 0), nv_pair(wv[i], s, 1), nv_pair(wv[i], s, 2),
                          nv_pair(wv[i], s, 3));
    }
  }
}

__device__ __forceinline__ float blob_tscale(const uint8_t* blob, int m) {
  return ((const BlobHeader*)blob)->tensor_scale[m];
}

// MODE 0: gate/up + SwiGLU -> hperm; MODE 1: down -> Yperm.  NB feature blocks.
// Block (token block g, feature block fb) sits on XCD g % 8 (workgroup ids go round-robin
// over the 8 XCDs), so all feature blocks of one token block share that XCD's L2 for x.
template <int MODE>
__global__ __launch_bounds__(256) void k_ggemm(PrefillLaunch a, int NB) {
  constexpr int XS = kTileK + 8;               // LDS row stride of the token tile (bf16)
  __shared__ uint16_t xs[kGemmM][XS];          // 34 KB
  __shared__ uint4 ws[8][4][64];               // 32 KB: [weight tile][k-step][lane]
  __shared__ int s_e;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int n = lane & 15, g = lane >> 4;
  const int Lb = blockIdx.x, xcd = Lb & 7, jj = Lb >> 3;
  const int gblk = xcd + 8 * (jj / NB), fb = jj % NB;
  const int G = a.tb_off[a.E];
  if (gblk >= G) return;
  if (tid == 0) {  // expert of this token block: tb_off[e] <= gblk < tb_off[e + 1]
    int lo = 0, hi = a.E - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (a.tb_off[mid] <= gblk) lo = mid; else hi = mid - 1;
    }
    s_e = lo;
  }
  __syncthreads();
  const int e = s_e;
  const int row0 = a.offsets[e] + (gblk - a.tb_off[e]) * kGemmM;
  const int nrows = min(kGemmM, a.offsets[e + 1] - row0);
  const int K = MODE == 0 ? a.H : a.I;
  const int KC = K / kTileK;
  const uint8_t* blob = a.pool + (uint64_t)e * a.stride;
  const int fmt = a.L.fmt;
  const int wm = wave >> 1, wn = wave & 1;
  // staging role: row r of the token tile, half h2 (64 K values)
  const int sr = tid >> 1, sh = tid & 1;
  // rows past the expert's last token re-read its last row (always valid) and are zeroed
  const bool srow = sr < nrows;
  const int rr = row0 + min(sr, nrows - 1);
  const uint16_t* src = MODE == 0 ? a.x + (uint64_t)a.perm_tok[rr] * a.H
                                  : a.hperm + (uint64_t)rr * a.I;
  // weight tiles this wave decodes: q = 2*wave, 2*wave + 1 of the block's 8
  const uint8_t* wc[2];
  const uint8_t* wsc[2];
  uint64_t wrow[2];
#pragma unroll
  for (int d = 0; d < 2; ++d) {
    const int q = 2 * wave + d;
    int m, rt;
    if (MODE == 0) { m = q < 4 ? 0 : 1; rt = fb * 4 + (q & 3); }
    else { m = 2; rt = fb * 8 + q; }
    wc[d] = blob + a.L.off[2 * m];
    wsc[d] = blob + a.L.off[2 * m + 1];
    wrow[d] = (uint64_t)rt * KC;
  }
  // the wave's four weight tiles in the block tile (gate/up: two gate + the same two up)
  int wt[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) wt[j] = MODE == 0 ? ((j < 2) ? 2 * wn + j : 4 + 2 * wn + j - 2) : 4 * wn + j;

  f32x4 acc[4][4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[j][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // software pipeline: the global loads of chunk kc + 1 (token tile rows and this wave's
  // two weight tiles) are in flight while the MFMAs of chunk kc run
  uint4 xv[8], cw[2];
  uint32_t sc[2][2];
  auto load_chunk = [&](int kc) {
#pragma unroll
    for (int i = 0; i < 8; ++i) xv[i] = *(const uint4*)(src + kc * kTileK + sh * 64 + 8 * i);
#pragma unroll
    for (int d = 0; d < 2; ++d) {
      const uint64_t tile = wrow[d] + kc;
      cw[d] = ((const uint4*)wc[d])[tile * 64 + lane];
      if (fmt == FT_MXFP4) {
        sc[d][0] = wsc[d][tile * 64 + lane];
        sc[d][1] = 0u;
      } else {
        sc[d][0] = wsc[d][tile * 128 + 2 * lane];
        sc[d][1] = wsc[d][tile * 128 + 2 * lane + 1];
      }
    }
  };
  load_chunk(0);
  for (int kc = 0; kc < KC; ++kc) {
    uint4 dq[2][4];
#pragma unroll
    for (int d = 0; d < 2; ++d) decode_tile_regs(fmt, cw[d], sc[d][0], sc[d][1], dq[d]);
    __syncthreads();  // the previous chunk's MFMAs are done with the LDS tiles
#pragma unroll
    for (int i = 0; i < 8; ++i)
      *(uint4*)&xs[sr][sh * 64 + 8 * i] = srow ? xv[i] : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
    for (int d = 0; d < 2; ++d)
#pragma unroll
      for (int i = 0; i < 4; ++i) ws[2 * wave + d][i][lane] = dq[d][i];
    __syncthreads();
    if (kc + 1 < KC) load_chunk(kc + 1);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      bf16x8 A[4], B[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) A[j] = as_bf16x8(ws[wt[j]][i][lane]);
#pragma unroll
      for (int t = 0; t < 4; ++t)
        B[t] = as_bf16x8(*(const uint4*)&xs[wm * 64 + t * 16 + n][32 * g + 8 * i]);
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int t = 0; t < 4; ++t)
          acc[j][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[j], B[t], acc[j][t], 0, 0, 0);
    }
  }

  if (MODE == 0) {
    const float tsg = blob_tscale(blob, 0), tsu = blob_tscale(blob, 1);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int row = wm * 64 + t * 16 + n;
      if (row < nrows) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int f = fb * 64 + wn * 32 + j * 16 + 4 * g;
          uint16_t hv[4];
#pragma unroll
          for (int r = 0; r < 4; ++r)
            hv[r] = f32_to_bf16_rne(silu_f32(acc[j][t][r] * tsg) * (acc[j + 2][t][r] * tsu));
          *(uint2*)(a.hperm + (uint64_t)(row0 + row) * a.I + f) =
              make_uint2((uint32_t)hv[0] | ((uint32_t)hv[1] << 16),
                         (uint32_t)hv[2] | ((uint32_t)hv[3] << 16));
        }
      }
    }
  } else {
    const float tsd = blob_tscale(blob, 2);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int row = wm * 64 + t * 16 + n;
      if (row < nrows) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int f = fb * kGemmN + wn * 64 + j * 16 + 4 * g;
          *(float4*)(a.Yperm + (uint64_t)(row0 + row) * a.H + f) =
              make_float4(acc[j][t][0] * tsd, acc[j][t][1] * tsd, acc[j][t][2] * tsd,
                          acc[j][t][3] * tsd);
        }
      }
    }
  }
}

// ---- scaled-FP4 mode (both MFMA operands FP4) ------------------------------------------------
typedef int i32x8 __attribute__((ext_vector_type(8)));

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
// MODE 1: down -> Y_perm.  A workgroup owns 8 weight tiles (MODE 0: 4 gate + the same 4 up
// row tiles, 64 features; MODE 1: 8 row tiles of W_d) and a block of up to 256 token rows of
// one expert.  Weights stream from HBM once per block through a double-buffered LDS stage
// (two chunks of 128 K in flight in registers); each wave takes the token tiles
// wave, wave + 4, ... and loads their FP4 rows straight into MFMA operands, so tokens are
// never staged.  Block (token block g, feature block fb) sits on XCD g % 8.
template <int N>
struct ic { static constexpr int value = N; };

template <int MODE, int NS, bool TAIL>
__global__ __launch_bounds__(256) void k_s1_gemm(PrefillLaunch a, int NB) {
  __shared__ uint4 wl[2][8][64];        // [buffer][weight tile][lane] codes, 16 KB
  __shared__ uint32_t wsl[2][64][2];    // [buffer][lane]: scale byte of tile t at t / 4, t % 4
  __shared__ int s_e;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, g = lane >> 4;
  const int Lb = blockIdx.x, xcd = Lb & 7, jj = Lb >> 3;
  const int gblk = xcd + 8 * (jj / NB), fb = jj % NB;
  if (gblk >= a.tb_off[a.E]) return;
  if (tid == 0) {  // expert of this token block: tb_off[e] <= gblk < tb_off[e + 1]
    int lo = 0, hi = a.E - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (a.tb_off[mid] <= gblk) lo = mid; else hi = mid - 1;
    }
    s_e = lo;
  }
  __syncthreads();
  const int e = __builtin_amdgcn_readfirstlane(s_e);
  const int row0 = a.offsets[e] + (gblk - a.tb_off[e]) * kS1Rows;
  const int nrows = min(kS1Rows, a.offsets[e + 1] - row0);
  const int ntile = (nrows + 15) >> 4;
  const int nj = __builtin_amdgcn_readfirstlane(max(0, (ntile - wave + 3) >> 2));
  const int KC = (MODE == 0 ? a.H : a.I) / kTileK;
  const uint8_t* blob = a.mxpool + (uint64_t)e * a.mxstride;

  // staging roles: 32 code bytes (lanes 2 sp, 2 sp + 1) of tile st; waves 0 and 1 also stage
  // the scale bytes of lanes 4 sq .. 4 sq + 3 of tile sct
  const int st = tid >> 5, sp = tid & 31;
  const int sct = (tid >> 4) & 7, sq = tid & 15;
  const bool stage_scales = wave < 2;
  const int mc = MODE == 0 ? (st < 4 ? 0 : 1) : 2;
  const int rc = MODE == 0 ? fb * 4 + (st & 3) : fb * 8 + st;
  const int ms = MODE == 0 ? (sct < 4 ? 0 : 1) : 2;
  const int rs = MODE == 0 ? fb * 4 + (sct & 3) : fb * 8 + sct;
  const uint8_t* wsrc = blob + a.ML.off[2 * mc] + (uint64_t)rc * KC * kTileCodeBytes + sp * 32;
  const uint8_t* ssrc = blob + a.ML.off[2 * ms + 1] + (uint64_t)rs * KC * 64 + sq * 4;

  // token operand sources of the wave's tiles (rows past the block's end re-read its last
  // row, which is valid, and are never stored)
  const uint8_t* tsrc[4];
  const uint8_t* tssrc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int rr = row0 + min(16 * (wave + 4 * j) + n, nrows - 1);
    if (MODE == 0) {
      const uint64_t t = (uint64_t)a.perm_tok[rr];
      tsrc[j] = a.xq + t * (a.H / 2) + 16 * g;
      tssrc[j] = a.xqs + t * (a.H / 32) + g;
    } else {
      tsrc[j] = a.hq + (uint64_t)rr * (a.I / 2) + 16 * g;
      tssrc[j] = a.hqs + (uint64_t)rr * (a.I / 32) + g;
    }
  }

  f32x4 acc[8][4];
#pragma unroll
  for (int f = 0; f < 8; ++f)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[f][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // NS register sets of weight chunks in flight (chunk kc lives in set kc % NS) and two sets
  // of token operands (chunk kc in set kc % 2), all in separately named registers.  Every load
  // is unconditional, so the compiler's wait counts stay exact: chunk indices past the end
  // re-read the last chunk (an L2 hit) and are never used.
  static_assert(NS == 2 || NS == 4, "two or four weight chunks in flight");
  uint4 w0a, w0b, w1a, w1b, w2a, w2b, w3a, w3b;
  uint32_t s0, s1, s2, s3;
  uint4 tA[4], tB[4];
  uint32_t uA[4], uB[4];

#define FT_S1_WLOAD(kc_, A_, B_, S_)                                                   \
  do {                                                                                 \
    const uint64_t c_ = (uint64_t)min((kc_), KC - 1);                                  \
    const uint4* p_ = (const uint4*)(wsrc + c_ * kTileCodeBytes);                      \
    A_ = p_[0];                                                                        \
    B_ = p_[1];                                                                        \
    S_ = *(const uint32_t*)(ssrc + c_ * 64);                                           \
  } while (0)
#define FT_S1_TLOAD(kc_, T_, U_)                                                       \
  do {                                                                                 \
    const uint64_t c_ = (uint64_t)min((kc_), KC - 1);                                  \
    _Pragma("unroll") for (int j_ = 0; j_ < 4; ++j_) {                                 \
      T_[j_] = *(const uint4*)(tsrc[j_] + c_ * 64);                                    \
      U_[j_] = tssrc[j_][c_ * 4];                                                      \
    }                                                                                  \
  } while (0)
  // chunk kc: stage its weights into LDS buffer kc & 1 (last read by chunk kc - 2, which every
  // wave finished before the barrier of chunk kc - 1), load the tokens of chunk kc + 1, refill
  // the register set with chunk kc + NS, then run chunk kc's MFMAs.  The token loads go out
  // before the weight loads: waits retire loads in issue order, so waiting for the tokens
  // of the next chunk leaves the weight chunks in flight.
#define FT_S1_STEP(kc_, A_, B_, S_, T_, U_, TN_, UN_)                                    \
  do {                                                                                   \
    const int buf_ = (kc_) & 1;                                                          \
    wl[buf_][st][2 * sp] = A_;                                                           \
    wl[buf_][st][2 * sp + 1] = B_;                                                       \
    if (stage_scales) {                                                                  \
      uint8_t* sb_ = (uint8_t*)&wsl[buf_][0][0];                                         \
      _Pragma("unroll") for (int i_ = 0; i_ < 4; ++i_)                                   \
        sb_[(4 * sq + i_) * 8 + sct] = (uint8_t)(S_ >> (8 * i_));                        \
    }                                                                                    \
    FT_S1_TLOAD((kc_) + 1, TN_, UN_);                                                    \
    FT_S1_WLOAD((kc_) + NS, A_, B_, S_);                                                 \
    __syncthreads();                                                                     \
    const uint32_t slo_ = wsl[buf_][lane][0], shi_ = wsl[buf_][lane][1];                 \
    uint4 Aop_[8];                                                                       \
    _Pragma("unroll") for (int f_ = 0; f_ < 8; ++f_) Aop_[f_] = wl[buf_][f_][lane];      \
    _Pragma("unroll") for (int j_ = 0; j_ < 4; ++j_) {                                   \
      if (j_ < nj) {                                                                     \
        _Pragma("unroll") for (int f_ = 0; f_ < 8; ++f_)                                 \
          acc[f_][j_] = mfma_fp4(Aop_[f_], T_[j_], acc[f_][j_],                          \
                                 (f_ < 4 ? slo_ : shi_) >> (8 * (f_ & 3)), U_[j_]);      \
      }                                                                                  \
    }                                                                                    \
  } while (0)

  FT_S1_WLOAD(0, w0a, w0b, s0);
  FT_S1_WLOAD(1, w1a, w1b, s1);
  if (NS == 4) {
    FT_S1_WLOAD(2, w2a, w2b, s2);
    FT_S1_WLOAD(3, w3a, w3b, s3);
  }
  FT_S1_TLOAD(0, tA, uA);
  // without TAIL, KC is a multiple of NS and the loop body has no branches
  for (int kc = 0; kc < KC; kc += NS) {
    FT_S1_STEP(kc, w0a, w0b, s0, tA, uA, tB, uB);
    if (!TAIL || kc + 1 < KC) FT_S1_STEP(kc + 1, w1a, w1b, s1, tB, uB, tA, uA);
    if (NS == 4) {
      if (!TAIL || kc + 2 < KC) FT_S1_STEP(kc + 2, w2a, w2b, s2, tA, uA, tB, uB);
      if (!TAIL || kc + 3 < KC) FT_S1_STEP(kc + 3, w3a, w3b, s3, tB, uB, tA, uA);
    }
  }
#undef FT_S1_STEP
#undef FT_S1_TLOAD
#undef FT_S1_WLOAD

  if (MODE == 0) {
    // h = silu(G) * U per (feature, token); MX block b (32 features) of a token is spread over
    // the four lanes n, n + 16, n + 32, n + 48 (tiles 2b, 2b + 1, four rows each)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (j >= nj) continue;
      const int row = 16 * (wave + 4 * j) + n;
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        float hv[2][4];
        float amax = 0.f;
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float h = silu_f32(acc[2 * b + t2][j][r]) * acc[4 + 2 * b + t2][j][r];
            hv[t2][r] = h;
            amax = fmaxf(amax, fabsf(h));
          }
        amax = fmaxf(amax, __shfl_xor(amax, 16, 64));
        amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
        const uint32_t sc = mx_scale_code(amax);
        const float inv = mx_inv_scale(sc);
        // features 4g .. 4g + 3 of tile 2b + t2 are block bytes 8 t2 + 2g, 8 t2 + 2g + 1
        uint32_t half[2];
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2)
          half[t2] = mx_code(hv[t2][0], inv) | (mx_code(hv[t2][1], inv) << 4) |
                     (mx_code(hv[t2][2], inv) << 8) | (mx_code(hv[t2][3], inv) << 12);
        const uint32_t mine = half[0] | (half[1] << 16);
        // lane group g writes block bytes 4g .. 4g + 3: the halves t2 = g / 2 of groups
        // 2 (g % 2) and 2 (g % 2) + 1
        const int src0 = n + 32 * (g & 1);
        const uint32_t v0 = (uint32_t)__shfl((int)mine, src0, 64);
        const uint32_t v1 = (uint32_t)__shfl((int)mine, src0 + 16, 64);
        const uint32_t word = g < 2 ? ((v0 & 0xffffu) | (v1 << 16))
                                    : ((v0 >> 16) | (v1 & 0xffff0000u));
        if (row < nrows) {
          const uint64_t pr = (uint64_t)(row0 + row);
          *(uint32_t*)(a.hq + pr * (a.I / 2) + (fb * 64 + 32 * b) / 2 + 4 * g) = word;
          if (g == 0) a.hqs[pr * (a.I / 32) + fb * 2 + b] = (uint8_t)sc;
        }
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (j >= nj) continue;
      const int row = 16 * (wave + 4 * j) + n;
      if (row < nrows) {
#pragma unroll
        for (int f = 0; f < 8; ++f) {
          const int col = fb * kGemmN + f * 16 + 4 * g;
          *(float4*)(a.Yperm + (uint64_t)(row0 + row) * a.H + col) =
              make_float4(acc[f][j][0], acc[f][j][1], acc[f][j][2], acc[f][j][3]);
        }
      }
    }
  }
}

// y[t][h] = sum_j w[t][j] Y_perm[pos[t][j]][h], j in rank order; four h per thread.
__global__ __launch_bounds__(256) void k_unpermute(PrefillLaunch a) {
  const int t = blockIdx.y;
  const int h = (blockIdx.x * 256 + threadIdx.x) * 4;
  if (h >= a.H) return;
  float4 v[FT_MAX_TOPK];
  float wj[FT_MAX_TOPK];
#pragma unroll
  for (int j = 0; j < FT_MAX_TOPK; ++j) {
    const int jc = min(j, a.k - 1);
    const int p = a.pos[(uint64_t)t * a.k + jc];
    wj[j] = a.w[(uint64_t)t * a.k + jc];
    v[j] = *(const float4*)(a.Yperm + (uint64_t)p * a.H + h);
  }
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int j = 0; j < FT_MAX_TOPK; ++j) {
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
  const int n = E * H;
  hipLaunchKernelGGL(k_split_router, dim3((n + 255) / 256), dim3(256), 0, st, wr, n, planes);
  return (int)hipGetLastError();
}

#define FT_PLAUNCH(kern, grid, evs, eve, ...)                                              \
  do {                                                                                     \
    auto* kfn_ = kern;                                                                     \
    if (evs) hipExtLaunchKernelGGL(kfn_, grid, dim3(256), 0, st, evs, eve, 0, __VA_ARGS__); \
    else hipLaunchKernelGGL(kfn_, grid, dim3(256), 0, st, __VA_ARGS__);                    \
  } while (0)

// ev: null or 4 events (gate/up start, stop, down start, stop).
extern "C" int ftk_prefill(const PrefillLaunch* ap, hipStream_t st, const hipEvent_t* ev) {
  const PrefillLaunch& a = *ap;
  const int nblk = (a.T + kPermBlock - 1) / kPermBlock;
  hipLaunchKernelGGL(k_router_prefill,
                     dim3((a.T + kRouterTokens - 1) / kRouterTokens,
                          (a.E + kRouterExperts - 1) / kRouterExperts),
                     dim3(256), 0, st, a);
  if (a.mode == FT_PREFILL_MXFP4) {
    const uint64_t nq = (uint64_t)a.T * (a.H / 32);
    hipLaunchKernelGGL(k_quant_x, dim3((unsigned)((nq + 255) / 256)), dim3(256), 0, st, a);
  }
  const dim3 tg((a.T + 15) / 16);
  if (a.E <= 64) hipLaunchKernelGGL(k_topk_many<1>, tg, dim3(256), 0, st, a.logits, a.T, a.E, a.k, a.idx, a.w);
  else if (a.E <= 128) hipLaunchKernelGGL(k_topk_many<2>, tg, dim3(256), 0, st, a.logits, a.T, a.E, a.k, a.idx, a.w);
  else if (a.E <= 256) hipLaunchKernelGGL(k_topk_many<4>, tg, dim3(256), 0, st, a.logits, a.T, a.E, a.k, a.idx, a.w);
  else hipLaunchKernelGGL(k_topk_many<16>, tg, dim3(256), 0, st, a.logits, a.T, a.E, a.k, a.idx, a.w);
  hipLaunchKernelGGL(k_perm_masks, dim3(nblk), dim3(256), 0, st, a);
  hipLaunchKernelGGL(k_perm_scan, dim3(1), dim3(256), 0, st, a);
  hipLaunchKernelGGL(k_perm_place, dim3(nblk), dim3(256), 0, st, a);
  // upper bound on mrows-row token blocks: sum_e ceil(c_e / mrows) <= T*k/mrows + E
  const int gmax = (a.T * a.k + a.mrows - 1) / a.mrows + a.E;
  const int g8 = (gmax + 7) / 8 * 8;
  hipEvent_t e0 = ev ? ev[0] : nullptr, e1 = ev ? ev[1] : nullptr;
  hipEvent_t e2 = ev ? ev[2] : nullptr, e3 = ev ? ev[3] : nullptr;
  const int nb0 = a.I / 64, nb1 = a.H / kGemmN;
  if (a.mode == FT_PREFILL_MXFP4) {
    // four weight chunks in flight when the chunk count allows a branch-free loop
    const int kc0 = a.H / kTileK, kc1 = a.I / kTileK;
    if (kc0 % 4 == 0) FT_PLAUNCH((k_s1_gemm<0, 4, false>), dim3(g8 * nb0), e0, e1, a, nb0);
    else if (kc0 % 2 == 0) FT_PLAUNCH((k_s1_gemm<0, 2, false>), dim3(g8 * nb0), e0, e1, a, nb0);
    else FT_PLAUNCH((k_s1_gemm<0, 2, true>), dim3(g8 * nb0), e0, e1, a, nb0);
    if (kc1 % 4 == 0) FT_PLAUNCH((k_s1_gemm<1, 4, false>), dim3(g8 * nb1), e2, e3, a, nb1);
    else if (kc1 % 2 == 0) FT_PLAUNCH((k_s1_gemm<1, 2, false>), dim3(g8 * nb1), e2, e3, a, nb1);
    else FT_PLAUNCH((k_s1_gemm<1, 2, true>), dim3(g8 * nb1), e2, e3, a, nb1);
  } else {
    FT_PLAUNCH(k_ggemm<0>, dim3(g8 * nb0), e0, e1, a, nb0);
    FT_PLAUNCH(k_ggemm<1>, dim3(g8 * nb1), e2, e3, a, nb1);
  }
  hipLaunchKernelGGL(k_unpermute, dim3((a.H / 4 + 255) / 256, a.T), dim3(256), 0, st, a);
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
