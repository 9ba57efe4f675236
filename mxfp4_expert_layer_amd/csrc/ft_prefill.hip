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

// One workgroup: counts, offsets, bases and the 128-row block map.
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
    blk[i] = (c + kGemmM - 1) / kGemmM;
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
  const dim3 tg((a.T + 15) / 16);
  if (a.E <= 64) hipLaunchKernelGGL(k_topk_many<1>, tg, dim3(256), 0, st, a.logits, a.T, a.E, a.k, a.idx, a.w);
  else if (a.E <= 128) hipLaunchKernelGGL(k_topk_many<2>, tg, dim3(256), 0, st, a.logits, a.T, a.E, a.k, a.idx, a.w);
  else if (a.E <= 256) hipLaunchKernelGGL(k_topk_many<4>, tg, dim3(256), 0, st, a.logits, a.T, a.E, a.k, a.idx, a.w);
  else hipLaunchKernelGGL(k_topk_many<16>, tg, dim3(256), 0, st, a.logits, a.T, a.E, a.k, a.idx, a.w);
  hipLaunchKernelGGL(k_perm_masks, dim3(nblk), dim3(256), 0, st, a);
  hipLaunchKernelGGL(k_perm_scan, dim3(1), dim3(256), 0, st, a);
  hipLaunchKernelGGL(k_perm_place, dim3(nblk), dim3(256), 0, st, a);
  // upper bound on 128-row token blocks: sum_e ceil(c_e / 128) <= T*k/128 + E
  const int gmax = (a.T * a.k + kGemmM - 1) / kGemmM + a.E;
  const int g8 = (gmax + 7) / 8 * 8;
  hipEvent_t e0 = ev ? ev[0] : nullptr, e1 = ev ? ev[1] : nullptr;
  hipEvent_t e2 = ev ? ev[2] : nullptr, e3 = ev ? ev[3] : nullptr;
  const int nb0 = a.I / 64, nb1 = a.H / kGemmN;
  FT_PLAUNCH(k_ggemm<0>, dim3(g8 * nb0), e0, e1, a, nb0);
  FT_PLAUNCH(k_ggemm<1>, dim3(g8 * nb1), e2, e3, a, nb1);
  hipLaunchKernelGGL(k_unpermute, dim3((a.H / 4 + 255) / 256, a.T), dim3(256), 0, st, a);
  return (int)hipGetLastError();
}
