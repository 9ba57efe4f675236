// Internal declarations of libft shared by the host runtime (g++) and the HIP kernels.
#pragma once

#include <stdint.h>
#include <stddef.h>

#include "../../include/ft.h"

#if defined(__HIPCC__)
#define FT_HD __host__ __device__
#else
#define FT_HD
#endif

namespace ft {

// ---- tiled blob layout ------------------------------------------------------------------
// A matrix [R][K] (K = contraction axis) is stored in tiles of 16 rows x 128 K.  Tile
// (rt, kc) holds 1024 code bytes; lane l (0..63) of a wave owns bytes [16 l, 16 l + 16):
// row rt*16 + l%16, K elements kc*128 + 32*(l/16) .. +31, two codes per byte, low nibble
// first.  This is the operand layout of one 16-row x 32-K slab per lane group of the
// 16x16x32 MFMA, so one 128-bit load per lane feeds four MFMAs with no shuffles.
// Scales: MXFP4 one E8M0 byte per lane per tile (64 B per tile, lane l's byte = block
// kc*4 + l/16 of row l%16); NVFP4 two E4M3 bytes per lane (128 B per tile, lane l's pair =
// blocks kc*8 + 2*(l/16) + {0,1}).  Tiles are ordered row-tile major: tile index =
// rt * (K/128) + kc, so a wave walking K for one row tile reads contiguous memory.

constexpr int kTileRows = 16;
constexpr int kTileK = 128;
constexpr int kTileCodeBytes = 1024;
constexpr uint64_t kAlign = 4096;
constexpr uint32_t kBlobMagic = 0x31425446u;  // "FTB1"

FT_HD inline uint64_t align_up(uint64_t v, uint64_t a) { return (v + a - 1) / a * a; }
FT_HD inline int scale_tile_bytes(int fmt) { return fmt == FT_MXFP4 ? 64 : 128; }

struct BlobLayout {
  int fmt, H, I;
  uint64_t off[6];   // gate codes, gate scales, up codes, up scales, down codes, down scales
  uint64_t bytes;    // whole blob, multiple of 4096
};

struct BlobHeader {
  uint32_t magic;
  int32_t fmt, H, I;
  float tensor_scale[3];
  int32_t reserved[9];
};

FT_HD inline BlobLayout blob_layout(int fmt, int H, int I) {
  BlobLayout L;
  L.fmt = fmt; L.H = H; L.I = I;
  const uint64_t gc = (uint64_t)I * H / 2, dc = (uint64_t)H * I / 2;
  const uint64_t sb = (uint64_t)scale_tile_bytes(fmt);
  const uint64_t gs = (uint64_t)(I / kTileRows) * (H / kTileK) * sb;
  const uint64_t ds = (uint64_t)(H / kTileRows) * (I / kTileK) * sb;
  uint64_t o = kAlign;  // header
  const uint64_t sz[6] = {gc, gs, gc, gs, dc, ds};
  for (int i = 0; i < 6; ++i) { L.off[i] = o; o = align_up(o + sz[i], kAlign); }
  L.bytes = o;
  return L;
}

// ---- decode work list ------------------------------------------------------------------
// One entry per distinct expert of a decode call (plus one per shared expert): the blob to
// read and up to 16 (token, pair) columns.  `pair` indexes the per-(token, choice) partial
// buffer P[T * kk + j] with kk = k + n_shared (j = k + s for shared expert s).
constexpr int kMaxCols = 16;
struct WorkItem {
  int32_t expert;    // routed expert id, or -1 - s for shared expert s
  int32_t slot;      // pool slot, or -1 - s for shared expert s
  int32_t ntok;      // columns in use (1..16; 0 marks an unused entry of a GPU-built list)
  int32_t pad;
  int32_t tok[kMaxCols];
  int32_t pair[kMaxCols];
  float wt[kMaxCols];  // GPU-built lists: the column's routing weight (1 for shared experts)
};

// Arguments of one decode expert pass (gate/up + SwiGLU, then down) as the host hands them
// to the kernel launcher.
struct DecodeLaunch {
  const uint16_t* x;            // device bf16 tokens [T][H]
  int T, H, I, E, k, n_shared;
  int route;                    // 0: work list from `items`; 1: top-k + list from `logits`;
                                // 2: list from the routed indices in `idx_out`
  const float* logits;          // [T][E] (route)
  const int32_t* e2s;           // [E] (route)
  int32_t* idx_out;             // [T][k] (route: written by workgroup 0)
  float* w_out;                 // [T][k] (route)
  WorkItem* items;              // route: written; otherwise read
  int* n_items;
  int max_items;                // launch sizing bound on the item count
  const uint8_t* pool;
  const uint8_t* shared;
  uint64_t stride;
  BlobLayout L;
  uint16_t* h;                  // [max_items][16][I]
  float* P;                     // [T * (k + n_shared)][H] (miss path: combined by k_combine)
  float* y;                     // [T][H]: all-resident calls combine inside the down kernel
  int fuse_combine;             // list mode: 1 = the down kernel combines the whole list into y
                                // (the items carry their weights)
};

// One-launch routing of a miss-path call (k_route_small): the layer's own router and, when
// n_routers == 2, a second router over the same tokens (cross-layer prefetch prediction).
struct RouteSmall {
  const uint16_t* x;            // device bf16 [T][H]
  uint16_t* x_host;             // mapped pinned copy of x, or null
  int T, H, n_routers;
  const float* wr[2];           // [E][H]
  const float* b[2];            // [E] or null
  int E[2], k[2];
  float* logits[2];             // [T][E]
  int32_t* idx[2];              // [T][k], device
  float* w[2];
  int32_t* idx_host[2];         // [T][k], mapped pinned
  float* w_host[2];
  unsigned int* counter;        // device, zero between launches
  uint32_t* flag_host;          // mapped pinned word: set to seq once the outputs are in host memory
  uint32_t seq;
};

// Prefill of T tokens through an all-resident layer (slot e = expert e).
constexpr int kPermBlock = 256;   // tokens per permutation block (one mask word per 32)
constexpr int kGemmM = 256;       // token rows per exact-mode grouped-GEMM block
constexpr int kS1Rows = 256;      // token rows per scaled-FP4 grouped-GEMM block

// Prefill router: 128 tokens per workgroup, up to 6 tiles of 32 experts per workgroup, and the
// contraction over H split into `splits` ranges (partial logits summed in order by the top-k
// pass) so that the grid covers the chip.
constexpr int kRouterTokens = 128;
constexpr int kRouterGroupTiles = 6;
constexpr int kRouterMaxSplits = 8;
FT_HD inline int router_expert_tiles(int E) { return (E + 31) / 32; }
FT_HD inline int router_splits(int T, int E, int H) {
  const int blocks = ((T + kRouterTokens - 1) / kRouterTokens) *
                     ((router_expert_tiles(E) + kRouterGroupTiles - 1) / kRouterGroupTiles);
  int s = 1;
  while (s < kRouterMaxSplits && blocks * s < 256 && (H / 32) % (2 * s) == 0) s *= 2;
  return s;
}
// bytes of the router weight planes: [3 planes][E/32 tiles][H/16 K-steps][64 lanes][16 B]
FT_HD inline uint64_t router_plane_bytes(int E, int H) {
  return (uint64_t)3 * router_expert_tiles(E) * (H / 16) * 1024;
}

struct PrefillLaunch {
  const uint16_t* x;            // device bf16 [T][H]
  int T, H, I, E, k;
  int splits;                   // router contraction splits (router_splits)
  // the fp32 router weights as three bf16 planes whose sum is exactly W_r, each in the operand
  // order of the 32x32x16 MFMA: plane p, expert tile et, K-step ks: lane l holds expert
  // 32 et + l % 32, K 16 ks + 8 (l / 32) .. + 7 (experts past E are zero)
  const uint16_t* wr_planes;
  const float* router_b;        // [E] or null
  const uint8_t* pool;          // slot e holds expert e
  uint64_t stride;
  BlobLayout L;
  int mode;                     // FT_PREFILL_EXACT or FT_PREFILL_MXFP4
  int mrows;                    // token rows per grouped-GEMM block (kGemmM or kS1Rows)
  int pad_rows;                 // every expert's permuted rows padded to a multiple of this in
                                // the token-operand tiles (16: scaled-FP4 mode; 32: exact mode)
  const uint8_t* mxpool;        // FT_PREFILL_MXFP4: MXFP4 blob of expert e at e * mxstride
  uint64_t mxstride;
  BlobLayout ML;                // layout of those blobs
  // workspace (caller-owned, carved by the host)
  float* logits;                // [splits][T][E] partial router logits (no bias)
  int32_t* idx;                 // [T][k]
  float* w;                     // [T][k]
  uint32_t* masks;              // [T/256][E][8] token bitmasks per permutation block
  int32_t* bcnt;                // [T/256][E]
  int32_t* counts;              // [E]
  int32_t* offsets;             // [E+1]
  int32_t* base;                // [T/256][E]
  int32_t* tb_off;              // [E+1] prefix of mrows-row token blocks per expert
  int32_t* blk_e;               // [T*k/mrows + E] expert of each token block
  int32_t* tile_e;              // [P/pad_rows] expert of each padded row group
  int32_t* pos;                 // [T][k]
  int32_t* perm_tok;            // [T*k] token of each permuted row
  float* perm_w;                // [T*k] routing weight of each permuted row
  // exact mode: the GEMMs' token operands as bf16 tiles of 32 padded rows x 16 K in the
  // operand order of the 32x32x16 MFMA, 1 KB each: tile (row group g, 64-K chunk c, step s)
  // at ((g * K/64 + c) * 4 + s) * 1 KB, lane (t, h) holding row 32 g + t, K 64 c + 32 h + 8 s
  // .. + 7; expert e's rows start at padded row poff[e]
  uint16_t* xtb;                // x rows, K = H (padding rows zero)
  uint16_t* htb;                // h rows, K = I (padding rows unspecified)
  uint8_t* xq;                  // MXFP4 mode: quantised x, codes [T][H/2]
  uint8_t* xqs;                 //   and E8M0 scales [T][H/32]
  // MXFP4 mode: the grouped GEMMs' token operands in the blob's tile format (16 rows x 128 K
  // per 1 KB tile, 64 B of scales per tile), rows in permuted order with every expert's rows
  // padded to a multiple of 16 (expert e's rows start at padded row poff[e]); padding rows
  // hold zero codes and scales
  int32_t* poff;                // [E+1]
  uint8_t* xt;                  // quantised x rows: codes [P/16][H/128][1 KB]
  uint8_t* xts;                 //   scales [P/16][H/128][64 B]
  uint8_t* ht;                  // quantised h rows: codes [P/16][I/128][1 KB]
  uint8_t* hts;                 //   scales [P/16][I/128][64 B]
  float* Yperm;                 // MXFP4 mode: [T*k][H] 24-bit floats, 4 in 12 bytes
  float* y;                     // [T][H]
};

}  // namespace ft
