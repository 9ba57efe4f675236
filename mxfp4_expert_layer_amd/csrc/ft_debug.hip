// Test-hook kernels of libft: dequantise one matrix of a blob to fp32 in logical order.
#include <hip/hip_runtime.h>

#include "ft_device.h"

namespace ft {

// One wave per tile; MXFP4 decodes with the same conversion the GEMVs use.
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
    const bf16x8 v = fp4x8_bf16(w[i], s);
#pragma unroll
    for (int q = 0; q < 8; ++q) out[(uint64_t)row * K + k0 + 8 * i + q] = (float)v[q];
  }
}

// NVFP4: E2M1 value * E4M3 block scale * tensor scale in fp32.
__global__ __launch_bounds__(64) void k_dequant_nv(const uint8_t* codes, const uint8_t* scales,
                                                   int R, int K, float ts, float* out) {
  const int KC = K / kTileK;
  const int tile = blockIdx.x, lane = threadIdx.x;
  const int rt = tile / KC, kc = tile % KC;
  const int row = rt * kTileRows + (lane & 15);
  const int k0 = kc * kTileK + 32 * (lane >> 4);
  const uint4 c = ((const uint4*)codes)[(uint64_t)tile * 64 + lane];
  const float s0 = e4m3_f32_fast(scales[(uint64_t)tile * 128 + 2 * lane]);
  const float s1 = e4m3_f32_fast(scales[(uint64_t)tile * 128 + 2 * lane + 1]);
  const uint32_t w[4] = {c.x, c.y, c.z, c.w};
  for (int q = 0; q < 32; ++q) {
    const uint32_t code = (w[q >> 3] >> (4 * (q & 7))) & 15;
    out[(uint64_t)row * K + k0 + q] = e2m1_f32(code) * (q < 16 ? s0 : s1) * ts;
  }
}

}  // namespace ft

using namespace ft;

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

// HBM read-bandwidth probes.  k_read_probe: every lane streams 16-byte loads over the buffer
// (grid-stride, eight loads in flight) and folds them into one word, so nothing is dead code; a
// sweep on an MI355X (1K-16K workgroups, 4-16 loads in flight) peaked at 32 workgroups per
// compute unit and eight loads: 5.8 TB/s.
__global__ __launch_bounds__(256) void k_read_probe(const uint4* __restrict__ p, uint64_t n16,
                                                    uint32_t* __restrict__ sink) {
  const uint64_t stride = (uint64_t)gridDim.x * 256;
  uint32_t acc = 0;
  uint64_t i = (uint64_t)blockIdx.x * 256 + threadIdx.x;
  for (; i + 7 * stride < n16; i += 8 * stride) {
    uint4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = p[i + u * stride];
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const uint4 a = p[i];
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  if (acc == 0x9e3779b9u) atomicXor(&sink[blockIdx.x], acc);   // practically never taken
}

// k_read_probe_lds: one workgroup per compute unit (its 128 KB of LDS keeps a second one off)
// whose waves copy 1 KB blocks of the buffer (grid-stride over waves) into LDS with the direct
// global -> LDS load, up to 33 blocks in flight per wave and no register holding data.  On an
// MI355X this reaches 6.4-6.5 TB/s where the register loads above stop at 5.8 (more workgroups
// per CU lower both).  The tail below 1 KB is read by plain loads of workgroup 0.
__global__ __launch_bounds__(256) void k_read_probe_lds(const uint8_t* __restrict__ p,
                                                        uint64_t bytes, uint32_t* __restrict__ sink) {
  __shared__ uint4 ring[8192];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const uint64_t n1k = bytes >> 10, nw = (uint64_t)gridDim.x * 4;
  uint64_t i = (uint64_t)blockIdx.x * 4 + wave;
  for (int k = 0; i < n1k; i += nw, ++k) {
    dma16(p + i * 1024 + lane * 16, &ring[(wave * 32 + (k & 31)) * 64]);
    __builtin_amdgcn_s_waitcnt(FT_VMCNT(32));
  }
  __builtin_amdgcn_s_waitcnt(FT_VMCNT(0));
  uint32_t acc = 0;
  if (blockIdx.x == 0)
    for (uint64_t o = (n1k << 10) + 16 * threadIdx.x; o + 16 <= bytes; o += 16 * 256) {
      const uint4 a = *(const uint4*)(p + o);
      acc ^= a.x ^ a.y ^ a.z ^ a.w;
    }
  if (acc == 0x9e3779b9u) atomicXor(&sink[blockIdx.x], acc);   // practically never taken
}

extern "C" int ftk_read_probe(const void* buf, uint64_t bytes, uint32_t* sink, int grid,
                              int lds_form, hipStream_t st) {
  if (lds_form)
    hipLaunchKernelGGL(k_read_probe_lds, dim3(grid), dim3(256), 0, st, (const uint8_t*)buf, bytes,
                       sink);
  else
    hipLaunchKernelGGL(k_read_probe, dim3(grid), dim3(256), 0, st, (const uint4*)buf, bytes / 16,
                       sink);
  return (int)hipGetLastError();
}
