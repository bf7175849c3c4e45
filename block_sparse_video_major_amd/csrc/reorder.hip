// Token reordering between raster (t, h, w) order and cube-major order.
//
// "VSA: Accelerating Video Diffusion Inference with Sparse Attention on AMD
// GPUs", §Two-Stage Architecture (pre-stage reordering, Stage 1 cubes): the
// sequence is reordered so that every run of ct*ch*cw consecutive tokens is
// one spatio-temporal cube.  Cube-major order: cubes in raster order over
// the cube grid, tokens in raster order inside a cube.
//
// Both directions are one row gather, dst[row] = src[map(row)], written so
// that stores are fully contiguous and loads come in runs of cw tokens
// (cw * row_bytes contiguous bytes, 1 KiB for 4 bf16 tokens of d = 128).
// HBM-bound: each element is read once and written once.
#include "vsa_internal.h"

namespace vsa {
namespace {

// Cube-major position p -> raster token index.
__device__ __forceinline__ int64_t cube_to_raster(int64_t p, const Geom& g) {
  const int64_t c = p / g.vol;
  const int32_t l = (int32_t)(p - c * g.vol);
  const int32_t lw = l % g.cw, lh = (l / g.cw) % g.ch, lt = l / (g.cw * g.ch);
  const int64_t cw_i = c % g.gW, ch_i = (c / g.gW) % g.gH, ct_i = c / ((int64_t)g.gW * g.gH);
  const int64_t t = ct_i * g.ct + lt, h = ch_i * g.ch + lh, w = cw_i * g.cw + lw;
  return (t * g.H + h) * g.W + w;
}

// Raster token index r -> cube-major position.
__device__ __forceinline__ int64_t raster_to_cube(int64_t r, const Geom& g) {
  const int64_t w = r % g.W, h = (r / g.W) % g.H, t = r / ((int64_t)g.W * g.H);
  const int64_t c = ((t / g.ct) * g.gH + h / g.ch) * g.gW + w / g.cw;
  const int32_t l = (int32_t)(((t % g.ct) * g.ch + h % g.ch) * g.cw + w % g.cw);
  return c * g.vol + l;
}

constexpr int kThreads = 256;
constexpr int kUnroll = 4;   // 16-byte chunks per thread per pass

// CPR = 16-byte chunks per token row.  Every thread moves kUnroll chunks with
// all loads issued before the stores.
template <int CPR, bool TO_CUBE>
__global__ __launch_bounds__(kThreads) void gather_rows_kernel(const uint4* __restrict__ src,
                                                               uint4* __restrict__ dst, Geom g) {
  const int64_t total = g.BH * g.N * CPR;
  const int64_t base = (int64_t)blockIdx.x * (kThreads * kUnroll) + threadIdx.x;
  uint4 buf[kUnroll];
  int64_t dst_idx[kUnroll];
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const int64_t c = base + (int64_t)u * kThreads;
    dst_idx[u] = c;
    if (c < total) {
      const int64_t row = c / CPR;
      const int col = (int)(c - row * CPR);
      const int64_t bh = row / g.N;
      const int64_t p = row - bh * g.N;
      const int64_t srow = TO_CUBE ? cube_to_raster(p, g) : raster_to_cube(p, g);
      buf[u] = src[(bh * g.N + srow) * CPR + col];
    }
  }
#pragma unroll
  for (int u = 0; u < kUnroll; ++u)
    if (dst_idx[u] < total) dst[dst_idx[u]] = buf[u];
}

template <int CPR>
hipError_t launch_cpr(const Geom& g, const void* src, void* dst, bool to_cube, hipStream_t s) {
  const int64_t total = g.BH * g.N * CPR;
  const int64_t blocks = (total + kThreads * kUnroll - 1) / (kThreads * kUnroll);
  if (to_cube)
    hipLaunchKernelGGL((gather_rows_kernel<CPR, true>), dim3((unsigned)blocks), dim3(kThreads), 0, s,
                       (const uint4*)src, (uint4*)dst, g);
  else
    hipLaunchKernelGGL((gather_rows_kernel<CPR, false>), dim3((unsigned)blocks), dim3(kThreads), 0, s,
                       (const uint4*)src, (uint4*)dst, g);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_reorder(const Geom& g, int elem_bytes, const void* src, void* dst, bool to_cube,
                          hipStream_t s) {
  const int row_bytes = g.D * elem_bytes;
  switch (row_bytes / 16) {
    case 8: return launch_cpr<8>(g, src, dst, to_cube, s);
    case 16: return launch_cpr<16>(g, src, dst, to_cube, s);
    case 32: return launch_cpr<32>(g, src, dst, to_cube, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace vsa
