// Cube mean-pool: xc[bh, c, :] = (1/vol) * sum_l x_cube[bh, c*vol + l, :].
//
// "VSA: Accelerating Video Diffusion Inference with Sparse Attention on AMD
// GPUs", §Two-Stage Architecture, Stage 1: each cube is mean-pooled into one
// cube-level vector (Qc, Kc, Vc).
//
// One workgroup per cube.  Thread t owns a 16-byte column chunk and a row
// phase; it sums rows phase, phase + RG, ... in float32, then the RG partial
// rows are added in a fixed order through LDS.  The order never depends on
// timing, so results are bit-reproducible.  HBM-bound: the cube-major input
// is read once (contiguous), the pooled row is written once.
#include "vsa_internal.h"

namespace vsa {
namespace {

constexpr int kThreads = 256;

template <typename T>
__device__ __forceinline__ void widen(const uint4& raw, float* out);

template <>
__device__ __forceinline__ void widen<__bf16>(const uint4& raw, float* out) {
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = __uint_as_float(w[i] << 16);
    out[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

template <>
__device__ __forceinline__ void widen<float>(const uint4& raw, float* out) {
  out[0] = __uint_as_float(raw.x);
  out[1] = __uint_as_float(raw.y);
  out[2] = __uint_as_float(raw.z);
  out[3] = __uint_as_float(raw.w);
}

// E = elements per 16-byte chunk, CPR = chunks per row, RG = row phases.
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void pool_kernel(const uint4* __restrict__ x, float* __restrict__ xc,
                                                        int vol, int64_t n_cubes) {
  constexpr int E = 16 / sizeof(T);
  constexpr int CPR = D / E;
  constexpr int RG = kThreads / CPR;
  __shared__ float part[RG][D + 1];
  const int64_t cube = blockIdx.x;
  if (cube >= n_cubes) return;
  const int col = threadIdx.x % CPR;
  const int phase = threadIdx.x / CPR;
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  const uint4* src = x + cube * (int64_t)vol * CPR;
  for (int r = phase; r < vol; r += RG) {
    float v[E];
    widen<T>(src[(int64_t)r * CPR + col], v);
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] += v[e];
  }
#pragma unroll
  for (int e = 0; e < E; ++e) part[phase][col * E + e] = acc[e];
  __syncthreads();
  const float fvol = (float)vol;
  for (int d = threadIdx.x; d < D; d += kThreads) {
    float s = 0.f;
#pragma unroll
    for (int p = 0; p < RG; ++p) s += part[p][d];
    xc[cube * D + d] = s / fvol;
  }
}

template <typename T>
hipError_t launch_t(const Geom& g, const void* x, float* xc, hipStream_t s) {
  const int64_t n_cubes = g.BH * g.Nc;
  if (g.D == 64)
    hipLaunchKernelGGL((pool_kernel<T, 64>), dim3((unsigned)n_cubes), dim3(kThreads), 0, s,
                       (const uint4*)x, xc, g.vol, n_cubes);
  else if (g.D == 128)
    hipLaunchKernelGGL((pool_kernel<T, 128>), dim3((unsigned)n_cubes), dim3(kThreads), 0, s,
                       (const uint4*)x, xc, g.vol, n_cubes);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace

hipError_t launch_pool(const Geom& g, int dtype, const void* x_cube, float* xc, hipStream_t s) {
  return dtype == VSA_BF16 ? launch_t<__bf16>(g, x_cube, xc, s) : launch_t<float>(g, x_cube, xc, s);
}

}  // namespace vsa
