// LUT validator: counts LUT rows that the fine kernel must not be given
// ("VSA: Accelerating Video Diffusion Inference with Sparse Attention on AMD
// GPUs", §Block-Sparse Encoding: per query block a valid count and that many
// key-block indices).  A row is bad if its count is outside
// [0, max_kv_blocks] or one of its first `count` entries is outside [0, Nc).
#include "vsa_internal.h"

namespace vsa {
namespace {

constexpr int kThreads = 256;

__global__ void zero_kernel(int32_t* p) { *p = 0; }

// One wavefront per LUT row.
__global__ __launch_bounds__(kThreads) void check_lut_kernel(const int32_t* __restrict__ lut,
                                                             const int32_t* __restrict__ valid,
                                                             int max_kv, int Nc, int64_t rows,
                                                             int32_t* bad_rows) {
  const int64_t row = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  const int n = valid[row];
  bool bad = n < 0 || n > max_kv;
  if (!bad) {
    for (int i = lane; i < n; i += 64) {
      const int j = lut[row * max_kv + i];
      bad |= (j < 0 || j >= Nc);
    }
  }
  const bool any = __ballot(bad) != 0ull;
  if (any && lane == 0) atomicAdd(bad_rows, 1);
}

}  // namespace

hipError_t launch_check_lut(const Geom& g, const int32_t* lut, const int32_t* valid, int max_kv,
                            int32_t* bad_rows, hipStream_t s) {
  const int64_t rows = g.BH * g.Nc;
  hipLaunchKernelGGL(zero_kernel, dim3(1), dim3(1), 0, s, bad_rows);
  const int64_t blocks = (rows + 3) / 4;
  hipLaunchKernelGGL(check_lut_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, s, lut, valid, max_kv,
                     (int)g.Nc, rows, bad_rows);
  return hipGetLastError();
}

}  // namespace vsa
