// Block relation matrix -> VSA index list.
//
// "VSA: Accelerating Video Diffusion Inference with Sparse Attention on AMD
// GPUs", §Comparison with Jenga ("Sparse Encoding in CK Tile": a block-mask
// method keeps the M x M one-hot relation B, B[i][j] = 1 when query block i
// attends key block j; VSA keeps the selected key-block indices and their
// count) and §Block-Sparse Encoding.  The list is written in ascending order;
// a row with more than max_kv selected blocks keeps its first max_kv and is
// counted in *overflow_rows.
//
// One wavefront per row: 256 mask bytes per pass (64 when Nc is not a
// multiple of 4), ballots mark the selected ones and ballot prefix counts
// give each its slot in the list.  Entries past a row's count are not
// written.
#include "vsa_internal.h"

namespace vsa {
namespace {

constexpr int kThreads = 256;

__global__ void zero_counter_kernel(int32_t* p) { *p = 0; }

// VEC = mask bytes per lane per pass (4 when every row starts 4-byte aligned,
// i.e. Nc % 4 == 0, else 1).  Within a pass lane i owns columns
// base + VEC*i .. base + VEC*i + VEC - 1; one ballot per byte position gives
// every selected column its slot in ascending column order.
template <int VEC>
__global__ __launch_bounds__(kThreads) void mask_to_lut_kernel(const uint8_t* __restrict__ mask, int Nc,
                                                               int max_kv, int64_t rows,
                                                               int32_t* __restrict__ lut,
                                                               int32_t* __restrict__ valid,
                                                               int32_t* __restrict__ overflow_rows) {
  const int64_t row = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  const uint8_t* m = mask + row * (int64_t)Nc;
  int32_t* out = lut + row * (int64_t)max_kv;
  const uint64_t lt = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  int seen = 0;   // selected blocks in earlier passes
  for (int base = 0; base < Nc; base += 64 * VEC) {
    const int j0 = base + VEC * lane;
    uint32_t bytes = 0;
    if (VEC == 4) {
      if (j0 < Nc) bytes = *reinterpret_cast<const uint32_t*>(m + j0);   // Nc % 4 == 0: all 4 in the row
    } else {
      if (j0 < Nc) bytes = m[j0];
    }
    uint64_t b[VEC];
    int total = 0;
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      b[e] = __ballot(((bytes >> (8 * e)) & 0xffu) != 0u);
      total += __popcll(b[e]);
    }
    // slot of column j0 + e = selected columns of lower lanes + earlier bytes of this lane
    int slot = seen;
#pragma unroll
    for (int e = 0; e < VEC; ++e) slot += __popcll(b[e] & lt);
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      if (((bytes >> (8 * e)) & 0xffu) != 0u) {
        if (slot < max_kv) out[slot] = j0 + e;
        ++slot;
      }
    }
    seen += total;
  }
  if (lane == 0) {
    valid[row] = seen < max_kv ? seen : max_kv;
    if (seen > max_kv) atomicAdd(overflow_rows, 1);
  }
}

}  // namespace

hipError_t launch_mask_to_lut(const Geom& g, const uint8_t* mask, int max_kv, int32_t* lut, int32_t* valid,
                              int32_t* overflow_rows, hipStream_t s) {
  const int64_t rows = g.BH * g.Nc;
  hipLaunchKernelGGL(zero_counter_kernel, dim3(1), dim3(1), 0, s, overflow_rows);
  const int64_t blocks = (rows + 3) / 4;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  if (g.Nc % 4 == 0 && reinterpret_cast<uintptr_t>(mask) % 4 == 0)
    hipLaunchKernelGGL(mask_to_lut_kernel<4>, dim3((unsigned)blocks), dim3(kThreads), 0, s, mask, (int)g.Nc,
                       max_kv, rows, lut, valid, overflow_rows);
  else
    hipLaunchKernelGGL(mask_to_lut_kernel<1>, dim3((unsigned)blocks), dim3(kThreads), 0, s, mask, (int)g.Nc,
                       max_kv, rows, lut, valid, overflow_rows);
  return hipGetLastError();
}

}  // namespace vsa
