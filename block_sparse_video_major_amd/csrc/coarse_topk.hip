// Coarse stage: cube-to-cube scores, Top-K key-cube selection (the LUT) and
// the coarse attention output O_c.
//
// "VSA: Accelerating Video Diffusion Inference with Sparse Attention on AMD
// GPUs", §Two-Stage Architecture (Stage 1: coarse scores, Top-K cubes per
// query cube, coarse output kept for global context), §Block-Sparse Encoding
// (index list + valid count) and §Generating Sparsity Patterns (scores are
// the pooled-query / pooled-key inner products, Top-K per query row);
// "VSA: Faster Video Diffusion with Trainable Sparse Attention", Abstract.
//
// One workgroup = R query cubes of one (batch, head).
//   phase 1  all threads: raw scores s[r][j] = <qc[i0+r], kc[j]> in float32
//            (sequential FMA over d), kept in LDS;
//   phase 2  one wavefront per row: Top-K by radix select over the 32-bit
//            order-preserving key of each score, one bit per pass, counting
//            with wavefront ballots; the selected indices are emitted in
//            ascending order through a ballot prefix count.  Ties at the
//            threshold go to the lower index.  Then the row softmax
//            p_j = exp(scale*(s_j - max)), summed in a fixed order;
//   phase 3  all threads: O_c[r] = sum_j p_j * vc[j] / sum_j p_j.
// The scale 1/sqrt(d) > 0 does not change the ranking, so ranking uses the
// raw scores.
#include "vsa_internal.h"

namespace vsa {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

// Order-preserving map float -> uint32 (larger float -> larger key).  -0 is
// folded onto +0 so that equal scores compare equal.
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t b = __float_as_uint(f);
  if (b == 0x80000000u) b = 0u;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ int popc64(uint64_t m) { return __popcll(m); }

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

template <int D>
__global__ __launch_bounds__(kThreads) void coarse_topk_kernel(
    const float* __restrict__ qc, const float* __restrict__ kc, const float* __restrict__ vc,
    int32_t* __restrict__ lut, int32_t* __restrict__ valid, float* __restrict__ oc, int Nc, int top_k,
    int R, int tiles_per_head, float scale) {
  extern __shared__ float smem[];
  float* qs = smem;                 // [R][D]
  float* srow = smem + R * D;       // [R][Nc]
  float* inv_sum = srow + (int64_t)R * Nc;  // [R]

  const int64_t bh = blockIdx.x / tiles_per_head;
  const int i0 = (int)(blockIdx.x - bh * tiles_per_head) * R;
  const int rows = min(R, Nc - i0);
  const float* qh = qc + bh * (int64_t)Nc * D;
  const float* kh = kc + bh * (int64_t)Nc * D;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  for (int e = tid; e < R * D; e += kThreads) {
    const int r = e / D;
    qs[e] = (r < rows) ? qh[(int64_t)(i0 + r) * D + (e - r * D)] : 0.f;
  }
  __syncthreads();

  // phase 1: raw scores
  for (int j = tid; j < Nc; j += kThreads) {
    const float4* kr = reinterpret_cast<const float4*>(kh + (int64_t)j * D);
    for (int r0 = 0; r0 < R; r0 += 8) {
      float acc[8];
#pragma unroll
      for (int r = 0; r < 8; ++r) acc[r] = 0.f;
#pragma unroll 4
      for (int d4 = 0; d4 < D / 4; ++d4) {
        const float4 kv = kr[d4];
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          if (r0 + r < R) {
            const float4 qv = *reinterpret_cast<const float4*>(qs + (r0 + r) * D + 4 * d4);
            acc[r] = fmaf(qv.x, kv.x, acc[r]);
            acc[r] = fmaf(qv.y, kv.y, acc[r]);
            acc[r] = fmaf(qv.z, kv.z, acc[r]);
            acc[r] = fmaf(qv.w, kv.w, acc[r]);
          }
        }
      }
#pragma unroll
      for (int r = 0; r < 8; ++r)
        if (r0 + r < R) srow[(int64_t)(r0 + r) * Nc + j] = acc[r];
    }
  }
  __syncthreads();

  // phase 2: per-row Top-K and softmax weights, one wavefront per row
  const int nslots = (Nc + 63) / 64;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int r = wave; r < rows; r += kWaves) {
    float* sr = srow + (int64_t)r * Nc;
    const int64_t row = bh * Nc + i0 + r;
    int32_t* out_idx = lut + row * top_k;
    // K-th largest key: build the threshold from the top bit down.
    uint32_t thr = 0u;
    if (top_k < Nc) {
      for (int bit = 31; bit >= 0; --bit) {
        const uint32_t cand = thr | (1u << bit);
        int cnt = 0;
        for (int s = 0; s < nslots; ++s) {
          const int j = s * 64 + lane;
          const bool ge = (j < Nc) && (order_key(sr[j]) >= cand);
          cnt += popc64(__ballot(ge));
        }
        if (cnt >= top_k) thr = cand;
      }
    }
    int gt = 0;
    for (int s = 0; s < nslots; ++s) {
      const int j = s * 64 + lane;
      gt += popc64(__ballot((j < Nc) && (order_key(sr[j]) > thr)));
    }
    const int need = top_k - gt;   // >= 1 entries equal to thr are taken
    int eq_before = 0, sel_before = 0;
    for (int s = 0; s < nslots; ++s) {
      const int j = s * 64 + lane;
      const uint32_t key = (j < Nc) ? order_key(sr[j]) : 0u;
      const bool in = j < Nc;
      const bool eq = in && key == thr;
      const uint64_t eqm = __ballot(eq);
      const int eq_rank = eq_before + popc64(eqm & lt_mask);
      const bool take = in && (key > thr || (eq && eq_rank < need));
      const uint64_t tm = __ballot(take);
      if (take) out_idx[sel_before + popc64(tm & lt_mask)] = j;
      sel_before += popc64(tm);
      eq_before += popc64(eqm);
    }
    if (lane == 0) valid[row] = top_k;

    if (oc != nullptr) {
      float m = -INFINITY;
      for (int j = lane; j < Nc; j += 64) m = fmaxf(m, sr[j]);
      m = wave_max(m);
      float sum = 0.f;
      for (int j = lane; j < Nc; j += 64) {
        const float p = expf(scale * (sr[j] - m));
        sr[j] = p;
        sum += p;
      }
      sum = wave_sum(sum);
      if (lane == 0) inv_sum[r] = 1.f / sum;
    }
  }
  if (oc == nullptr) return;
  __syncthreads();

  // phase 3: O_c rows; thread -> (column d, row phase)
  const float* vh = vc + bh * (int64_t)Nc * D;
  constexpr int G = kThreads / D;
  const int d = tid % D;
  const int ph = tid / D;
  for (int r0 = ph; r0 < rows; r0 += 4 * G) {
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < Nc; ++j) {
      const float vv = vh[(int64_t)j * D + d];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int r = r0 + u * G;
        if (r < rows) acc[u] = fmaf(srow[(int64_t)r * Nc + j], vv, acc[u]);
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int r = r0 + u * G;
      if (r < rows) oc[(bh * Nc + i0 + r) * D + d] = acc[u] * inv_sum[r];
    }
  }
}

}  // namespace

static size_t coarse_lds_bytes(int R, int64_t Nc, int D) {
  return sizeof(float) * ((size_t)R * D + (size_t)R * Nc + R);
}

hipError_t launch_coarse_topk(const Geom& g, int top_k, const float* qc, const float* kc,
                              const float* vc, int32_t* lut, int32_t* valid, float* oc,
                              hipStream_t s) {
  const int Nc = (int)g.Nc;
  const int R = Nc > 1536 ? 4 : 8;
  const int tiles = (Nc + R - 1) / R;
  const int64_t blocks = g.BH * tiles;
  const size_t lds = coarse_lds_bytes(R, Nc, g.D);
  const float scale = 1.0f / sqrtf((float)g.D);
  if (g.D == 64) {
    auto k = coarse_topk_kernel<64>;
    if (lds > 65536) (void)hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    hipLaunchKernelGGL(k, dim3((unsigned)blocks), dim3(kThreads), lds, s, qc, kc, vc, lut, valid, oc, Nc,
                       top_k, R, tiles, scale);
  } else if (g.D == 128) {
    auto k = coarse_topk_kernel<128>;
    if (lds > 65536) (void)hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    hipLaunchKernelGGL(k, dim3((unsigned)blocks), dim3(kThreads), lds, s, qc, kc, vc, lut, valid, oc, Nc,
                       top_k, R, tiles, scale);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace vsa
