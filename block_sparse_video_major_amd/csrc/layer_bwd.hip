// Backward of the steps around the fine attention, for training a whole VSA
// layer end to end ("VSA: Faster Video Diffusion with Trainable Sparse
// Attention", Abstract), the index list held fixed (Top-K selection has no
// gradient):
//   * the gated combination ("VSA: Accelerating Video Diffusion Inference with
//     Sparse Attention on AMD GPUs", §Two-Stage Architecture: learnable gates
//     between the coarse and fine outputs), out = g_f * O_f + g_c * O_c[cube]:
//       dO_f = g_f * dout,  dO_c[c] = sum over the cube's tokens of g_c * dout,
//       dg_f = dout * O_f,  dg_c = dout * O_c[cube];
//   * the coarse attention (same page, Stage 1), O_c = softmax(scale Qc Kc^T) Vc
//     over all cubes: with P recomputed and Dc = rowsum(dO_c * O_c),
//       dVc = P^T dO_c,  dS = P * (dO_c Vc^T - Dc),
//       dQc = scale dS Kc,  dKc = scale dS^T Qc.
// (The pooling and reorder gradients are the cube_pass gradient mode.)
//
// Combine: one workgroup per cube, thread t owns column chunk t % CPR of rows
// t / CPR + RG k; the per-cube sum for dO_c is reduced through LDS in a fixed
// order (bit-reproducible).  Coarse, float32 throughout: five batched
// products over the heads (S and dP, then dQc, dKc and dVc) with
// register-blocked 64 x 64 tiles, and one row pass for the softmax and dS;
// S / P and dP / dS live in the caller's workspace.
#include "vsa_internal.h"

namespace vsa {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ void unpack8(const uint4& raw, float* f) {
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

__device__ __forceinline__ uint32_t pack2(float a, float b) {
  const __bf16 ha = (__bf16)a, hb = (__bf16)b;
  return (uint32_t)__builtin_bit_cast(uint16_t, ha) | ((uint32_t)__builtin_bit_cast(uint16_t, hb) << 16);
}

// ---- combine -------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kThreads) void combine_bwd_kernel(
    const __bf16* __restrict__ dout, const __bf16* __restrict__ of, const float* __restrict__ oc,
    const __bf16* __restrict__ gate_c, const __bf16* __restrict__ gate_f, __bf16* __restrict__ d_of,
    float* __restrict__ d_oc, float* __restrict__ d_gate_c, float* __restrict__ d_gate_f, int64_t units,
    int vol) {
  constexpr int CPR = D / 8;          // 16-byte chunks of 8 bf16 per row
  constexpr int RG = kThreads / CPR;  // row groups
  __shared__ float part[RG][D + 1];
  const int col = threadIdx.x % CPR;
  const int phase = threadIdx.x / CPR;
  for (int64_t unit = blockIdx.x; unit < units; unit += gridDim.x) {
    float ocv[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f}, acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
    if (gate_c != nullptr) {
      const float4 a = reinterpret_cast<const float4*>(oc + unit * D + col * 8)[0];
      const float4 b = reinterpret_cast<const float4*>(oc + unit * D + col * 8)[1];
      ocv[0] = a.x; ocv[1] = a.y; ocv[2] = a.z; ocv[3] = a.w;
      ocv[4] = b.x; ocv[5] = b.y; ocv[6] = b.z; ocv[7] = b.w;
    }
    for (int l = phase; l < vol; l += RG) {
      const int64_t off = (unit * vol + l) * D + col * 8;
      float dv[8], g[8];
      unpack8(*reinterpret_cast<const uint4*>(dout + off), dv);
      if (gate_f != nullptr) {
        unpack8(*reinterpret_cast<const uint4*>(gate_f + off), g);
        float o[8];
        unpack8(*reinterpret_cast<const uint4*>(of + off), o);
        float4* dg = reinterpret_cast<float4*>(d_gate_f + off);
        dg[0] = make_float4(dv[0] * o[0], dv[1] * o[1], dv[2] * o[2], dv[3] * o[3]);
        dg[1] = make_float4(dv[4] * o[4], dv[5] * o[5], dv[6] * o[6], dv[7] * o[7]);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) g[e] = 1.f;
      }
      uint4 pk;
      pk.x = pack2(g[0] * dv[0], g[1] * dv[1]);
      pk.y = pack2(g[2] * dv[2], g[3] * dv[3]);
      pk.z = pack2(g[4] * dv[4], g[5] * dv[5]);
      pk.w = pack2(g[6] * dv[6], g[7] * dv[7]);
      *reinterpret_cast<uint4*>(d_of + off) = pk;
      if (gate_c != nullptr) {
        float gc[8];
        unpack8(*reinterpret_cast<const uint4*>(gate_c + off), gc);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = fmaf(gc[e], dv[e], acc[e]);
        float4* dg = reinterpret_cast<float4*>(d_gate_c + off);
        dg[0] = make_float4(dv[0] * ocv[0], dv[1] * ocv[1], dv[2] * ocv[2], dv[3] * ocv[3]);
        dg[1] = make_float4(dv[4] * ocv[4], dv[5] * ocv[5], dv[6] * ocv[6], dv[7] * ocv[7]);
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) part[phase][col * 8 + e] = acc[e];
    __syncthreads();
    for (int d = threadIdx.x; d < D; d += kThreads) {
      float sum = 0.f;
#pragma unroll
      for (int p = 0; p < RG; ++p) sum += part[p][d];
      d_oc[unit * D + d] = sum;
    }
    __syncthreads();
  }
}

// ---- coarse: batched float32 products -------------------------------------------
// C[h] = alpha * op(A[h]) op(B[h]) for every (batch, head) h (grid z), with
// op(X) = X or X^T as stored row-major.  64 x 64 output tiles per workgroup,
// k in steps of 16 staged in LDS (A as [k][m], B as [k][n], rows padded to
// 68 floats), each thread a 4 x 4 block from two 16-byte LDS reads per k.
// Global loads run along whichever dimension is contiguous, 16 bytes at a
// time when the dimension and the row stride allow it.
constexpr int kTM = 64, kTN = 64, kTK = 16, kPad = 68;

template <bool TA, bool TB>
__global__ __launch_bounds__(kThreads) void gemm_f32_kernel(const float* __restrict__ A, const float* __restrict__ B,
                                                           float* __restrict__ C, int M, int N, int K, int lda,
                                                           int ldb, int ldc, int64_t sa, int64_t sb, int64_t sc,
                                                           float alpha) {
  __shared__ __attribute__((aligned(16))) float As[kTK][kPad];
  __shared__ __attribute__((aligned(16))) float Bs[kTK][kPad];
  const int tid = threadIdx.x;
  const int m0 = blockIdx.y * kTM, n0 = blockIdx.x * kTN;
  A += blockIdx.z * sa;
  B += blockIdx.z * sb;
  C += blockIdx.z * sc;
  const int tm = tid / 16, tn = tid % 16;   // 4 x 4 block (4 tm.., 4 tn..)
  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;
  // element (m, k) of op(A) is A[m * lda + k] (TA: A[k * lda + m]); (k, n) of
  // op(B) is B[k * ldb + n] (TB: B[n * ldb + k])
  for (int k0 = 0; k0 < K; k0 += kTK) {
    // 64 x 16 = 1024 elements of each tile, 4 per thread
    if (!TA) {   // contiguous along k: thread -> (m = tid / 4, k = 4 * (tid % 4) ..)
      const int m = m0 + tid / 4, k = k0 + 4 * (tid % 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) As[4 * (tid % 4) + e][tid / 4] = (m < M && k + e < K) ? A[(int64_t)m * lda + k + e] : 0.f;
    } else {     // contiguous along m: thread -> (k = tid / 16, m = 4 * (tid % 16) ..)
      const int k = k0 + tid / 16, m = m0 + 4 * (tid % 16);
#pragma unroll
      for (int e = 0; e < 4; ++e) As[tid / 16][4 * (tid % 16) + e] = (k < K && m + e < M) ? A[(int64_t)k * lda + m + e] : 0.f;
    }
    if (!TB) {   // contiguous along n
      const int k = k0 + tid / 16, n = n0 + 4 * (tid % 16);
#pragma unroll
      for (int e = 0; e < 4; ++e) Bs[tid / 16][4 * (tid % 16) + e] = (k < K && n + e < N) ? B[(int64_t)k * ldb + n + e] : 0.f;
    } else {     // contiguous along k
      const int n = n0 + tid / 4, k = k0 + 4 * (tid % 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) Bs[4 * (tid % 4) + e][tid / 4] = (n < N && k + e < K) ? B[(int64_t)n * ldb + k + e] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kTK; ++kk) {
      const float4 a = *reinterpret_cast<const float4*>(&As[kk][4 * tm]);
      const float4 b = *reinterpret_cast<const float4*>(&Bs[kk][4 * tn]);
      const float av[4] = {a.x, a.y, a.z, a.w}, bv[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + 4 * tm + i;
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + 4 * tn + j;
      if (n < N) C[(int64_t)m * ldc + n] = alpha * acc[i][j];
    }
  }
}

// Row i of one head: P = softmax(S) in place of S, and, with
// Dc = rowsum(dO_c * O_c), dS = P * (dP - Dc) in place of dP.  One wavefront
// per row.
__global__ __launch_bounds__(kThreads) void coarse_softmax_ds_kernel(float* __restrict__ smat, float* __restrict__ dpmat,
                                                                    const float* __restrict__ oc,
                                                                    const float* __restrict__ doc, int Nc, int D,
                                                                    int64_t rows) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (row >= rows) return;
  float* srow = smat + row * Nc;
  float* drow = dpmat + row * Nc;
  float m = -INFINITY;
  for (int j = lane; j < Nc; j += 64) m = fmaxf(m, srow[j]);
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  float sum = 0.f;
  for (int j = lane; j < Nc; j += 64) sum += __expf(srow[j] - m);
  for (int o = 32; o >= 1; o >>= 1) sum += __shfl_xor(sum, o);
  float dc = 0.f;
  for (int d = lane; d < D; d += 64) dc = fmaf(doc[row * D + d], oc[row * D + d], dc);
  for (int o = 32; o >= 1; o >>= 1) dc += __shfl_xor(dc, o);
  const float inv = 1.f / sum;
  for (int j = lane; j < Nc; j += 64) {
    const float p = __expf(srow[j] - m) * inv;
    srow[j] = p;
    drow[j] = p * (drow[j] - dc);
  }
}

template <bool TA, bool TB>
hipError_t gemm(int heads, const float* A, const float* B, float* C, int M, int N, int K, int lda, int ldb, int ldc,
                int64_t sa, int64_t sb, int64_t sc, float alpha, hipStream_t s) {
  const dim3 grid((unsigned)((N + kTN - 1) / kTN), (unsigned)((M + kTM - 1) / kTM), (unsigned)heads);
  hipLaunchKernelGGL((gemm_f32_kernel<TA, TB>), grid, dim3(kThreads), 0, s, A, B, C, M, N, K, lda, ldb, ldc, sa,
                     sb, sc, alpha);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_combine_bwd(const Geom& g, const void* dout, const void* of, const float* oc, const void* gate_c,
                              const void* gate_f, void* d_of, float* d_oc, float* d_gate_c, float* d_gate_f,
                              hipStream_t s) {
  const int64_t units = g.BH * g.Nc;
  const unsigned grid = (unsigned)(units < (1 << 20) ? units : (1 << 20));
  if (g.Dv == 128)   // every tensor here is as wide as V
    hipLaunchKernelGGL(combine_bwd_kernel<128>, dim3(grid), dim3(kThreads), 0, s, (const __bf16*)dout,
                       (const __bf16*)of, oc, (const __bf16*)gate_c, (const __bf16*)gate_f, (__bf16*)d_of, d_oc,
                       d_gate_c, d_gate_f, units, g.vol);
  else if (g.Dv == 64)
    hipLaunchKernelGGL(combine_bwd_kernel<64>, dim3(grid), dim3(kThreads), 0, s, (const __bf16*)dout,
                       (const __bf16*)of, oc, (const __bf16*)gate_c, (const __bf16*)gate_f, (__bf16*)d_of, d_oc,
                       d_gate_c, d_gate_f, units, g.vol);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

size_t coarse_bwd_workspace(const Geom& g) {
  return 2 * sizeof(float) * (size_t)g.BH * (size_t)g.Nc * (size_t)g.Nc;
}

// S = scale Qc Kc^T and dP = dO_c Vc^T, then P and dS in place, then
// dQc = scale dS Kc, dKc = scale dS^T Qc, dVc = P^T dO_c.  Each product is
// batched over key/value heads: the `group` query heads sharing one are
// contiguous, so their Qc, dO_c, S and dS rows stack into one M = group * Nc
// operand and dKc, dVc sum over the group inside the product.
hipError_t launch_coarse_bwd(const Geom& g, const float* qc, const float* kc, const float* vc, const float* oc,
                             const float* doc, float* dqc, float* dkc, float* dvc, void* workspace,
                             hipStream_t s) {
  // D: query/key width (Qc, Kc), DV: value width (Vc, O_c, dO_c)
  const int Nc = (int)g.Nc, D = g.D, DV = g.Dv, Hk = (int)g.BHkv, Mq = g.group * Nc;
  const int64_t sq = (int64_t)Mq * D, sk = (int64_t)Nc * D, sm = (int64_t)Mq * Nc;
  const int64_t sqv = (int64_t)Mq * DV, skv = (int64_t)Nc * DV;
  float* smat = static_cast<float*>(workspace);
  float* dpmat = smat + (size_t)g.BH * g.Nc * g.Nc;
  const float scale = 1.0f / sqrtf((float)D);
  hipError_t e;
  if ((e = gemm<false, true>(Hk, qc, kc, smat, Mq, Nc, D, D, D, Nc, sq, sk, sm, scale, s)) != hipSuccess) return e;
  if ((e = gemm<false, true>(Hk, doc, vc, dpmat, Mq, Nc, DV, DV, DV, Nc, sqv, skv, sm, 1.0f, s)) != hipSuccess)
    return e;
  const int64_t rows = g.BH * g.Nc;
  hipLaunchKernelGGL(coarse_softmax_ds_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(kThreads), 0, s, smat, dpmat,
                     oc, doc, Nc, DV, rows);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = gemm<false, false>(Hk, dpmat, kc, dqc, Mq, D, Nc, Nc, D, D, sm, sk, sq, scale, s)) != hipSuccess) return e;
  if ((e = gemm<true, false>(Hk, dpmat, qc, dkc, Nc, D, Mq, Nc, D, D, sm, sq, sk, scale, s)) != hipSuccess) return e;
  return gemm<true, false>(Hk, smat, doc, dvc, Nc, DV, Mq, Nc, DV, DV, sm, sqv, skv, 1.0f, s);
}

}  // namespace vsa
