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
// order (bit-reproducible).  Coarse, fp32 throughout: the rows kernel takes R
// query cubes per workgroup, forms their score and dP rows against key chunks
// staged in LDS, the row softmax, P and dS (written to the workspace) and dQc;
// the columns kernel takes R key cubes and sums dKc and dVc over query chunks
// staged the same way.
#include "vsa_internal.h"

namespace vsa {
namespace {

constexpr int kThreads = 256;
constexpr int kChunk = 32;   // key (or query) cubes staged in LDS at a time

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

// ---- coarse: rows ----------------------------------------------------------------
// Query cubes i0 .. i0 + R - 1 of one (batch, head).  LDS: their Qc and dO_c
// rows, their score / P rows and dP / dS rows over all Nc key cubes, and one
// staged chunk of Kc and Vc rows.
template <int D, int R>
__global__ __launch_bounds__(kThreads) void coarse_bwd_rows_kernel(
    const float* __restrict__ qc, const float* __restrict__ kc, const float* __restrict__ vc,
    const float* __restrict__ oc, const float* __restrict__ doc, float* __restrict__ dqc,
    float* __restrict__ pmat, float* __restrict__ dsmat, int Nc, float scale) {
  constexpr int KS = D + 1;   // padded row stride of staged chunks
  extern __shared__ float sm[];
  float* qr = sm;                      // [R][D]
  float* dr = qr + R * D;              // [R][D]
  float* sr = dr + R * D;              // [R][Nc]  scores, then P
  float* pr = sr + R * Nc;             // [R][Nc]  dP, then dS
  float* kch = pr + R * Nc;            // [kChunk][KS]
  float* vch = kch + kChunk * KS;      // [kChunk][KS]
  const int tid = threadIdx.x;
  const int blocks = (Nc + R - 1) / R;
  const int64_t bh = blockIdx.x / blocks;
  const int i0 = (int)(blockIdx.x - bh * blocks) * R;
  const int64_t base = bh * (int64_t)Nc * D;
  for (int e = tid; e < R * D; e += kThreads) {
    const int r = e / D, i = i0 + r;
    qr[e] = i < Nc ? qc[base + (int64_t)i * D + e % D] : 0.f;
    dr[e] = i < Nc ? doc[base + (int64_t)i * D + e % D] : 0.f;
  }
  // scores and dP against key chunks
  for (int j0 = 0; j0 < Nc; j0 += kChunk) {
    __syncthreads();
    for (int e = tid; e < kChunk * D; e += kThreads) {
      const int jj = e / D, j = j0 + jj;
      kch[jj * KS + e % D] = j < Nc ? kc[base + (int64_t)j * D + e % D] : 0.f;
      vch[jj * KS + e % D] = j < Nc ? vc[base + (int64_t)j * D + e % D] : 0.f;
    }
    __syncthreads();
    for (int pair = tid; pair < R * kChunk; pair += kThreads) {
      const int r = pair / kChunk, jj = pair % kChunk, j = j0 + jj;
      float s = 0.f, p = 0.f;
#pragma unroll 8
      for (int d = 0; d < D; ++d) {
        s = fmaf(qr[r * D + d], kch[jj * KS + d], s);
        p = fmaf(dr[r * D + d], vch[jj * KS + d], p);
      }
      if (j < Nc) {
        sr[r * Nc + j] = scale * s;
        pr[r * Nc + j] = p;
      }
    }
  }
  __syncthreads();
  // row softmax, Dc, dS; one wavefront per row
  const int wave = tid >> 6, lane = tid & 63;
  for (int r = wave; r < R; r += kThreads / 64) {
    const int i = i0 + r;
    if (i >= Nc) continue;
    float m = -INFINITY;
    for (int j = lane; j < Nc; j += 64) m = fmaxf(m, sr[r * Nc + j]);
    for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
    float sum = 0.f;
    for (int j = lane; j < Nc; j += 64) sum += __expf(sr[r * Nc + j] - m);
    for (int o = 32; o >= 1; o >>= 1) sum += __shfl_xor(sum, o);
    float dc = 0.f;
    for (int d = lane; d < D; d += 64) dc = fmaf(dr[r * D + d], oc[base + (int64_t)i * D + d], dc);
    for (int o = 32; o >= 1; o >>= 1) dc += __shfl_xor(dc, o);
    const float inv = 1.f / sum;
    float* prow = pmat + (bh * (int64_t)Nc + i) * Nc;
    float* dsrow = dsmat + (bh * (int64_t)Nc + i) * Nc;
    for (int j = lane; j < Nc; j += 64) {
      const float p = __expf(sr[r * Nc + j] - m) * inv;
      const float ds = p * (pr[r * Nc + j] - dc);
      sr[r * Nc + j] = p;
      pr[r * Nc + j] = ds;
      prow[j] = p;
      dsrow[j] = ds;
    }
  }
  // dQc = scale * dS Kc over key chunks
  constexpr int OUT = R * D / kThreads > 0 ? R * D / kThreads : 1;   // outputs per thread
  float acc[OUT];
#pragma unroll
  for (int u = 0; u < OUT; ++u) acc[u] = 0.f;
  for (int j0 = 0; j0 < Nc; j0 += kChunk) {
    __syncthreads();
    for (int e = tid; e < kChunk * D; e += kThreads) {
      const int jj = e / D, j = j0 + jj;
      kch[jj * KS + e % D] = j < Nc ? kc[base + (int64_t)j * D + e % D] : 0.f;
    }
    __syncthreads();
    const int jn = Nc - j0 < kChunk ? Nc - j0 : kChunk;
#pragma unroll
    for (int u = 0; u < OUT; ++u) {
      const int e = tid + u * kThreads;
      if (e < R * D) {
        const int r = e / D, d = e % D;
        float a = acc[u];
        for (int jj = 0; jj < jn; ++jj) a = fmaf(pr[r * Nc + j0 + jj], kch[jj * KS + d], a);
        acc[u] = a;
      }
    }
  }
#pragma unroll
  for (int u = 0; u < OUT; ++u) {
    const int e = tid + u * kThreads;
    if (e < R * D) {
      const int r = e / D, d = e % D, i = i0 + r;
      if (i < Nc) dqc[base + (int64_t)i * D + d] = scale * acc[u];
    }
  }
}

// ---- coarse: columns --------------------------------------------------------------
// Key cubes j0 .. j0 + R - 1: dKc = scale * dS^T Qc and dVc = P^T dO_c, summed
// over chunks of query cubes staged in LDS.
template <int D, int R>
__global__ __launch_bounds__(kThreads) void coarse_bwd_cols_kernel(
    const float* __restrict__ qc, const float* __restrict__ doc, const float* __restrict__ pmat,
    const float* __restrict__ dsmat, float* __restrict__ dkc, float* __restrict__ dvc, int Nc, float scale) {
  constexpr int KS = D + 1;
  __shared__ float qch[kChunk * KS];
  __shared__ float dch[kChunk * KS];
  __shared__ float pch[kChunk * R];
  __shared__ float sch[kChunk * R];
  const int tid = threadIdx.x;
  const int blocks = (Nc + R - 1) / R;
  const int64_t bh = blockIdx.x / blocks;
  const int j0 = (int)(blockIdx.x - bh * blocks) * R;
  const int64_t base = bh * (int64_t)Nc * D;
  const int64_t mbase = bh * (int64_t)Nc * Nc;
  constexpr int OUT = R * D / kThreads > 0 ? R * D / kThreads : 1;
  float ak[OUT], av[OUT];
#pragma unroll
  for (int u = 0; u < OUT; ++u) { ak[u] = 0.f; av[u] = 0.f; }
  for (int i0 = 0; i0 < Nc; i0 += kChunk) {
    __syncthreads();
    for (int e = tid; e < kChunk * D; e += kThreads) {
      const int ii = e / D, i = i0 + ii;
      qch[ii * KS + e % D] = i < Nc ? qc[base + (int64_t)i * D + e % D] : 0.f;
      dch[ii * KS + e % D] = i < Nc ? doc[base + (int64_t)i * D + e % D] : 0.f;
    }
    for (int e = tid; e < kChunk * R; e += kThreads) {
      const int ii = e / R, jr = e % R, i = i0 + ii, j = j0 + jr;
      const bool in = i < Nc && j < Nc;
      pch[e] = in ? pmat[mbase + (int64_t)i * Nc + j] : 0.f;
      sch[e] = in ? dsmat[mbase + (int64_t)i * Nc + j] : 0.f;
    }
    __syncthreads();
    const int in_n = Nc - i0 < kChunk ? Nc - i0 : kChunk;
#pragma unroll
    for (int u = 0; u < OUT; ++u) {
      const int e = tid + u * kThreads;
      if (e < R * D) {
        const int jr = e / D, d = e % D;
        float a = ak[u], b = av[u];
        for (int ii = 0; ii < in_n; ++ii) {
          a = fmaf(sch[ii * R + jr], qch[ii * KS + d], a);
          b = fmaf(pch[ii * R + jr], dch[ii * KS + d], b);
        }
        ak[u] = a;
        av[u] = b;
      }
    }
  }
#pragma unroll
  for (int u = 0; u < OUT; ++u) {
    const int e = tid + u * kThreads;
    if (e < R * D) {
      const int jr = e / D, d = e % D, j = j0 + jr;
      if (j < Nc) {
        dkc[base + (int64_t)j * D + d] = scale * ak[u];
        dvc[base + (int64_t)j * D + d] = av[u];
      }
    }
  }
}

constexpr int kLdsMax = 160 * 1024;

template <int D, int R>
size_t rows_lds(int Nc) {
  return sizeof(float) * ((size_t)2 * R * D + (size_t)2 * R * Nc + (size_t)2 * kChunk * (D + 1));
}

template <int D, int R>
hipError_t launch_coarse_r(const Geom& g, const float* qc, const float* kc, const float* vc, const float* oc,
                           const float* doc, float* dqc, float* dkc, float* dvc, float* pmat, float* dsmat,
                           hipStream_t s) {
  static int granted[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  const int Nc = (int)g.Nc;
  const size_t lds = rows_lds<D, R>(Nc);
  if (lds > (size_t)kLdsMax) return hipErrorInvalidValue;
  auto kr = coarse_bwd_rows_kernel<D, R>;
  if (granted[dev] < (int)lds) {
    const hipError_t e = hipFuncSetAttribute((const void*)kr, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    granted[dev] = (int)lds;
  }
  const float scale = 1.0f / sqrtf((float)D);
  const unsigned blocks = (unsigned)(g.BH * ((Nc + R - 1) / R));
  hipLaunchKernelGGL(kr, dim3(blocks), dim3(kThreads), lds, s, qc, kc, vc, oc, doc, dqc, pmat, dsmat, Nc, scale);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((coarse_bwd_cols_kernel<D, R>), dim3(blocks), dim3(kThreads), 0, s, qc, doc,
                     (const float*)pmat, (const float*)dsmat, dkc, dvc, Nc, scale);
  return hipGetLastError();
}

// R = query (key) cubes per workgroup: as many as let the score rows fit in LDS.
template <int D>
hipError_t launch_coarse_d(const Geom& g, const float* qc, const float* kc, const float* vc, const float* oc,
                           const float* doc, float* dqc, float* dkc, float* dvc, float* pmat, float* dsmat,
                           hipStream_t s) {
  const int Nc = (int)g.Nc;
  if (rows_lds<D, 8>(Nc) <= (size_t)kLdsMax)
    return launch_coarse_r<D, 8>(g, qc, kc, vc, oc, doc, dqc, dkc, dvc, pmat, dsmat, s);
  if (rows_lds<D, 4>(Nc) <= (size_t)kLdsMax)
    return launch_coarse_r<D, 4>(g, qc, kc, vc, oc, doc, dqc, dkc, dvc, pmat, dsmat, s);
  return launch_coarse_r<D, 2>(g, qc, kc, vc, oc, doc, dqc, dkc, dvc, pmat, dsmat, s);
}

}  // namespace

hipError_t launch_combine_bwd(const Geom& g, const void* dout, const void* of, const float* oc, const void* gate_c,
                              const void* gate_f, void* d_of, float* d_oc, float* d_gate_c, float* d_gate_f,
                              hipStream_t s) {
  const int64_t units = g.BH * g.Nc;
  const unsigned grid = (unsigned)(units < (1 << 20) ? units : (1 << 20));
  if (g.D == 128)
    hipLaunchKernelGGL(combine_bwd_kernel<128>, dim3(grid), dim3(kThreads), 0, s, (const __bf16*)dout,
                       (const __bf16*)of, oc, (const __bf16*)gate_c, (const __bf16*)gate_f, (__bf16*)d_of, d_oc,
                       d_gate_c, d_gate_f, units, g.vol);
  else if (g.D == 64)
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

hipError_t launch_coarse_bwd(const Geom& g, const float* qc, const float* kc, const float* vc, const float* oc,
                             const float* doc, float* dqc, float* dkc, float* dvc, void* workspace,
                             hipStream_t s) {
  float* pmat = static_cast<float*>(workspace);
  float* dsmat = pmat + (size_t)g.BH * g.Nc * g.Nc;
  if (g.D == 128) return launch_coarse_d<128>(g, qc, kc, vc, oc, doc, dqc, dkc, dvc, pmat, dsmat, s);
  if (g.D == 64) return launch_coarse_d<64>(g, qc, kc, vc, oc, doc, dqc, dkc, dvc, pmat, dsmat, s);
  return hipErrorInvalidValue;
}

}  // namespace vsa
