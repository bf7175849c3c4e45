// Token reordering between raster (t, h, w) order and cube-major order, the
// cube mean-pool, and both fused into one pass.
//
// "VSA: Accelerating Video Diffusion Inference with Sparse Attention on AMD
// GPUs", §Two-Stage Architecture: before Stage 1 the sequence is reordered so
// that every run of ct*ch*cw consecutive tokens is one spatio-temporal cube
// (cube-major order: cubes in raster order over the cube grid, tokens in
// raster order inside a cube), and Stage 1 mean-pools each cube into one
// cube-level vector (Qc, Kc, Vc).
//
// One workgroup per cube of one (batch, head) (grid-stride beyond 2^20).  The cube's vol token rows of
// CPR 16-byte chunks are spread over 256 threads: thread t always handles
// column chunk t % CPR of rows t / CPR, t / CPR + RG, ... (RG = 256 / CPR),
// so a wavefront touches whole rows.  On the cube-major side the cube is
// vol * row_bytes contiguous bytes; on the raster side it is ct * ch runs of
// cw tokens (cw * row_bytes contiguous bytes, 1 KiB for 4 bf16 tokens of
// d = 128).  All index arithmetic is 32-bit within a (batch, head) and done
// once per row, so the kernels stay HBM-bound.
//
// Cubes are numbered in the problem's cube order: raster over the cube grid,
// or a table of packed grid coordinates (one read per cube).
//
// A grid that does not divide into cubes is padded up to whole cubes: padded
// positions are written as zeros on the cube-major side, have no raster row,
// and are left out of the cube mean (which divides by the real-token count).
//
// The raster side is either [batch, heads, N, d] or the model's own
// [batch, N, heads, d] (a DiT's attention projections produce that order), so
// no separate transpose pass is needed on either side of the path.
//
// The pool also runs on its own from the raster rows (no cube-major copy
// written) for a fine stage that gathers its cube tiles from raster order.
//
// The gradient pass (float32 only) runs the reorder back and the adjoint of
// the pool at once: every token of cube c leaves with its own gradient plus
// xc[c] / vol, the gradient that reaches it through the cube mean.
//
// Pooling sums a thread's rows in increasing order in float32, then the RG
// partial rows in phase order through LDS, then divides by vol: the order
// never depends on timing, so results are bit-reproducible, and the fused
// pass produces exactly the bits of the separate reorder and pool passes.
#include <type_traits>

#include "mfma_util.h"
#include "vsa_internal.h"

namespace vsa {
namespace {

constexpr int kThreads = 256;
constexpr int64_t kMaxGrid = 1 << 20;   // larger problems loop over cubes

enum Mode { kToCube = 0, kToRaster = 1, kPool = 2, kToCubePool = 3, kToRasterAddPooled = 4, kPoolRaster = 5 };

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

// 16-byte load; NT marks it non-temporal (streamed once, not kept in the
// caches).  Measured on the 32K-token, 12-head, d = 128 tensors: plain
// reorders and the pool read 10-20% faster that way, the fused pass does
// not (its cube-major output is what the next stage reads).
template <bool NT>
__device__ __forceinline__ uint4 load16(const uint4* p) {
  if (!NT) return *p;
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(t.x, t.y, t.z, t.w);
}

// Geometry of one launch, all sizes that the row mapping needs.
struct CubeArgs {
  int32_t T, H, W;        // token grid
  int32_t ct, ch, cw;     // cube edges
  int32_t gT, gH, gW;     // cube grid
  const int32_t* coords;  // packed coordinates of each cube (Hilbert order), or null (raster order)
  int32_t vol;            // positions per cube
  int32_t N;              // real tokens per (batch, head): raster rows
  int32_t Np;             // cube-major positions per (batch, head)
  int32_t Nc;             // cubes per (batch, head)
  int32_t padded;         // the grid was padded up to whole cubes
  int32_t heads;          // heads per batch entry
  int32_t bnhd;           // raster side is [batch, N, heads, d] (else [batch, heads, N, d])
  int64_t units;          // batch * heads * Nc
};

// Raster offset, from the cube's first token, of token l of the cube.
__device__ __forceinline__ int32_t row_offset(int32_t l, const CubeArgs& a) {
  const int32_t plane = a.ch * a.cw;
  const int32_t lt = l / plane;
  const int32_t rem = l - lt * plane;
  const int32_t lh = rem / a.cw;
  const int32_t lw = rem - lh * a.cw;
  return (lt * a.H + lh) * a.W + lw;
}

// Where cube `unit` = (batch*head) * Nc + c lives on both sides: the raster
// row of its first token (row of token n of the (batch, head) = rbase + n *
// tstride), its first cube-major row, and its real extent along each axis
// (the cube edge unless the grid was padded).  ok is false for a table entry
// outside the grid (a table written for another problem).
struct UnitPos {
  bool ok;
  int64_t raster0, cube0, tstride;
  int32_t rem_t, rem_h, rem_w;
  // whether position l of the cube holds a real token
  __device__ __forceinline__ bool real(int32_t l, const CubeArgs& a) const {
    const int32_t plane = a.ch * a.cw;
    const int32_t lt = l / plane, rem = l - lt * plane;
    const int32_t lh = rem / a.cw;
    return lt < rem_t && lh < rem_h && rem - lh * a.cw < rem_w;
  }
};

__device__ __forceinline__ UnitPos unit_pos(const CubeArgs& a, int64_t unit) {
  UnitPos u;
  const int64_t bh = unit / a.Nc;
  const int32_t c = (int32_t)(unit - bh * a.Nc);
  int32_t ct_i, ch_i, cw_i;
  if (a.coords != nullptr) {
    const int32_t e = a.coords[c];   // the same for the whole workgroup
    ct_i = (e >> 20) & 1023;
    ch_i = (e >> 10) & 1023;
    cw_i = e & 1023;
    u.ok = ct_i < a.gT && ch_i < a.gH && cw_i < a.gW;
  } else {
    cw_i = c % a.gW;
    ch_i = (c / a.gW) % a.gH;
    ct_i = c / (a.gW * a.gH);
    u.ok = true;
  }
  int64_t rbase = bh * (int64_t)a.N;
  u.tstride = 1;
  if (a.bnhd) {
    const int64_t b = bh / a.heads;
    rbase = b * a.N * (int64_t)a.heads + (bh - b * a.heads);
    u.tstride = a.heads;
  }
  u.raster0 = rbase + (int64_t)((ct_i * a.ct * a.H + ch_i * a.ch) * a.W + cw_i * a.cw) * u.tstride;
  u.cube0 = bh * (int64_t)a.Np + (int64_t)c * a.vol;
  u.rem_t = min(a.ct, a.T - ct_i * a.ct);
  u.rem_h = min(a.ch, a.H - ch_i * a.ch);
  u.rem_w = min(a.cw, a.W - cw_i * a.cw);
  return u;
}

// T = element type (pool modes), D = head_dim; CPR = 16-byte chunks per row.
// Grid-stride over units = (batch*head) * Nc + cube.
template <typename T, int D, int MODE, bool PAD>
__global__ __launch_bounds__(kThreads) void cube_pass_kernel(const uint4* __restrict__ src,
                                                             uint4* __restrict__ dst,
                                                             float* __restrict__ xc, CubeArgs a) {
  constexpr int E = 16 / sizeof(T);
  constexpr int CPR = D / E;
  constexpr int RG = kThreads / CPR;
  constexpr int KB = RG >= 64 ? 1 : 64 / RG;   // rows per thread in flight: a 64-token cube in one batch
  constexpr bool kPooling = MODE == kPool || MODE == kToCubePool || MODE == kPoolRaster;
  constexpr bool kCopy = MODE != kPool && MODE != kPoolRaster;
  constexpr bool kFromRaster = MODE == kToCube || MODE == kToCubePool || MODE == kPoolRaster;
  // (the pool from raster rows streams too: measured on the 32K-token layer,
  // 56.7 against 58.6 us for three tensors, and the fine stage that then
  // gathers from the same rows runs no slower)
  constexpr bool kStreamLoads = MODE != kToCubePool;
  constexpr bool kAddPooled = MODE == kToRasterAddPooled;
  static_assert(!kAddPooled || std::is_same<T, float>::value, "the gradient pass is float32");
  __shared__ float part[kPooling ? RG : 1][kPooling ? D + 1 : 1];
  const int col = threadIdx.x % CPR;
  const int phase = threadIdx.x / CPR;

  for (int64_t unit = blockIdx.x; unit < a.units; unit += gridDim.x) {
    const UnitPos u = unit_pos(a, unit);
    if (!u.ok) continue;   // not a table for this grid
    const int64_t raster0 = u.raster0, cube0 = u.cube0, tstride = u.tstride;
    const int32_t rem_t = u.rem_t, rem_h = u.rem_h, rem_w = u.rem_w;
    auto real = [&](int32_t l) {
      if constexpr (!PAD) return true;
      return u.real(l, a);
    };
    float acc[kPooling ? E : 1];
#pragma unroll
    for (int e = 0; e < (kPooling ? E : 1); ++e) acc[e] = 0.f;
    const int32_t n_real = PAD ? rem_t * rem_h * rem_w : a.vol;
    float4 add = make_float4(0.f, 0.f, 0.f, 0.f);   // xc[c] / n_real of this thread's columns
    if (kAddPooled) {
      const float4 x = reinterpret_cast<const float4*>(xc + unit * D)[col];
      const float inv = 1.0f / (float)n_real;
      add = make_float4(x.x * inv, x.y * inv, x.z * inv, x.w * inv);
    }

    // Batches of KB rows per thread.  A full batch issues all its loads
    // before the first store; only a cube's ragged last batch is guarded.
    auto batch = [&](int32_t l0, auto guarded) {
      uint4 buf[KB];
      int64_t rrow[KB];   // raster row of token l0 + b*RG
      bool isreal[KB];    // a real token (not padding)
#pragma unroll
      for (int b = 0; b < KB; ++b) {
        const int32_t l = l0 + b * RG;
        if (!guarded.value || l < a.vol) {
          isreal[b] = real(l);
          rrow[b] = raster0 + (int64_t)row_offset(l, a) * tstride;
          if (PAD && !isreal[b])
            buf[b] = make_uint4(0u, 0u, 0u, 0u);
          else
            buf[b] = load16<kStreamLoads>(src + (kFromRaster ? rrow[b] : cube0 + l) * CPR + col);
        }
      }
#pragma unroll
      for (int b = 0; b < KB; ++b) {
        const int32_t l = l0 + b * RG;
        if (!guarded.value || l < a.vol) {
          if (PAD && !kFromRaster && !isreal[b]) continue;   // padding has no raster row
          if (kAddPooled) {
            float4 f = make_float4(__uint_as_float(buf[b].x) + add.x, __uint_as_float(buf[b].y) + add.y,
                                   __uint_as_float(buf[b].z) + add.z, __uint_as_float(buf[b].w) + add.w);
            dst[rrow[b] * CPR + col] = make_uint4(__float_as_uint(f.x), __float_as_uint(f.y),
                                                  __float_as_uint(f.z), __float_as_uint(f.w));
          } else if (kCopy) {
            dst[(kFromRaster ? cube0 + l : rrow[b]) * CPR + col] = buf[b];
          }
          if (kPooling) {
            float v[E];
            widen<T>(buf[b], v);
#pragma unroll
            for (int e = 0; e < E; ++e) acc[e] += v[e];
          }
        }
      }
    };
    int32_t l0 = phase;
    for (; l0 + (KB - 1) * RG < a.vol; l0 += KB * RG) batch(l0, std::false_type{});
    if (l0 < a.vol) batch(l0, std::true_type{});
    if (kPooling) {
#pragma unroll
      for (int e = 0; e < E; ++e) part[phase][col * E + e] = acc[e];
      __syncthreads();
      const float fvol = (float)n_real;
      for (int d = threadIdx.x; d < D; d += kThreads) {
        float s = 0.f;
#pragma unroll
        for (int p = 0; p < RG; ++p) s += part[p][d];
        xc[unit * D + d] = s / fvol;
      }
      __syncthreads();   // part is reused by the next unit
    }
  }
}

// The combination of the fine and coarse outputs as a pass of its own ("VSA:
// Accelerating Video Diffusion Inference with Sparse Attention on AMD GPUs",
// §Two-Stage Architecture: the output combines the coarse-stage and the
// fine-stage outputs through gates), for callers that keep the fine output O_f
// itself (a training forward: the backward needs O_f without gates).  Token l
// of cube c leaves for its raster row as g_f * O_f + g_c * O_c[c], formed in
// float32 from the bf16 O_f and gates in the order the fine kernel's epilogue
// uses (the product with g_f, then one fused multiply-add with g_c), rounded
// to bf16 once.  A missing gate_f reads as 1 and a missing gate_c as 0 (O_c
// is then not read): without gates the pass is the reorder back.  Padded
// positions have no raster row.  D = the output's head size; one workgroup
// per cube as in the passes above.
template <int D, bool PAD>
__global__ __launch_bounds__(kThreads) void combine_kernel(const uint4* __restrict__ o_f,
                                                           const float* __restrict__ oc,
                                                           const uint4* __restrict__ gate_c,
                                                           const uint4* __restrict__ gate_f,
                                                           uint4* __restrict__ out, CubeArgs a) {
  constexpr int CPR = D / 8;   // 16-byte chunks (8 bf16) per row
  constexpr int RG = kThreads / CPR;
  const int col = threadIdx.x % CPR;
  const int phase = threadIdx.x / CPR;
  for (int64_t unit = blockIdx.x; unit < a.units; unit += gridDim.x) {
    const UnitPos u = unit_pos(a, unit);
    if (!u.ok) continue;
    float cv[8];
    if (gate_c != nullptr) {
      const float4 c0 = reinterpret_cast<const float4*>(oc + unit * D)[2 * col];
      const float4 c1 = reinterpret_cast<const float4*>(oc + unit * D)[2 * col + 1];
      cv[0] = c0.x; cv[1] = c0.y; cv[2] = c0.z; cv[3] = c0.w;
      cv[4] = c1.x; cv[5] = c1.y; cv[6] = c1.z; cv[7] = c1.w;
    }
    for (int32_t l = phase; l < a.vol; l += RG) {
      if (PAD && !u.real(l, a)) continue;   // padding: no raster row
      const int64_t rrow = u.raster0 + (int64_t)row_offset(l, a) * u.tstride;
      float v[8];
      widen<__bf16>(o_f[(u.cube0 + l) * CPR + col], v);
      if (gate_f != nullptr) {
        float gf[8];
        widen<__bf16>(gate_f[rrow * CPR + col], gf);
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] *= gf[e];
      }
      if (gate_c != nullptr) {
        float gc[8];
        widen<__bf16>(gate_c[rrow * CPR + col], gc);
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = fmaf(gc[e], cv[e], v[e]);
      }
      out[rrow * CPR + col] = make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                                         pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7]));
    }
  }
}

CubeArgs cube_args(const Geom& g, RasterLayout layout) {
  CubeArgs a;
  a.heads = g.heads;
  a.bnhd = layout == kBNHD ? 1 : 0;
  a.T = g.T; a.H = g.H; a.W = g.W;
  a.ct = g.ct; a.ch = g.ch; a.cw = g.cw;
  a.gT = g.gT; a.gH = g.gH; a.gW = g.gW;
  a.coords = g.coords;
  a.vol = g.vol;
  a.N = (int32_t)g.N;
  a.Np = (int32_t)g.Np;
  a.Nc = (int32_t)g.Nc;
  a.padded = g.padded;
  a.units = g.BH * g.Nc;
  return a;
}

template <typename T, int MODE>
hipError_t launch_mode(const Geom& g, const void* src, void* dst, float* xc, hipStream_t s,
                       RasterLayout layout = kBHND) {
  const CubeArgs a = cube_args(g, layout);
  const dim3 grid((unsigned)(a.units < kMaxGrid ? a.units : kMaxGrid));
  if (g.D == 64 && g.padded)
    hipLaunchKernelGGL((cube_pass_kernel<T, 64, MODE, true>), grid, dim3(kThreads), 0, s, (const uint4*)src,
                       (uint4*)dst, xc, a);
  else if (g.D == 64)
    hipLaunchKernelGGL((cube_pass_kernel<T, 64, MODE, false>), grid, dim3(kThreads), 0, s, (const uint4*)src,
                       (uint4*)dst, xc, a);
  else if (g.D == 128 && g.padded)
    hipLaunchKernelGGL((cube_pass_kernel<T, 128, MODE, true>), grid, dim3(kThreads), 0, s, (const uint4*)src,
                       (uint4*)dst, xc, a);
  else if (g.D == 128)
    hipLaunchKernelGGL((cube_pass_kernel<T, 128, MODE, false>), grid, dim3(kThreads), 0, s, (const uint4*)src,
                       (uint4*)dst, xc, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

template <int MODE>
hipError_t launch_dtype(const Geom& g, int dtype, const void* src, void* dst, float* xc, hipStream_t s,
                        RasterLayout layout = kBHND) {
  return dtype == VSA_BF16 ? launch_mode<__bf16, MODE>(g, src, dst, xc, s, layout)
                           : launch_mode<float, MODE>(g, src, dst, xc, s, layout);
}

}  // namespace

hipError_t launch_reorder(const Geom& g, int dtype, const void* src, void* dst, bool to_cube,
                          hipStream_t s, RasterLayout layout) {
  return to_cube ? launch_dtype<kToCube>(g, dtype, src, dst, nullptr, s, layout)
                 : launch_dtype<kToRaster>(g, dtype, src, dst, nullptr, s, layout);
}

hipError_t launch_pool(const Geom& g, int dtype, const void* x_cube, float* xc, hipStream_t s) {
  return launch_dtype<kPool>(g, dtype, x_cube, nullptr, xc, s);
}

hipError_t launch_permute_pool(const Geom& g, int dtype, const void* x_raster, void* x_cube, float* xc,
                               hipStream_t s, RasterLayout layout) {
  if (x_cube == nullptr) return launch_dtype<kPoolRaster>(g, dtype, x_raster, nullptr, xc, s, layout);
  return launch_dtype<kToCubePool>(g, dtype, x_raster, x_cube, xc, s, layout);
}

hipError_t launch_pool_unpermute_bwd(const Geom& g, const float* dx_cube, const float* dxc, float* dx_raster,
                                     hipStream_t s, RasterLayout layout) {
  if (dxc == nullptr) return launch_mode<float, kToRaster>(g, dx_cube, dx_raster, nullptr, s, layout);
  return launch_mode<float, kToRasterAddPooled>(g, dx_cube, dx_raster, const_cast<float*>(dxc), s, layout);
}

hipError_t launch_combine(const Geom& g, const void* o_f, const float* oc, const void* gate_c, const void* gate_f,
                          void* out, hipStream_t s) {
  const CubeArgs a = cube_args(g, kBHND);
  const dim3 grid((unsigned)(a.units < kMaxGrid ? a.units : kMaxGrid));
  const auto* of4 = static_cast<const uint4*>(o_f);
  const auto* gc4 = static_cast<const uint4*>(gate_c);
  const auto* gf4 = static_cast<const uint4*>(gate_f);
  auto* out4 = static_cast<uint4*>(out);
  if (g.Dv == 64 && g.padded)
    hipLaunchKernelGGL((combine_kernel<64, true>), grid, dim3(kThreads), 0, s, of4, oc, gc4, gf4, out4, a);
  else if (g.Dv == 64)
    hipLaunchKernelGGL((combine_kernel<64, false>), grid, dim3(kThreads), 0, s, of4, oc, gc4, gf4, out4, a);
  else if (g.Dv == 128 && g.padded)
    hipLaunchKernelGGL((combine_kernel<128, true>), grid, dim3(kThreads), 0, s, of4, oc, gc4, gf4, out4, a);
  else if (g.Dv == 128)
    hipLaunchKernelGGL((combine_kernel<128, false>), grid, dim3(kThreads), 0, s, of4, oc, gc4, gf4, out4, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace vsa
