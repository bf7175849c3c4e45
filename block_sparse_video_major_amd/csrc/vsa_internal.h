// Internal declarations shared by the host entry points and the kernel
// launchers of libvsa.so.  Not part of the public ABI (include/vsa.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/vsa.h"

namespace vsa {

// Token grid and cube geometry with the derived sizes every kernel needs.
// A grid that does not divide into cubes is padded up to whole cubes: the
// cube-major tensors have Np = Nc * vol rows per (batch, head), the raster
// tensors the N real tokens.
struct Geom {
  int32_t T, H, W;        // token grid
  int32_t ct, ch, cw;     // cube edges
  int32_t gT, gH, gW;     // cube grid = grid / cube, rounded up
  int32_t vol;            // ct * ch * cw
  int64_t N;              // real tokens per (batch, head): raster rows
  int64_t Np;             // cube-major positions per (batch, head): Nc * vol
  int64_t Nc;             // cubes per (batch, head)
  int32_t padded;         // Np != N
  const int32_t* coords;  // device table of packed cube coordinates (Hilbert order), or null (raster)
  int64_t BH;             // batch * heads
  int32_t heads;          // heads per batch entry
  int32_t group;          // query heads per key/value head; key/value head of bh is bh / group
  int64_t BHkv;           // batch * key/value heads
  int32_t D;              // head_dim (queries and keys)
  int32_t Dv;             // value head size (head_dim_v, or head_dim)
};

inline Geom make_geom(const vsa_problem& p) {
  Geom g;
  g.T = p.T; g.H = p.H; g.W = p.W;
  g.ct = p.ct; g.ch = p.ch; g.cw = p.cw;
  g.gT = (int32_t)(((int64_t)p.T + p.ct - 1) / p.ct);
  g.gH = (int32_t)(((int64_t)p.H + p.ch - 1) / p.ch);
  g.gW = (int32_t)(((int64_t)p.W + p.cw - 1) / p.cw);
  g.vol = p.ct * p.ch * p.cw;
  g.N = (int64_t)p.T * p.H * p.W;
  g.Nc = (int64_t)g.gT * g.gH * g.gW;
  g.Np = g.Nc * g.vol;
  g.padded = g.Np != g.N ? 1 : 0;
  g.coords = p.cube_order == VSA_CUBES_RASTER ? nullptr : p.cube_coords;
  g.BH = (int64_t)p.batch * p.heads;
  g.heads = p.heads;
  g.group = p.heads_kv > 0 ? p.heads / p.heads_kv : 1;
  g.BHkv = g.BH / g.group;
  g.D = p.head_dim;
  g.Dv = p.head_dim_v > 0 ? p.head_dim_v : p.head_dim;
  return g;
}

// Launchers (each returns the hipGetLastError() of its launch).
// Raster-side row order of the reorder kernels: [batch, heads, N, d] or the
// model's [batch, N, heads, d].
enum RasterLayout { kBHND = 0, kBNHD = 1 };
hipError_t launch_reorder(const Geom& g, int dtype, const void* src, void* dst, bool to_cube,
                          hipStream_t s, RasterLayout layout = kBHND);
hipError_t launch_pool(const Geom& g, int dtype, const void* x_cube, float* xc, hipStream_t s);
hipError_t launch_permute_pool(const Geom& g, int dtype, const void* x_raster, void* x_cube, float* xc,
                               hipStream_t s, RasterLayout layout = kBHND);
hipError_t launch_coarse_topk(const Geom& g, int top_k, const float* qc, const float* kc,
                              const float* vc, int32_t* lut, int32_t* valid, float* oc,
                              hipStream_t s);
// Whether the fine kernel handles this cube count and LUT row length.
bool sparse_attn_fwd_fits(const Geom& g, int max_kv);
// Fine forward when the value head size differs from the query/key head
// size (d_qk, d_v) in {(128, 64), (64, 128)}; same arguments and output
// orders as launch_sparse_attn_fwd, with v, out, the gates and oc d_v wide.
bool sparse_attn_fwd_dv_fits(const Geom& g, int max_kv);
hipError_t launch_sparse_attn_fwd_dv(const Geom& g, const void* q, const void* k, const void* v,
                                     const int32_t* lut, const int32_t* valid, int max_kv, const float* oc,
                                     const void* gate_c, const void* gate_f, void* out, float* lse, int out_order,
                                     hipStream_t s);
// The fine forward over quads of query cubes (d = d_v in {64, 128}), used
// whenever its step list and load ring fit in LDS; same arguments as below.
bool sparse_attn_fwd_quad_fits(const Geom& g, int max_kv);
hipError_t launch_sparse_attn_fwd_quad(const Geom& g, const void* q, const void* k, const void* v,
                                       const int32_t* lut, const int32_t* valid, int max_kv, const float* oc,
                                       const void* gate_c, const void* gate_f, void* out, float* lse,
                                       int out_order, hipStream_t s);
// out_order: 0 cube-major, 1 raster, 2 raster [batch, N, heads, d].  With
// gather, q, k and v are in raster [batch, heads, N, d] order and the pair
// kernel gathers their cube tiles itself (out_order 1 only; see
// sparse_attn_fwd_gather_fits).
hipError_t launch_sparse_attn_fwd(const Geom& g, const void* q, const void* k, const void* v,
                                  const int32_t* lut, const int32_t* valid, int max_kv,
                                  const float* oc, const void* gate_c, const void* gate_f,
                                  void* out, float* lse, int out_order, hipStream_t s, bool gather = false);
// Whether the gathering pair kernel handles this problem: d = d_v = 128,
// cubes 4 tokens wide (one 1 KiB run per piece of a tile), a grid that
// divides into cubes, and the pair kernel's limits.
bool sparse_attn_fwd_gather_fits(const Geom& g, int max_kv);
hipError_t launch_check_lut(const Geom& g, const int32_t* lut, const int32_t* valid, int max_kv,
                            int32_t* bad_rows, hipStream_t s);
hipError_t launch_mask_to_lut(const Geom& g, const uint8_t* mask, int max_kv, int32_t* lut, int32_t* valid,
                              int32_t* overflow_rows, hipStream_t s);

// Backward of the fine stage: the workspace it needs (bytes), whether it
// handles this geometry, and the launcher (prep, transposed index list, dQ,
// then dK/dV, all on stream s).
size_t sparse_attn_bwd_workspace(const Geom& g, int max_kv);
bool sparse_attn_bwd_fits(const Geom& g, int max_kv);
hipError_t launch_sparse_attn_bwd(const Geom& g, const void* q, const void* k, const void* v, const int32_t* lut,
                                  const int32_t* valid, int max_kv, const void* o, const float* lse,
                                  const void* dout, float* dq, float* dk, float* dv, void* workspace,
                                  hipStream_t s);

// Backward of the other steps: the gated combination (cube-major), the coarse
// attention (workspace: P and dS, 2 * BH * Nc^2 floats) and the reorder back
// with the pooled gradient added (float32).
hipError_t launch_combine_bwd(const Geom& g, const void* dout, const void* of, const float* oc, const void* gate_c,
                              const void* gate_f, void* d_of, float* d_oc, float* d_gate_c, float* d_gate_f,
                              hipStream_t s);
size_t coarse_bwd_workspace(const Geom& g);
hipError_t launch_coarse_bwd(const Geom& g, const float* qc, const float* kc, const float* vc, const float* oc,
                             const float* doc, float* dqc, float* dkc, float* dvc, void* workspace, hipStream_t s);
hipError_t launch_pool_unpermute_bwd(const Geom& g, const float* dx_cube, const float* dxc, float* dx_raster,
                                     hipStream_t s, RasterLayout layout = kBHND);
// out (raster, Dv wide) = g_f * O_f (cube-major) + g_c * O_c per cube; null
// gates read as g_f = 1, g_c = 0.
hipError_t launch_combine(const Geom& g, const void* o_f, const float* oc, const void* gate_c, const void* gate_f,
                          void* out, hipStream_t s);

// Largest number of cubes per (batch, head) the coarse stage handles.
constexpr int64_t kMaxCoarseCubes = 4096;
// ... and the backward (one LDS counter per key cube in the list build).
constexpr int64_t kMaxBwdCubes = 8192;

// Workgroups are handed to the 8 XCDs of an MI355X round-robin by id.  This
// maps a hardware id to a logical id so that each XCD receives one contiguous
// range of logical ids (neighbouring query cubes share key/value cubes, and
// each XCD has its own L2).  Bijective on [0, total).
__device__ __forceinline__ int64_t xcd_remap(int64_t hw_id, int64_t total) {
  constexpr int kXcd = 8;
  const int64_t q = total / kXcd, r = total % kXcd;
  const int64_t x = hw_id % kXcd, idx = hw_id / kXcd;
  return (x < r) ? x * (q + 1) + idx : r * (q + 1) + (x - r) * q + idx;
}

}  // namespace vsa
