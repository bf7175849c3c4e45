// Where the fine forward kernels read and write each token: the cube-major
// order of a problem, its raster (t, h, w) order and the model's
// [batch, N, heads, d] rows; which cube positions hold real tokens when the
// grid was padded up to whole cubes; and the grid coordinates of a cube in
// the problem's cube order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "vsa_internal.h"

namespace vsa {

inline constexpr int kCubeTokens = 64;   // positions per cube in the fine kernels

// Token order of out, gate_c, gate_f and lse: cube-major (on == 0) or raster
// (t, h, w) order (on == 1; the reorder back fused into the epilogue).  A
// grid padded up to whole cubes has positions with no token: they are never
// keys and, in raster order, have no output row.  With
// bnhd == 1 (raster only) out and the gates are the model's [batch, N, heads,
// d] rows instead of [batch, heads, N, d]; lse stays [batch, heads, N].
struct TokenMap {
  int32_t on;
  int32_t bnhd;
  int32_t T, H, W;      // token grid (frames, rows and columns of a frame)
  int32_t ct, ch, cw;   // cube edges
  int32_t gT, gH, gW;   // cube grid
  const int32_t* coords;  // packed grid coordinates of each cube (Hilbert order), or null (raster)
  int32_t heads;        // heads per batch entry
  int32_t N;            // real tokens per (batch, head): raster rows
  int32_t Np;           // cube-major positions per (batch, head)
  int32_t padded;       // the grid was padded up to whole cubes
  int32_t mag_plane;    // ceil(2^16 / (ch * cw)): see small_div
  int32_t mag_cw;       // ceil(2^16 / cw)
};

// l / d for 0 <= l < 64 and 1 <= d <= 64, as (l * ceil(2^16 / d)) >> 16.
// With ceil(2^16 / d) = (2^16 + e) / d, 0 <= e < d, the product over 2^16
// is l / d + l e / (d 2^16), and the added term is below l / 2^16 < 1 / d,
// so it never carries the quotient past the next multiple: the result is
// exact.  One 24-bit multiply and a shift instead of an integer division.
__device__ __forceinline__ int32_t small_div(int32_t l, int32_t mag) {
  return (int32_t)(((uint32_t)l * (uint32_t)mag) >> 16);
}

// Grid coordinates of cube c: raster order over the cube grid, or the
// problem's table of packed coordinates.  A table entry outside the grid
// (a table written for another problem) marks the cube invalid: it then has
// no real token, so it is never read as keys or written in raster order.
struct CubeAt {
  int32_t t, h, w;
  bool ok;
};

__device__ __forceinline__ CubeAt cube_at(const TokenMap& m, int32_t c) {
  CubeAt r;
  if (m.coords != nullptr) {
    const int32_t e = m.coords[c];
    r.t = (e >> 20) & 1023;
    r.h = (e >> 10) & 1023;
    r.w = e & 1023;
    r.ok = r.t < m.gT && r.h < m.gH && r.w < m.gW;
  } else {
    r.w = c % m.gW;
    r.h = (c / m.gW) % m.gH;
    r.t = c / (m.gW * m.gH);
    r.ok = true;
  }
  return r;
}

// Whether position l of cube q holds a real token (not padding).
__device__ __forceinline__ bool token_real(const TokenMap& m, const CubeAt& q, int32_t l) {
  const int32_t lt = small_div(l, m.mag_plane), rem = l - lt * (m.ch * m.cw);
  const int32_t lh = small_div(rem, m.mag_cw), lw = rem - lh * m.cw;
  return q.ok && q.t * m.ct + lt < m.T && q.h * m.ch + lh < m.H && q.w * m.cw + lw < m.W;
}

// Bit l set when position l of cube q holds a real token.  The cube edges
// multiply to 64 positions; tokens run w fastest, then h, then t.
__device__ __forceinline__ uint64_t cube_mask(const TokenMap& m, const CubeAt& q) {
  if (!q.ok) return 0;
  const int32_t rt = min(m.ct, m.T - q.t * m.ct), rh = min(m.ch, m.H - q.h * m.ch), rw = min(m.cw, m.W - q.w * m.cw);
  const uint64_t row = rw >= 64 ? ~0ull : ((1ull << rw) - 1);
  uint64_t plane = 0, all = 0;
  for (int32_t h = 0; h < rh; ++h) plane |= row << (h * m.cw);
  for (int32_t t = 0; t < rt; ++t) all |= plane << (t * m.ch * m.cw);
  return all;
}

// Whether cube q reaches past the grid (holds padded positions).
__device__ __forceinline__ bool cube_partial(const TokenMap& m, const CubeAt& q) {
  return !q.ok || (q.t + 1) * m.ct > m.T || (q.h + 1) * m.ch > m.H || (q.w + 1) * m.cw > m.W;
}

// Position of token l (< 64) of cube c (coordinates q) within its (batch,
// head) in the order the map selects.
__device__ __forceinline__ int32_t token_pos(const TokenMap& m, int32_t c, const CubeAt& q, int32_t l) {
  if (!m.on) return c * kCubeTokens + l;
  const int32_t lt = small_div(l, m.mag_plane), rem = l - lt * (m.ch * m.cw);
  const int32_t lh = small_div(rem, m.mag_cw), lw = rem - lh * m.cw;
  return ((q.t * m.ct + lt) * m.H + q.h * m.ch + lh) * m.W + q.w * m.cw + lw;
}

// Element offset of token l of cube c (coordinates q) of (batch, head) bh in
// out and the gates.
__device__ __forceinline__ int64_t token_elem(const TokenMap& m, int64_t bh, int32_t c, const CubeAt& q, int32_t l,
                                              int D) {
  const int64_t n = token_pos(m, c, q, l);
  if (!m.on) return (bh * m.Np + n) * D;
  if (!m.bnhd) return (bh * m.N + n) * D;
  const int64_t b = bh / m.heads, h = bh - b * m.heads;
  return ((b * m.N + n) * m.heads + h) * D;
}

// out_order: 0 cube-major, 1 raster [batch, heads, N, d], 2 raster
// [batch, N, heads, d].
inline TokenMap make_token_map(const Geom& g, int out_order) {
  TokenMap m;
  m.on = out_order != 0 ? 1 : 0;
  m.bnhd = out_order == 2 ? 1 : 0;
  m.heads = g.heads;
  m.N = (int32_t)g.N;
  m.Np = (int32_t)g.Np;
  m.padded = g.padded;
  m.T = g.T; m.H = g.H; m.W = g.W;
  m.ct = g.ct; m.ch = g.ch; m.cw = g.cw;
  m.gT = g.gT; m.gH = g.gH; m.gW = g.gW;
  m.coords = g.coords;
  m.mag_plane = (int32_t)((65536 + g.ch * g.cw - 1) / (g.ch * g.cw));
  m.mag_cw = (int32_t)((65536 + g.cw - 1) / g.cw);
  return m;
}

}  // namespace vsa
