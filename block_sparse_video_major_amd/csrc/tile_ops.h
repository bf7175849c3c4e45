// Tile helpers shared by the kernels that give each query or key cube a
// workgroup of four wavefronts (the fine backward, and the forward for a
// value head size different from the query/key head size): 64-token bf16
// tiles in LDS under one chunk swizzle, direct global->LDS loads, the MFMA
// operand reads of both layouts (row reads and transposing reads), fp32
// staging of accumulator tiles and a register window over an index list.
#pragma once

#include "mfma_util.h"
#include "vsa_internal.h"

namespace vsa {

inline constexpr int kBlk = 64;            // tokens per cube
inline constexpr int kThreads = 256;       // four wavefronts per cube
inline constexpr float kLog2e = 1.4426950408889634f;

template <int D>
struct BCfg {
  static constexpr int ROWB = D * 2;                       // bytes per token row
  static constexpr int CPR = D / 8;                        // 16-byte chunks per row
  static constexpr int TILE = kBlk * ROWB;                 // one 64-token tile
  static constexpr int LOADS = TILE / (kThreads * 16);     // 16-byte loads per lane per tile
  static constexpr int OT = D / 32;                        // 32-row tiles of a d x 32 product
  static constexpr int KS = D / 16;                        // k-steps of a contraction over d
  static constexpr int SSTR = D + 4;                       // fp32 staging row stride
  static constexpr int STAGE = kBlk * SSTR * 4;            // one 64 x d fp32 staging tile
  // Logical 16-byte chunk c of row r sits at c ^ swz(r).  Row reads touch 16
  // consecutive rows at one chunk: swz is a bijection on every aligned group
  // of 16 rows (d = 128) or on the 8 rows of one parity in it (d = 64, two
  // rows per 256 bytes).  Transposing reads touch 4 consecutive rows (aligned
  // to 4) at 4 consecutive chunks: bits 2-3 of swz differ across those rows.
  __device__ static constexpr int swz(int r) {
    return D == 128 ? ((4 * (r & 3)) | ((r >> 2) & 3)) : ((4 * ((r >> 1) & 1)) | ((r >> 2) & 3));
  }
};

__device__ __forceinline__ int clamp_cube(int c, int Nc) { return c < 0 ? 0 : (c >= Nc ? Nc - 1 : c); }
__device__ __forceinline__ int clamp_count(int n, int max_kv) { return n < 0 ? 0 : (n > max_kv ? max_kv : n); }

// One 16-byte direct global->LDS load per lane: base + voff -> lds_base + 16 * lane.
__device__ __forceinline__ void dma_piece(const void* base, uint32_t voff, uint32_t lds_base) {
  lds_base = __builtin_amdgcn_readfirstlane(lds_base);
  asm volatile(
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, %2"
      :
      : "v"(voff), "s"(lds_base), "s"(base)
      : "memory", "m0");
}

// Piece N of a tile by direct load: every lane moves the 16 bytes at
// base + voff + 1024 N to LDS byte address lds_base + 1024 N + 16 * lane
// (voff as in the tile offsets, which subtract 1024 N).  Issuing the pieces of
// a step one at a time between MFMAs keeps the CU's address unit (about 16
// cycles per 1 KiB piece) from backing up and stalling the issuing waves.
template <int N>
__device__ __forceinline__ void dma_one(const void* base, uint32_t voff, uint32_t lds_base) {
  lds_base = __builtin_amdgcn_readfirstlane(lds_base);
  asm volatile(
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, %2 offset:%3"
      :
      : "v"(voff), "s"(lds_base), "s"(base), "i"(N * 1024)
      : "memory", "m0");
}

// Per-lane LDS offsets shared by both gradient kernels.  `half` is the 32-row
// half of the tile this wave reads as MFMA A operands (key half in the dQ
// kernel, query half in the dK/dV kernel).
template <int D>
struct LaneOffsets {
  using C = BCfg<D>;
  uint32_t g_off[C::LOADS];   // direct-load source offsets (minus the instruction offset)
  int row_off[C::KS];         // row reads: row 32*half + n32, logical chunk 2*ks + g
  int tr_off[C::OT][2];       // transposing reads, row step 8*hi
  __device__ __forceinline__ LaneOffsets(int wave, int lane, int half) {
    const int n32 = lane & 31, g = lane >> 5, l16 = lane & 15, h16 = (lane >> 4) & 1;
#pragma unroll
    for (int n = 0; n < C::LOADS; ++n) {
      const int L = (wave * C::LOADS + n) * 64 + lane;
      const int r = L / C::CPR, x = L % C::CPR;
      g_off[n] = (uint32_t)(r * C::ROWB + ((x ^ C::swz(r)) * 16) - n * 1024);
    }
    {
      const int r = 32 * half + n32;
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) row_off[ks] = r * C::ROWB + (((2 * ks + g) ^ C::swz(r)) * 16);
    }
    // Source lane l16 of a transposing read addresses row
    // 32*half + 16*j + 8*hi + 4*g + l16/4 and columns 32*t + 16*h16 + 4*(l16%4);
    // the 16*j row step leaves the swizzle unchanged and is added at the read.
#pragma unroll
    for (int hi = 0; hi < 2; ++hi) {
      const int r = 32 * half + 8 * hi + 4 * g + (l16 >> 2);
      const int byte_base = 32 * h16 + 8 * (l16 & 3);
#pragma unroll
      for (int t = 0; t < C::OT; ++t) {
        const int b = 64 * t + byte_base;
        tr_off[t][hi] = r * C::ROWB + ((((b >> 4) ^ C::swz(r)) << 4) | (b & 15));
      }
    }
  }
};

// A operand of a d x 16 block of a transposed tile: for k-step j, the lane of
// (g, row m) receives tile rows 32*half + 16*j + 4*g + {0..3, 8..11} at column
// 32*t + m, the row order in which a lane of an accumulator holds its 16 rows.
template <int D>
__device__ __forceinline__ bf16x8 read_tr(const char* tile, const LaneOffsets<D>& o, int t, int j) {
  using C = BCfg<D>;
  const i16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tile + o.tr_off[t][0] + (16 * j) * C::ROWB));
  const i16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tile + o.tr_off[t][1] + (16 * j) * C::ROWB));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
}

// 32 tokens x d of a cube tile as MFMA B operands: token 32*half + n32,
// columns 16*s + 8*g + 0..7.
template <int D>
__device__ __forceinline__ void load_b_operand(const __bf16* tile_rows, int half, int lane, bf16x8 (&f)[D / 16]) {
  const __bf16* row = tile_rows + (int64_t)(32 * half + (lane & 31)) * D + 8 * (lane >> 5);
#pragma unroll
  for (int s = 0; s < D / 16; ++s) f[s] = *reinterpret_cast<const bf16x8*>(row + 16 * s);
}

// Accumulator tiles acc[t] (rows d = 32*t + 8*(r/4) + 4*g + r%4, column = this
// lane's token 32*half + n32) to and from an fp32 staging tile [64][SSTR].
template <int D>
__device__ __forceinline__ void stage_store(float* stg, const f32x16 (&acc)[D / 32], int half, int lane,
                                            float mul) {
  using C = BCfg<D>;
  float* row = stg + (32 * half + (lane & 31)) * C::SSTR + 4 * (lane >> 5);
#pragma unroll
  for (int t = 0; t < C::OT; ++t)
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      float4 w;
      w.x = acc[t][4 * rq + 0] * mul;
      w.y = acc[t][4 * rq + 1] * mul;
      w.z = acc[t][4 * rq + 2] * mul;
      w.w = acc[t][4 * rq + 3] * mul;
      *reinterpret_cast<float4*>(row + 32 * t + 8 * rq) = w;
    }
}

template <int D>
__device__ __forceinline__ void stage_add(float* stg, const f32x16 (&acc)[D / 32], int half, int lane, float mul) {
  using C = BCfg<D>;
  float* row = stg + (32 * half + (lane & 31)) * C::SSTR + 4 * (lane >> 5);
#pragma unroll
  for (int t = 0; t < C::OT; ++t)
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      float4* p = reinterpret_cast<float4*>(row + 32 * t + 8 * rq);
      const float4 u = *p;
      float4 w;
      w.x = (acc[t][4 * rq + 0] + u.x) * mul;
      w.y = (acc[t][4 * rq + 1] + u.y) * mul;
      w.z = (acc[t][4 * rq + 2] + u.z) * mul;
      w.w = (acc[t][4 * rq + 3] + u.w) * mul;
      *p = w;
    }
}

// Coalesced copy of a staged 64 x d fp32 tile to 64 consecutive token rows.
template <int D>
__device__ __forceinline__ void stage_flush(const float* stg, float* dst, int tid) {
  using C = BCfg<D>;
  constexpr int V4 = D / 4;   // float4 per row
#pragma unroll
  for (int u = 0; u < kBlk * V4 / kThreads; ++u) {
    const int c = tid + u * kThreads;
    const int row = c / V4, col = c % V4;
    *reinterpret_cast<float4*>(dst + (int64_t)row * D + 4 * col) =
        *reinterpret_cast<const float4*>(stg + row * C::SSTR + 4 * col);
  }
}

// Sliding 64-entry register window over an int32 list: lane l holds
// list[win + l]; entries are clamped to [0, Nc).
struct ListWindow {
  const int32_t* list;
  int n, Nc, win, w;
  __device__ __forceinline__ ListWindow(const int32_t* l, int n_, int Nc_, int lane)
      : list(l), n(n_), Nc(Nc_), win(0) {
    w = lane < n ? clamp_cube(list[lane], Nc) : 0;
  }
  __device__ __forceinline__ int at(int s, int lane) {   // s ascending, wave-uniform
    if (s - win >= 64) {
      win += 64;
      w = win + lane < n ? clamp_cube(list[win + lane], Nc) : 0;
    }
    return __builtin_amdgcn_readlane(w, s - win);
  }
};

}  // namespace vsa
