// Fine block-sparse attention with the gated combination when the value head
// size differs from the query/key head size, for gfx950.
//
// Same computation as sparse_attn_fwd.hip: "VSA: Accelerating Video
// Diffusion Inference with Sparse Attention on AMD GPUs", §Two-Stage
// Architecture (Stage 2: token-level attention over the selected key/value
// cubes, combined with the coarse output through gates), §Block-Sparse
// Encoding, §Kernel Architecture and §Sparse Traversal; the value head size
// of its own is the hdim_v of the CK interface (§Using VSA with CK Tile).
// Softmax(QK^T / sqrt(d)) V with d the query/key head size (§The Attention
// Bottleneck in Video Diffusion).
//
// Work decomposition (the tile layout and operand reads of the fine
// backward, tile_ops.h):
//   * One workgroup of four wavefronts per query cube, two workgroups per
//     CU; wave w owns query half qh = w & 1 (32 of the cube's 64 queries)
//     and key half kh = w >> 1 (32 of the 64 tokens of each key cube).
//   * S^T = K Q^T on the matrix cores (v_mfma_f32_32x32x16_bf16, DQ / 16
//     k-steps; K rows from LDS as A, Q in registers as B): each lane owns one
//     query and 16 of the wave's keys, so the softmax state is lane-local and
//     the row max needs one v_permlane32_swap.
//   * O^T += V^T P^T: P in registers is already the B operand; V^T comes
//     from the V tile by transposing LDS reads (DV / 32 output tiles).
//   * The K and V tiles (64 x DQ and 64 x DV bf16) of the next listed cube
//     load by direct global->LDS loads while the current ones are used: two
//     stages, one barrier per step.  The offset of the exponentials moves
//     lazily, only when a block's max exceeds it by more than 8 (log2 units).
//   * The two key halves' softmax states are merged through LDS, O is
//     normalised and staged in LDS, then combined with the gates and the
//     broadcast coarse output and written with 16-byte stores in the token
//     order of the map (cube-major, raster, or [batch, N, heads, d]).
#include <mutex>

#include "tile_ops.h"
#include "token_map.h"

namespace vsa {
namespace {

constexpr float kTauDv = 8.0f;          // lazy-rescale threshold (log2 units)
constexpr float kNegBigDv = -1.0e30f;   // initial exponent offset: finite, so no inf - inf

__device__ __forceinline__ float pair_max32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float pair_sum32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int DQ, int DV>
struct DvCfg {
  using CK = BCfg<DQ>;
  using CV = BCfg<DV>;
  static constexpr int SLOT = CK::TILE + CV::TILE;              // K tile, then V tile
  static constexpr int MERGE = 2 * (CV::OT * 16 + 2) * 64 * 4;  // key-half merge buffer, both query halves
  static constexpr int RING = 2 * SLOT;
  static constexpr int EPI = MERGE + CV::STAGE;
  static constexpr int LDS = RING > EPI ? RING : EPI;
};

template <int DQ, int DV, bool PAD>
__global__ __launch_bounds__(kThreads, 2) void sparse_attn_fwd_dv_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    const int32_t* __restrict__ lut, const int32_t* __restrict__ valid, int max_kv,
    const float* __restrict__ oc, const __bf16* __restrict__ gate_c, const __bf16* __restrict__ gate_f,
    __bf16* __restrict__ out, float* __restrict__ lse, int Nc, int64_t total_cubes, float c_log2,
    TokenMap tmap, int group) {
  using CK = BCfg<DQ>;
  using CV = BCfg<DV>;
  using C = DvCfg<DQ, DV>;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int qh = wave & 1, kh = wave >> 1;
  const int g = lane >> 5;

  const int64_t cube = xcd_remap(blockIdx.x, total_cubes);   // = LUT row
  const int64_t bh = cube / Nc;
  const int ci = (int)(cube - bh * Nc);
  const int64_t np = (int64_t)Nc * kBlk;                     // cube-major rows per head
  const int64_t kvh = bh / group;                            // its key/value head
  const char* k_head = reinterpret_cast<const char*>(k + kvh * np * DQ);
  const char* v_head = reinterpret_cast<const char*>(v + kvh * np * DV);
  const int n = clamp_count(valid[cube], max_kv);
  ListWindow lw(lut + cube * (int64_t)max_kv, n, Nc, lane);

  const LaneOffsets<DQ> ok(wave, lane, kh);
  const LaneOffsets<DV> ov(wave, lane, kh);
  const uint32_t lds_k = __builtin_amdgcn_readfirstlane(lds_addr(smem) + (uint32_t)(wave * CK::LOADS * 1024));
  const uint32_t lds_v =
      __builtin_amdgcn_readfirstlane(lds_addr(smem) + (uint32_t)(CK::TILE + wave * CV::LOADS * 1024));
  auto issue = [&](int cb, int stage) {
    dma_tile(uniform_ptr(k_head + (int64_t)cb * CK::TILE), ok.g_off, lds_k + stage * C::SLOT);
    dma_tile(uniform_ptr(v_head + (int64_t)cb * CV::TILE), ov.g_off, lds_v + stage * C::SLOT);
  };
  int cb_next = n > 0 ? lw.at(0, lane) : 0;
  if (n > 0) issue(cb_next, 0);

  // Q of this wave's 32 queries as the B operand: query 32*qh + n32, d = 16*s + 8*g + 0..7
  bf16x8 qf[CK::KS];
  load_b_operand<DQ>(q + bh * np * DQ + (int64_t)ci * kBlk * DQ, qh, lane, qf);
  f32x16 acc[CV::OT];   // O^T: rows d = 32*t + 8*(r/4) + 4*g + r%4, column = this lane's query
#pragma unroll
  for (int t = 0; t < CV::OT; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[t][r] = 0.f;
  float m_run = kNegBigDv;   // exponent offset (log2 units) of this lane's query
  float l_part = 0.f;        // this lane's partial row sum over its 16 keys per step
  wait_vmem<0>();
  __syncthreads();

  for (int s = 0; s < n; ++s) {
    const int st = s & 1;
    const int cb = cb_next;
    if (s + 1 < n) {
      cb_next = lw.at(s + 1, lane);
      issue(cb_next, st ^ 1);
    }
    const char* kt = smem + st * C::SLOT;
    const char* vt = kt + CK::TILE;
    // S^T: rows = keys 32*kh + 8*(r/4) + 4*g + r%4 of the key cube, column = query
    f32x16 sT;
#pragma unroll
    for (int r = 0; r < 16; ++r) sT[r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < CK::KS; ++ks)
      sT = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8*>(kt + ok.row_off[ks]), qf[ks],
                                                   sT, 0, 0, 0);
    if constexpr (PAD) {
      // padded positions of a key cube that reaches past the grid are not keys
      const CubeAt kc = cube_at(tmap, cb);
      if (cube_partial(tmap, kc)) {
        const uint64_t m = cube_mask(tmap, kc) >> (32 * kh + 4 * g);
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (!((m >> (8 * (r >> 2) + (r & 3))) & 1ull)) sT[r] = -INFINITY;
      }
    }
    float mx = kNegBigDv;
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sT[r]);
    mx = pair_max32(mx) * c_log2;
    if (__ballot(mx > m_run + kTauDv) != 0ull) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      l_part *= alpha;
#pragma unroll
      for (int t = 0; t < CV::OT; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[t][r] *= alpha;
      m_run = m_new;
    }
    // P^T as the B operand: k-step j holds registers 8j..8j+7
    bf16x8 pb[2];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p = __builtin_amdgcn_exp2f(fmaf(sT[r], c_log2, -m_run));
      l_part += p;
      pb[r >> 3][r & 7] = (__bf16)p;
    }
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int t = 0; t < CV::OT; ++t)
        acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_tr<DV>(vt, ov, t, j), pb[j], acc[t], 0, 0, 0);
    wait_vmem<0>();
    __syncthreads();
  }

  // ---- merge the two key halves, normalise, stage ----
  const float l_row = pair_sum32(l_part);
  float* mbuf = reinterpret_cast<float*>(smem) + qh * (CV::OT * 16 + 2) * 64;   // [2 + 16*OT][64]
  float* stg = reinterpret_cast<float*>(smem + C::MERGE);                        // [64][SSTR]
  if (kh == 1) {
    mbuf[lane] = m_run;
    mbuf[64 + lane] = l_row;
#pragma unroll
    for (int t = 0; t < CV::OT; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) mbuf[(2 + t * 16 + r) * 64 + lane] = acc[t][r];
  }
  __syncthreads();
  const CubeAt mq = tmap.on ? cube_at(tmap, ci) : CubeAt{0, 0, 0, true};
  if (kh == 0) {
    const float m1 = mbuf[lane], l1 = mbuf[64 + lane];
    const float m = fmaxf(m_run, m1);
    const float a0 = __builtin_amdgcn_exp2f(m_run - m), a1 = __builtin_amdgcn_exp2f(m1 - m);
    const float l = l_row * a0 + l1 * a1;
    const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
    for (int t = 0; t < CV::OT; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[t][r] = acc[t][r] * a0 + mbuf[(2 + t * 16 + r) * 64 + lane] * a1;
    stage_store<DV>(stg, acc, qh, lane, inv);
    const int32_t my_tok = 32 * qh + (lane & 31);
    if (lse != nullptr && g == 0 && mq.ok && (!PAD || !tmap.on || token_real(tmap, mq, my_tok))) {
      const float val = l > 0.f ? (m + __log2f(l)) * 0.69314718055994531f : -INFINITY;
      lse[bh * (int64_t)(tmap.on ? tmap.N : tmap.Np) + token_pos(tmap, ci, mq, my_tok)] = val;
    }
  }
  __syncthreads();

  // ---- combine with the gates and O_c, write in the map's token order ----
  if (!mq.ok) return;
  const float* ocrow = oc != nullptr ? oc + cube * (int64_t)DV : nullptr;
#pragma unroll
  for (int u = 0; u < kBlk * CV::CPR / kThreads; ++u) {
    const int c = tid + u * kThreads;
    const int row = c / CV::CPR, col = c % CV::CPR;
    if (PAD && tmap.on && !token_real(tmap, mq, row)) continue;   // padding: no raster row
    const int64_t gidx = token_elem(tmap, bh, ci, mq, row, DV) + col * 8;
    const float4 v0 = *reinterpret_cast<const float4*>(stg + row * CV::SSTR + col * 8);
    const float4 v1 = *reinterpret_cast<const float4*>(stg + row * CV::SSTR + col * 8 + 4);
    float val[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
    if (gate_f != nullptr) {
      float gf[8];
      unpack_bf16x8(*reinterpret_cast<const uint4*>(gate_f + gidx), gf);
#pragma unroll
      for (int e = 0; e < 8; ++e) val[e] *= gf[e];
    }
    if (gate_c != nullptr) {
      float gc[8];
      unpack_bf16x8(*reinterpret_cast<const uint4*>(gate_c + gidx), gc);
      const float4 c0 = *reinterpret_cast<const float4*>(ocrow + col * 8);
      const float4 c1 = *reinterpret_cast<const float4*>(ocrow + col * 8 + 4);
      const float cv[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) val[e] = fmaf(gc[e], cv[e], val[e]);
    }
    uint4 packed;
    packed.x = pack_bf16x2(val[0], val[1]);
    packed.y = pack_bf16x2(val[2], val[3]);
    packed.z = pack_bf16x2(val[4], val[5]);
    packed.w = pack_bf16x2(val[6], val[7]);
    *reinterpret_cast<uint4*>(out + gidx) = packed;
  }
}

template <int DQ, int DV, bool PAD>
hipError_t launch_dv(const Geom& g, const void* q, const void* k, const void* v, const int32_t* lut,
                     const int32_t* valid, int max_kv, const float* oc, const void* gate_c, const void* gate_f,
                     void* out, float* lse, const TokenMap& tmap, hipStream_t s) {
  static int granted[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  constexpr int lds = DvCfg<DQ, DV>::LDS;
  auto kern = sparse_attn_fwd_dv_kernel<DQ, DV, PAD>;
  {
    static std::mutex mu;   // host threads may launch concurrently
    std::lock_guard<std::mutex> lock(mu);
    if (granted[dev] < lds) {
      const hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
      if (e != hipSuccess) return e;
      granted[dev] = lds;
    }
  }
  const int64_t total_cubes = g.BH * g.Nc;
  const float c_log2 = kLog2e / sqrtf((float)DQ);
  hipLaunchKernelGGL(kern, dim3((unsigned)total_cubes), dim3(kThreads), lds, s, (const __bf16*)q,
                     (const __bf16*)k, (const __bf16*)v, lut, valid, max_kv, oc, (const __bf16*)gate_c,
                     (const __bf16*)gate_f, (__bf16*)out, lse, (int)g.Nc, total_cubes, c_log2, tmap, g.group);
  return hipGetLastError();
}

template <int DQ, int DV>
hipError_t launch_pad(const Geom& g, const void* q, const void* k, const void* v, const int32_t* lut,
                      const int32_t* valid, int max_kv, const float* oc, const void* gate_c, const void* gate_f,
                      void* out, float* lse, const TokenMap& tmap, hipStream_t s) {
  if (g.padded)
    return launch_dv<DQ, DV, true>(g, q, k, v, lut, valid, max_kv, oc, gate_c, gate_f, out, lse, tmap, s);
  return launch_dv<DQ, DV, false>(g, q, k, v, lut, valid, max_kv, oc, gate_c, gate_f, out, lse, tmap, s);
}

}  // namespace

bool sparse_attn_fwd_dv_fits(const Geom& g, int max_kv) {
  return g.Nc >= 1 && max_kv >= 1 && g.BH * g.Nc < ((int64_t)1 << 31) &&
         ((g.D == 128 && g.Dv == 64) || (g.D == 64 && g.Dv == 128));
}

hipError_t launch_sparse_attn_fwd_dv(const Geom& g, const void* q, const void* k, const void* v,
                                     const int32_t* lut, const int32_t* valid, int max_kv, const float* oc,
                                     const void* gate_c, const void* gate_f, void* out, float* lse, int out_order,
                                     hipStream_t s) {
  const TokenMap m = make_token_map(g, out_order);
  if (g.D == 128 && g.Dv == 64)
    return launch_pad<128, 64>(g, q, k, v, lut, valid, max_kv, oc, gate_c, gate_f, out, lse, m, s);
  if (g.D == 64 && g.Dv == 128)
    return launch_pad<64, 128>(g, q, k, v, lut, valid, max_kv, oc, gate_c, gate_f, out, lse, m, s);
  return hipErrorInvalidValue;
}

}  // namespace vsa
