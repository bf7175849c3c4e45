// Backward of the fine block-sparse attention stage, for gfx950.
//
// "VSA: Faster Video Diffusion with Trainable Sparse Attention", Abstract: the
// sparse attention is trained end to end, so the fine stage needs gradients
// with respect to its queries, keys and values.  The function differentiated
// is the fine attention of "VSA: Accelerating Video Diffusion Inference with
// Sparse Attention on AMD GPUs", §Two-Stage Architecture (Stage 2), over the
// index list of §Block-Sparse Encoding: for query cube i and its listed key
// cubes R, O_i = softmax(scale * Q_i K_R^T) V_R.  With the forward's
// log-sum-exp LSE and Drow = rowsum(dO * O), the attention matrix is
// recomputed as P = exp(scale * Q K^T - LSE) and
//   dP = dO V^T,   dS = P * (dP - Drow),
//   dQ = scale * dS K,   dK = scale * dS^T Q,   dV = P^T dO,
// each product summed over the listed (query cube, key cube) pairs only.
//
// Work decomposition (no atomics on any gradient; every output element is
// written once, by one workgroup, so results are identical run to run):
//   * prep: one pass over O and dO writes, per token, the 8-byte record
//     (LSE * log2 e, Drow), which both gradient kernels read.
//   * transposed index list: for every key cube, the query cubes whose rows
//     list it, ascending (a cube listed twice by one row appears twice).  With
//     grouped key/value heads the list of a key cube runs over the query cubes
//     of all the query heads that share its key/value head (their LUT rows
//     are contiguous), so dK and dV sum over the group as well.  Built
//     without ordering races in three passes: per block of 16 rows the count
//     of each key cube, one scan per (batch, head) that turns counts into
//     list offsets, and a scatter in which one wavefront walks its block's
//     rows in order (lanes of one instruction that hit the same key cube
//     carry the same query cube, so their relative order is immaterial).
//   * dQ kernel: one workgroup (4 wavefronts) per query cube walks the cube's
//     index row.  Wave w owns query half qh = w & 1 and key half kh = w >> 1.
//     Scores are formed transposed, S^T = K Q^T and dP^T = V dO^T, with Q and
//     dO in registers as MFMA B operands, so each lane owns one query and its
//     LSE and Drow are per-lane scalars; dS^T is formed in registers and
//     becomes the B operand of dQ^T += K^T dS^T, whose A operand is read from
//     the K tile with transposing LDS reads.  The two key halves are summed
//     through LDS at the end.
//   * dK/dV kernel: one workgroup per key cube walks the cube's transposed
//     list, with K and V in registers as B operands: S = Q K^T and
//     dP = dO V^T (rows = queries), P and dS formed in registers (LSE and
//     Drow of the lane's 16 queries read from LDS), then dV^T += dO^T P and
//     dK^T += Q^T dS with transposing reads of the dO and Q tiles.  The two
//     query halves are summed through LDS at the end.
//   * Tiles (64 tokens x d bf16) arrive by direct global->LDS loads, one
//     barrier per step: a two-stage ring in the dQ kernel (two workgroups
//     share a CU, so each SIMD runs two waves that cover each other's
//     stalls), a four-stage ring with two steps of loads in flight in the
//     dK/dV kernel (its 128 accumulator registers per lane leave one wave per
//     SIMD, so it overlaps the matrix cores with its own vector work in a
//     two-phase software pipeline).  One chunk swizzle serves both LDS read
//     patterns (16 consecutive rows at one 16-byte chunk, and 4 consecutive
//     rows at 4 consecutive chunks) without bank conflicts.
//   * What bounds it (32K-token layer): neither kernel reaches the matrix-core
//     bound.  Per dK/dV step (~2500 cycles against 1024 of MFMA work) the
//     direct loads cost the issuing waves ~60 cycles per 1 KiB piece while
//     the CU's load path and LDS are busy, the exponentials and dS arithmetic
//     ~700 cycles of vector issue, and barrier plus load wait ~300.
//   * Workgroups are mapped to XCDs in contiguous ranges of cubes, so the
//     workgroups sharing an L2 walk overlapping lists.
#include <mutex>

#include "tile_ops.h"

namespace vsa {
namespace {

constexpr int kRowsPerBlk = 16;     // LUT rows per block of the transposed-list build

// ---- prep: (LSE * log2 e, Drow) per token ------------------------------------
template <int D>
__global__ __launch_bounds__(256) void bwd_prep_kernel(const __bf16* __restrict__ o,
                                                       const __bf16* __restrict__ dout,
                                                       const float* __restrict__ lse, float2* __restrict__ ld,
                                                       int64_t total) {
  constexpr int TPT = D / 8;   // lanes per token, 8 elements each
  const int64_t tok = (int64_t)blockIdx.x * (256 / TPT) + threadIdx.x / TPT;
  const int part = threadIdx.x % TPT;
  float acc = 0.f;
  if (tok < total) {
    float a[8], b[8];
    unpack_bf16x8(*reinterpret_cast<const uint4*>(o + tok * D + part * 8), a);
    unpack_bf16x8(*reinterpret_cast<const uint4*>(dout + tok * D + part * 8), b);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = fmaf(a[e], b[e], acc);
  }
#pragma unroll
  for (int m = TPT / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m);
  if (tok < total && part == 0) ld[tok] = make_float2(lse[tok] * kLog2e, acc);
}

// ---- transposed index list ----------------------------------------------------
// Rows: the Nr = group * Nc LUT rows of the query heads that share one
// key/value head (grp), contiguous in the LUT.  blkcnt[grp][rb][j] = how often
// rows 16*rb .. 16*rb + 15 of the group list key cube j.
__global__ __launch_bounds__(256) void csr_count_kernel(const int32_t* __restrict__ lut,
                                                        const int32_t* __restrict__ valid, int max_kv, int Nr,
                                                        int Nc, int nrb, int32_t* __restrict__ blkcnt) {
  extern __shared__ int cnt[];
  const int64_t bh = blockIdx.x / nrb;   // the group
  const int rb = (int)(blockIdx.x - bh * nrb);
  for (int j = threadIdx.x; j < Nc; j += 256) cnt[j] = 0;
  __syncthreads();
  const int r0 = rb * kRowsPerBlk, r1 = r0 + kRowsPerBlk < Nr ? r0 + kRowsPerBlk : Nr;
  for (int i = r0; i < r1; ++i) {
    const int64_t row = bh * Nr + i;
    const int n = clamp_count(valid[row], max_kv);
    for (int e = threadIdx.x; e < n; e += 256) atomicAdd(&cnt[clamp_cube(lut[row * max_kv + e], Nc)], 1);
  }
  __syncthreads();
  int32_t* out = blkcnt + (bh * nrb + rb) * (int64_t)Nc;
  for (int j = threadIdx.x; j < Nc; j += 256) out[j] = cnt[j];
}

// Per group: blkcnt becomes the exclusive prefix over row blocks, and
// coloff[j] the start of key cube j's list (coloff[Nc] = total entries).
__global__ __launch_bounds__(256) void csr_scan_kernel(int32_t* __restrict__ blkcnt, int Nc, int nrb,
                                                       int32_t* __restrict__ coloff) {
  extern __shared__ int tot[];
  __shared__ int part[256];
  const int tid = threadIdx.x;
  const int64_t bh = blockIdx.x;
  int32_t* base = blkcnt + bh * nrb * (int64_t)Nc;
  for (int j = tid; j < Nc; j += 256) {
    int run = 0;
    for (int rb = 0; rb < nrb; ++rb) {
      int32_t* p = base + (int64_t)rb * Nc + j;
      const int c = *p;
      *p = run;
      run += c;
    }
    tot[j] = run;
  }
  __syncthreads();
  const int per = (Nc + 255) / 256;
  const int j0 = tid * per, j1 = j0 + per < Nc ? j0 + per : Nc;
  int s = 0;
  for (int j = j0; j < j1; ++j) s += tot[j];
  part[tid] = s;
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int i = 0; i < 256; ++i) {
      const int c = part[i];
      part[i] = run;
      run += c;
    }
  }
  __syncthreads();
  int run = part[tid];
  int32_t* co = coloff + bh * (int64_t)(Nc + 1);
  for (int j = j0; j < j1; ++j) {
    co[j] = run;
    run += tot[j];
  }
  if (tid == 255) co[Nc] = run;
}

// One wavefront per row block writes the query cube of every listing into its
// key cube's list, rows in ascending order.
__global__ __launch_bounds__(64) void csr_scatter_kernel(const int32_t* __restrict__ lut,
                                                         const int32_t* __restrict__ valid, int max_kv, int Nr,
                                                         int Nc, int nrb, const int32_t* __restrict__ blkcnt,
                                                         const int32_t* __restrict__ coloff,
                                                         int32_t* __restrict__ csr) {
  extern __shared__ int cur[];
  const int lane = threadIdx.x;
  const int64_t bh = blockIdx.x / nrb;
  const int rb = (int)(blockIdx.x - bh * nrb);
  const int32_t* bc = blkcnt + (bh * nrb + rb) * (int64_t)Nc;
  const int32_t* co = coloff + bh * (int64_t)(Nc + 1);
  for (int j = lane; j < Nc; j += 64) cur[j] = co[j] + bc[j];
  __syncthreads();
  int32_t* out = csr + bh * (int64_t)Nr * max_kv;
  const int r0 = rb * kRowsPerBlk, r1 = r0 + kRowsPerBlk < Nr ? r0 + kRowsPerBlk : Nr;
  for (int i = r0; i < r1; ++i) {
    const int64_t row = bh * Nr + i;
    const int n = clamp_count(valid[row], max_kv);
    for (int e0 = 0; e0 < n; e0 += 64) {
      const int e = e0 + lane;
      if (e < n) {
        const int j = clamp_cube(lut[row * max_kv + e], Nc);
        out[atomicAdd(&cur[j], 1)] = i;
      }
    }
  }
}

// ---- dQ -------------------------------------------------------------------------
// D: query/key head size, DV: value head size (dP^T contracts over DV).
template <int D, int DV = D>
__global__ __launch_bounds__(kThreads) void sparse_attn_bwd_dq_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    const __bf16* __restrict__ dout, const int32_t* __restrict__ lut, const int32_t* __restrict__ valid,
    int max_kv, const float2* __restrict__ ld, float* __restrict__ dq, int Nc, int64_t total_cubes,
    float c_log2, float scale, int group) {
  using C = BCfg<D>;
  using CV = BCfg<DV>;
  constexpr int SLOT = C::TILE + CV::TILE;   // K tile, then V tile
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int qh = wave & 1, kh = wave >> 1;

  const int64_t cube = xcd_remap(blockIdx.x, total_cubes);   // = LUT row
  const int64_t bh = cube / Nc;
  const int ci = (int)(cube - bh * Nc);
  const int64_t rows_off = bh * (int64_t)Nc * kBlk;                  // this head's first row
  const int64_t kv_rows = (bh / group) * (int64_t)Nc * kBlk;         // its key/value head's
  const char* k_head = reinterpret_cast<const char*>(k + kv_rows * D);
  const char* v_head = reinterpret_cast<const char*>(v + kv_rows * DV);
  const int n = clamp_count(valid[cube], max_kv);
  ListWindow lw(lut + cube * (int64_t)max_kv, n, Nc, lane);

  const LaneOffsets<D> off(wave, lane, kh);
  const LaneOffsets<DV> offv(wave, lane, kh);
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_addr(smem) + (uint32_t)(wave * C::LOADS * 1024));
  const uint32_t lds0v =
      __builtin_amdgcn_readfirstlane(lds_addr(smem) + (uint32_t)(C::TILE + wave * CV::LOADS * 1024));
  auto issue = [&](int s, int stage) {
    const int cb = lw.at(s, lane);
    dma_tile(uniform_ptr(k_head + (int64_t)cb * C::TILE), off.g_off, lds0 + stage * SLOT);
    dma_tile(uniform_ptr(v_head + (int64_t)cb * CV::TILE), offv.g_off, lds0v + stage * SLOT);
  };
  if (n > 0) issue(0, 0);

  // Q and dO of this wave's 32 queries as B operands; this lane's query
  // 32*qh + n32 has its (LSE * log2 e, Drow) in registers.
  bf16x8 qf[C::KS], df[CV::KS];
  load_b_operand<D>(q + (rows_off + (int64_t)ci * kBlk) * D, qh, lane, qf);
  load_b_operand<DV>(dout + (rows_off + (int64_t)ci * kBlk) * DV, qh, lane, df);
  const float2 ldv = ld[cube * kBlk + 32 * qh + (lane & 31)];
  f32x16 acc[C::OT];
#pragma unroll
  for (int t = 0; t < C::OT; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[t][r] = 0.f;
  wait_vmem<0>();
  __syncthreads();

  for (int s = 0; s < n; ++s) {
    const int st = s & 1;
    if (s + 1 < n) issue(s + 1, st ^ 1);
    const char* kt = smem + st * SLOT;
    const char* vt = kt + C::TILE;
    f32x16 sT, pT;   // S^T and dP^T: rows = keys 32*kh + 8*(r/4) + 4*g + r%4, column = query
#pragma unroll
    for (int r = 0; r < 16; ++r) { sT[r] = 0.f; pT[r] = 0.f; }
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(kt + off.row_off[ks]);
      sT = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], sT, 0, 0, 0);
    }
#pragma unroll
    for (int ks = 0; ks < CV::KS; ++ks) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(vt + offv.row_off[ks]);
      pT = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, df[ks], pT, 0, 0, 0);
    }
    // dS^T = P^T * (dP^T - Drow) as the B operand of k-steps j = 0, 1
    bf16x8 dsb[2];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p = __builtin_amdgcn_exp2f(fmaf(sT[r], c_log2, -ldv.x));
      dsb[r >> 3][r & 7] = (__bf16)(p * (pT[r] - ldv.y));
    }
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int t = 0; t < C::OT; ++t)
        acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_tr<D>(kt, off, t, j), dsb[j], acc[t], 0, 0, 0);
    wait_vmem<0>();
    __syncthreads();
  }

  // dQ^T of the two key halves summed through LDS, scaled, stored.
  float* stg = reinterpret_cast<float*>(smem);
  if (kh == 1) stage_store<D>(stg, acc, qh, lane, 1.f);
  __syncthreads();
  if (kh == 0) stage_add<D>(stg, acc, qh, lane, scale);
  __syncthreads();
  stage_flush<D>(stg, dq + (rows_off + (int64_t)ci * kBlk) * D, tid);
}

// ---- dK, dV ---------------------------------------------------------------------
// Software pipeline (one wavefront per SIMD, so the overlap has to come from
// within each wave).  Iteration s: phase A forms S and dP of step s on the
// matrix cores, turning S into P (exponentials) while the dP products run;
// phase B runs the dV and dK products of step s - 1 while dS of step s is
// formed.  Tiles live in a four-stage ring: steps s + 1 and s + 2 load while
// steps s and s - 1 are read, and the loads of step s + 2 are issued one
// 1 KiB piece at a time between the MFMAs of phase A.
template <int D>
__global__ __launch_bounds__(kThreads, 1) void sparse_attn_bwd_dkdv_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    const __bf16* __restrict__ dout, const int32_t* __restrict__ coloff, const int32_t* __restrict__ csr,
    int max_kv, const float2* __restrict__ ld, float* __restrict__ dk, float* __restrict__ dv, int Nc,
    int64_t total_cubes, float c_log2, float scale, int group) {
  using C = BCfg<D>;
  constexpr int SLOT = 2 * C::TILE + 1024;   // Q tile, dO tile, (LSE log2 e, Drow) of 64 queries
  constexpr int NST = 4;                     // ring stages
  constexpr int G1 = 2 * C::KS;              // S and dP MFMAs per step
  constexpr int NTR = 4 * C::OT;             // dV and dK MFMAs per step
  constexpr int RPA = 16 / C::KS;            // P entries formed per dP MFMA
  constexpr int RPB = 16 / NTR;              // dS entries formed per dV/dK MFMA
  constexpr int NP = 2 * C::LOADS;           // tile pieces per wave per step
  constexpr int PF = 4;                      // operand reads kept in flight ahead of their MFMA
  static_assert(2 * NP <= G1, "pieces fit in phase A");
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int qh = wave & 1, kh = wave >> 1;
  const int g = lane >> 5;

  // cube = key cube cj of key/value head bh; its list indexes the Nr query
  // cubes of the `group` query heads that share that head (contiguous)
  const int64_t cube = xcd_remap(blockIdx.x, total_cubes);
  const int64_t bh = cube / Nc;
  const int cj = (int)(cube - bh * Nc);
  const int Nr = group * Nc;
  const int64_t head_off = bh * (int64_t)Nc * kBlk * D;        // K, V, dK, dV
  const int64_t qgrp_off = bh * (int64_t)Nr * kBlk * D;        // Q, dO of the group
  const char* q_head = reinterpret_cast<const char*>(q + qgrp_off);
  const char* d_head = reinterpret_cast<const char*>(dout + qgrp_off);
  const char* ld_head = reinterpret_cast<const char*>(ld + bh * (int64_t)Nr * kBlk);
  const int32_t* co = coloff + bh * (int64_t)(Nc + 1);
  const int b0 = co[cj];
  const int n = co[cj + 1] - b0;
  ListWindow lw(csr + bh * (int64_t)Nr * max_kv + b0, n, Nr, lane);

  const LaneOffsets<D> off(wave, lane, qh);
  const uint32_t lds_base = __builtin_amdgcn_readfirstlane(lds_addr(smem));
  const uint32_t lds0 = lds_base + (uint32_t)(wave * C::LOADS * 1024);
  const uint32_t ld_off = 16u * (uint32_t)(lane & 31);   // 512 bytes; lanes 32-63 repeat them
  auto stage = [&](int s) { return smem + (s % NST) * SLOT; };

  // The loads of one step: the Q and dO tiles of its query cube (NP pieces
  // per wave) and, from wave 0, the cube's 64 (LSE log2 e, Drow) records.
  struct StepLoads {
    const char* qb;
    const char* db;
    const char* lb;
    uint32_t so;   // stage offset
    bool on;
  };
  auto prepare = [&](int s) {
    StepLoads x;
    x.on = s < n;
    const int ci = x.on ? lw.at(s, lane) : 0;
    x.qb = uniform_ptr(q_head + (int64_t)ci * C::TILE);
    x.db = uniform_ptr(d_head + (int64_t)ci * C::TILE);
    x.lb = uniform_ptr(ld_head + (int64_t)ci * kBlk * 8);
    x.so = (uint32_t)((s % NST) * SLOT);
    return x;
  };
  auto piece = [&](const StepLoads& x, int i) {   // i < NP: Q pieces, then dO pieces
    const char* base = i < C::LOADS ? x.qb : x.db;
    const uint32_t dst = lds0 + x.so + (i < C::LOADS ? 0u : (uint32_t)C::TILE);
    switch (i % C::LOADS) {
      case 0: dma_one<0>(base, off.g_off[0], dst); break;
      case 1: dma_one<1>(base, off.g_off[1], dst); break;
      case 2: if constexpr (C::LOADS > 2) dma_one<2>(base, off.g_off[C::LOADS > 2 ? 2 : 0], dst); break;
      default: if constexpr (C::LOADS > 3) dma_one<3>(base, off.g_off[C::LOADS > 3 ? 3 : 0], dst); break;
    }
  };
  auto records_piece = [&](const StepLoads& x) {
    if (wave == 0) dma_piece(x.lb, ld_off, lds_base + x.so + 2 * C::TILE);
  };
  auto issue_all = [&](int s) {
    const StepLoads x = prepare(s);
#pragma unroll
    for (int i = 0; i < NP; ++i) piece(x, i);
    records_piece(x);
  };

  bf16x8 kf[C::KS], vf[C::KS];
  load_b_operand<D>(k + head_off + (int64_t)cj * kBlk * D, kh, lane, kf);
  load_b_operand<D>(v + head_off + (int64_t)cj * kBlk * D, kh, lane, vf);
  f32x16 acc_v[C::OT], acc_k[C::OT];
#pragma unroll
  for (int t = 0; t < C::OT; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) { acc_v[t][r] = 0.f; acc_k[t][r] = 0.f; }

  // (LSE log2 e, Drow) of the lane's 16 queries 32*qh + 8*(r/4) + 4*g + r%4.
  auto read_records = [&](const char* st, float4 (&rec)[8]) {
    const float* base = reinterpret_cast<const float*>(st + 2 * C::TILE) + 2 * (32 * qh + 4 * g);
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      rec[2 * rq] = *reinterpret_cast<const float4*>(base + 16 * rq);
      rec[2 * rq + 1] = *reinterpret_cast<const float4*>(base + 16 * rq + 4);
    }
  };
  auto rec_at = [](const float4 (&rec)[8], int r) -> const float4& { return rec[2 * (r >> 2) + ((r >> 1) & 1)]; };
  // Operand i of the dV / dK products of a step: dO^T (i < 2*OT) or Q^T,
  // k-step j, d tile t, read transposed from that step's stage.
  auto read_tr_op = [&](const char* tp, int i) {
    const int which = i / (2 * C::OT), j = (i / C::OT) & 1, t = i % C::OT;
    return read_tr<D>(tp + (which == 0 ? C::TILE : 0), off, t, j);
  };

  // Phase A: S and dP of one step (rows = queries 32*qh + 8*(r/4) + 4*g + r%4,
  // column = key 32*kh + n32); while the dP products run, P = exp2(S c -
  // LSE log2 e) is formed (fp32 in pf, bf16 operand in pbn).  Also issues the
  // pieces of `nx` and, when `prev`, starts the transposed reads of the
  // previous step's first dV / dK operands.
  auto phase_a = [&](const char* tc, const float4 (&rec)[8], f32x16& sS, f32x16& dP, float (&pf)[16],
                     bf16x8 (&pbn)[2], const StepLoads& nx, bool prev, const char* tp, bf16x8 (&tr)[PF]) {
    auto row_op = [&](int i) {
      return *reinterpret_cast<const bf16x8*>(tc + (i < C::KS ? 0 : C::TILE) + off.row_off[i % C::KS]);
    };
    bf16x8 a[PF];
#pragma unroll
    for (int i = 0; i < PF; ++i) a[i] = row_op(i);
#pragma unroll
    for (int r = 0; r < 16; ++r) { sS[r] = 0.f; dP[r] = 0.f; }
#pragma unroll
    for (int i = 0; i < G1; ++i) {
      if (i < C::KS)
        sS = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i % PF], kf[i], sS, 0, 0, 0);
      else
        dP = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i % PF], vf[i - C::KS], dP, 0, 0, 0);
      if (i + PF < G1) a[i % PF] = row_op(i + PF);
      if (nx.on) {
        if ((i & 1) == 0 && i / 2 < NP) piece(nx, i / 2);
        if (i == 1) records_piece(nx);
      }
      if (i >= C::KS) {
#pragma unroll
        for (int u = 0; u < RPA; ++u) {
          const int r = (i - C::KS) * RPA + u;
          const float4& rr = rec_at(rec, r);
          pf[r] = __builtin_amdgcn_exp2f(fmaf(sS[r], c_log2, -((r & 1) ? rr.z : rr.x)));
          pbn[r >> 3][r & 7] = (__bf16)pf[r];
        }
      }
      if (prev && i >= G1 - PF) tr[i - (G1 - PF)] = read_tr_op(tp, i - (G1 - PF));
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // Phase B: dV^T += dO^T P and dK^T += Q^T dS of the previous step (when
  // `prev`; operands 0..PF-1 already in tr) while dS = P (dP - Drow) of this
  // step is formed (when `cur`).
  auto phase_b = [&](bool prev, const char* tp, const bf16x8 (&pbp)[2], const bf16x8 (&dsbp)[2],
                     bf16x8 (&tr)[PF], bool cur, const f32x16& dP, const float (&pf)[16], const float4 (&rec)[8],
                     bf16x8 (&dsbn)[2]) {
#pragma unroll
    for (int i = 0; i < NTR; ++i) {
      if (prev) {
        const int which = i / (2 * C::OT), j = (i / C::OT) & 1, t = i % C::OT;
        if (which == 0)
          acc_v[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr[i % PF], pbp[j], acc_v[t], 0, 0, 0);
        else
          acc_k[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr[i % PF], dsbp[j], acc_k[t], 0, 0, 0);
        if (i + PF < NTR) tr[i % PF] = read_tr_op(tp, i + PF);
      }
      if (cur) {
#pragma unroll
        for (int u = 0; u < RPB; ++u) {
          const int r = i * RPB + u;
          const float4& rr = rec_at(rec, r);
          dsbn[r >> 3][r & 7] = (__bf16)(pf[r] * (dP[r] - ((r & 1) ? rr.w : rr.y)));
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  f32x16 sS, dP;
  float pf[16];
  float4 rec[8];
  bf16x8 pb[2], dsb[2], pbn[2], dsbn[2], tr[PF];
  // Top of step s: wait for this wave's loads of step s (those of step s + 1
  // may stay in flight) and publish them with the barrier, which also frees
  // the stage of step s - 2 for the loads of step s + 2.
  auto top = [&](int s) {
    if (s + 1 < n) {
      if (wave == 0) wait_vmem<NP + 1>(); else wait_vmem<NP>();
    } else {
      wait_vmem<0>();
    }
    __syncthreads();
  };
  if (n > 0) issue_all(0);
  if (n > 1) issue_all(1);
  if (n > 0) {
    // step 0: S, dP, then P and dS
    top(0);
    read_records(stage(0), rec);
    phase_a(stage(0), rec, sS, dP, pf, pb, prepare(2), false, stage(0), tr);
    phase_b(false, stage(0), pb, dsb, tr, true, dP, pf, rec, dsb);
    for (int s = 1; s < n; ++s) {
      top(s);
      const char* tc = stage(s);
      const char* tp = stage(s - 1);
      read_records(tc, rec);
      phase_a(tc, rec, sS, dP, pf, pbn, prepare(s + 2), true, tp, tr);
      phase_b(true, tp, pb, dsb, tr, true, dP, pf, rec, dsbn);
#pragma unroll
      for (int j = 0; j < 2; ++j) { pb[j] = pbn[j]; dsb[j] = dsbn[j]; }
    }
    // the last step's dV and dK products
    const char* tp = stage(n - 1);
#pragma unroll
    for (int i = 0; i < PF; ++i) tr[i] = read_tr_op(tp, i);
    phase_b(true, tp, pb, dsb, tr, false, dP, pf, rec, dsbn);
  }
  __syncthreads();   // every wave is done with the ring

  // dV^T and dK^T of the two query halves summed through LDS, stored.
  float* stg_v = reinterpret_cast<float*>(smem);
  float* stg_k = reinterpret_cast<float*>(smem + C::STAGE);
  if (qh == 1) {
    stage_store<D>(stg_v, acc_v, kh, lane, 1.f);
    stage_store<D>(stg_k, acc_k, kh, lane, 1.f);
  }
  __syncthreads();
  if (qh == 0) {
    stage_add<D>(stg_v, acc_v, kh, lane, 1.f);
    stage_add<D>(stg_k, acc_k, kh, lane, scale);
  }
  __syncthreads();
  stage_flush<D>(stg_v, dv + head_off + (int64_t)cj * kBlk * D, tid);
  stage_flush<D>(stg_k, dk + head_off + (int64_t)cj * kBlk * D, tid);
}

// ---- dK, dV when the value head size differs ------------------------------------
// The plain form of the kernel above, for (D, DV) with D != DV: the same
// products and layouts, K (D) and V (DV) in registers as B operands, one
// step per barrier with the next step's Q and dO tiles and records loading
// into the other of two stages, two workgroups per CU.
template <int D, int DV>
__global__ __launch_bounds__(kThreads, 2) void sparse_attn_bwd_dkdv_dv_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    const __bf16* __restrict__ dout, const int32_t* __restrict__ coloff, const int32_t* __restrict__ csr,
    int max_kv, const float2* __restrict__ ld, float* __restrict__ dk, float* __restrict__ dv, int Nc,
    int64_t total_cubes, float c_log2, float scale, int group) {
  using C = BCfg<D>;
  using CV = BCfg<DV>;
  constexpr int SLOT = C::TILE + CV::TILE + 1024;   // Q tile, dO tile, (LSE log2 e, Drow) of 64 queries
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int qh = wave & 1, kh = wave >> 1;
  const int g = lane >> 5;

  // cube = key cube cj of key/value head bh; its list indexes the Nr query
  // cubes of the `group` query heads that share that head (contiguous)
  const int64_t cube = xcd_remap(blockIdx.x, total_cubes);
  const int64_t bh = cube / Nc;
  const int cj = (int)(cube - bh * Nc);
  const int Nr = group * Nc;
  const int64_t kv_rows = bh * (int64_t)Nc * kBlk;    // K, V, dK, dV rows of this head
  const int64_t q_rows = bh * (int64_t)Nr * kBlk;     // Q, dO rows of the group
  const char* q_head = reinterpret_cast<const char*>(q + q_rows * D);
  const char* d_head = reinterpret_cast<const char*>(dout + q_rows * DV);
  const char* ld_head = reinterpret_cast<const char*>(ld + q_rows);
  const int32_t* co = coloff + bh * (int64_t)(Nc + 1);
  const int b0 = co[cj];
  const int n = co[cj + 1] - b0;
  ListWindow lw(csr + bh * (int64_t)Nr * max_kv + b0, n, Nr, lane);

  const LaneOffsets<D> oq(wave, lane, qh);
  const LaneOffsets<DV> od(wave, lane, qh);
  const uint32_t lds_base = __builtin_amdgcn_readfirstlane(lds_addr(smem));
  const uint32_t lds_q = lds_base + (uint32_t)(wave * C::LOADS * 1024);
  const uint32_t lds_d = lds_base + (uint32_t)(C::TILE + wave * CV::LOADS * 1024);
  const uint32_t ld_off = 16u * (uint32_t)(lane & 31);   // 512 bytes; lanes 32-63 repeat them
  auto issue = [&](int s, int stage) {
    const int ci = lw.at(s, lane);
    dma_tile(uniform_ptr(q_head + (int64_t)ci * C::TILE), oq.g_off, lds_q + stage * SLOT);
    dma_tile(uniform_ptr(d_head + (int64_t)ci * CV::TILE), od.g_off, lds_d + stage * SLOT);
    if (wave == 0)
      dma_piece(uniform_ptr(ld_head + (int64_t)ci * kBlk * 8), ld_off,
                lds_base + stage * SLOT + C::TILE + CV::TILE);
  };
  if (n > 0) issue(0, 0);

  bf16x8 kf[C::KS], vf[CV::KS];
  load_b_operand<D>(k + (kv_rows + (int64_t)cj * kBlk) * D, kh, lane, kf);
  load_b_operand<DV>(v + (kv_rows + (int64_t)cj * kBlk) * DV, kh, lane, vf);
  f32x16 acc_v[CV::OT], acc_k[C::OT];   // dV^T, dK^T: rows = d, column = key 32*kh + n32
#pragma unroll
  for (int t = 0; t < CV::OT; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc_v[t][r] = 0.f;
#pragma unroll
  for (int t = 0; t < C::OT; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc_k[t][r] = 0.f;
  wait_vmem<0>();
  __syncthreads();

  for (int s = 0; s < n; ++s) {
    const int st = s & 1;
    if (s + 1 < n) issue(s + 1, st ^ 1);
    const char* tq = smem + st * SLOT;
    const char* td = tq + C::TILE;
    // S and dP: rows = queries 32*qh + 8*(r/4) + 4*g + r%4, column = key
    f32x16 sS, dP;
#pragma unroll
    for (int r = 0; r < 16; ++r) { sS[r] = 0.f; dP[r] = 0.f; }
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks)
      sS = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8*>(tq + oq.row_off[ks]), kf[ks],
                                                   sS, 0, 0, 0);
#pragma unroll
    for (int ks = 0; ks < CV::KS; ++ks)
      dP = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8*>(td + od.row_off[ks]), vf[ks],
                                                   dP, 0, 0, 0);
    // (LSE log2 e, Drow) of the lane's 16 queries; P and dS as B operands
    // (k-step j holds registers 8j..8j+7)
    const float* rec = reinterpret_cast<const float*>(td + CV::TILE) + 2 * (32 * qh + 4 * g);
    bf16x8 pb[2], dsb[2];
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      const float4 r01 = *reinterpret_cast<const float4*>(rec + 16 * rq);
      const float4 r23 = *reinterpret_cast<const float4*>(rec + 16 * rq + 4);
      const float lse_[4] = {r01.x, r01.z, r23.x, r23.z};
      const float drw[4] = {r01.y, r01.w, r23.y, r23.w};
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int r = 4 * rq + u;
        const float p = __builtin_amdgcn_exp2f(fmaf(sS[r], c_log2, -lse_[u]));
        pb[r >> 3][r & 7] = (__bf16)p;
        dsb[r >> 3][r & 7] = (__bf16)(p * (dP[r] - drw[u]));
      }
    }
    // dV^T += dO^T P and dK^T += Q^T dS, transposing reads of the dO and Q tiles
#pragma unroll
    for (int j = 0; j < 2; ++j) {
#pragma unroll
      for (int t = 0; t < CV::OT; ++t)
        acc_v[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_tr<DV>(td, od, t, j), pb[j], acc_v[t], 0, 0, 0);
#pragma unroll
      for (int t = 0; t < C::OT; ++t)
        acc_k[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_tr<D>(tq, oq, t, j), dsb[j], acc_k[t], 0, 0, 0);
    }
    wait_vmem<0>();
    __syncthreads();
  }

  // the two query halves summed through LDS; dK scaled
  float* stg_v = reinterpret_cast<float*>(smem);
  float* stg_k = reinterpret_cast<float*>(smem + CV::STAGE);
  if (qh == 1) {
    stage_store<DV>(stg_v, acc_v, kh, lane, 1.f);
    stage_store<D>(stg_k, acc_k, kh, lane, 1.f);
  }
  __syncthreads();
  if (qh == 0) {
    stage_add<DV>(stg_v, acc_v, kh, lane, 1.f);
    stage_add<D>(stg_k, acc_k, kh, lane, scale);
  }
  __syncthreads();
  stage_flush<DV>(stg_v, dv + (kv_rows + (int64_t)cj * kBlk) * DV, tid);
  stage_flush<D>(stg_k, dk + (kv_rows + (int64_t)cj * kBlk) * D, tid);
}

constexpr int kLdsMax = 160 * 1024;

template <int D, int DV = D>
constexpr int dq_lds() {
  using C = BCfg<D>;
  constexpr int ring = 2 * (C::TILE + BCfg<DV>::TILE);
  return ring > C::STAGE ? ring : C::STAGE;
}
template <int D, int DV>
constexpr int dkdv_dv_lds() {
  constexpr int ring = 2 * (BCfg<D>::TILE + BCfg<DV>::TILE + 1024);
  constexpr int epi = BCfg<D>::STAGE + BCfg<DV>::STAGE;
  return ring > epi ? ring : epi;
}
template <int D>
constexpr int dkdv_lds() {
  using C = BCfg<D>;
  return 4 * (2 * C::TILE + 1024) > 2 * C::STAGE ? 4 * (2 * C::TILE + 1024) : 2 * C::STAGE;
}

template <typename K>
hipError_t grant_lds(K kern, int bytes, int& granted) {
  static std::mutex mu;   // host threads may launch concurrently
  std::lock_guard<std::mutex> lock(mu);
  if (granted >= bytes) return hipSuccess;
  const hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess) granted = bytes;
  return e;
}

struct WsLayout {
  size_t ld, blkcnt, coloff, csr, total;
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Lists are per key/value head: Nr = group * Nc query rows each.
WsLayout ws_layout(const Geom& g, int max_kv) {
  const size_t Nr = (size_t)g.group * g.Nc;
  const size_t nrb = (Nr + kRowsPerBlk - 1) / kRowsPerBlk;
  WsLayout w;
  w.ld = 0;
  w.blkcnt = w.ld + align256((size_t)g.BH * g.Np * 8);
  w.coloff = w.blkcnt + align256((size_t)g.BHkv * nrb * g.Nc * 4);
  w.csr = w.coloff + align256((size_t)g.BHkv * (g.Nc + 1) * 4);
  w.total = w.csr + align256((size_t)g.BHkv * Nr * max_kv * 4);
  return w;
}

// D: query/key head size, DV: value head size.
template <int D, int DV>
hipError_t launch_d(const Geom& g, const void* q, const void* k, const void* v, const int32_t* lut,
                    const int32_t* valid, int max_kv, const void* o, const float* lse, const void* dout,
                    float* dq, float* dk, float* dv, char* ws, hipStream_t s) {
  static int granted[64][2];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  const WsLayout w = ws_layout(g, max_kv);
  float2* ld = reinterpret_cast<float2*>(ws + w.ld);
  int32_t* blkcnt = reinterpret_cast<int32_t*>(ws + w.blkcnt);
  int32_t* coloff = reinterpret_cast<int32_t*>(ws + w.coloff);
  int32_t* csr = reinterpret_cast<int32_t*>(ws + w.csr);
  const int Nc = (int)g.Nc;
  const int Nr = g.group * Nc;   // query rows per key/value head
  const int nrb = (Nr + kRowsPerBlk - 1) / kRowsPerBlk;
  const int64_t total_tok = g.BH * g.Np;
  const int64_t total_cubes = g.BH * g.Nc;       // query cubes
  const int64_t total_kv_cubes = g.BHkv * g.Nc;  // key cubes

  constexpr int TOK_PER_BLOCK = 256 / (DV / 8);   // O and dO rows are DV wide
  hipLaunchKernelGGL(bwd_prep_kernel<DV>, dim3((unsigned)((total_tok + TOK_PER_BLOCK - 1) / TOK_PER_BLOCK)),
                     dim3(256), 0, s, (const __bf16*)o, (const __bf16*)dout, lse, ld, total_tok);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t cnt_lds = (size_t)Nc * 4;
  hipLaunchKernelGGL(csr_count_kernel, dim3((unsigned)(g.BHkv * nrb)), dim3(256), cnt_lds, s, lut, valid, max_kv,
                     Nr, Nc, nrb, blkcnt);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(csr_scan_kernel, dim3((unsigned)g.BHkv), dim3(256), cnt_lds, s, blkcnt, Nc, nrb, coloff);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(csr_scatter_kernel, dim3((unsigned)(g.BHkv * nrb)), dim3(64), cnt_lds, s, lut, valid, max_kv,
                     Nr, Nc, nrb, blkcnt, coloff, csr);
  if ((e = hipGetLastError()) != hipSuccess) return e;

  const float c_log2 = kLog2e / sqrtf((float)D);
  const float scale = 1.0f / sqrtf((float)D);
  auto kq = sparse_attn_bwd_dq_kernel<D, DV>;
  // equal head sizes: the pipelined dK/dV kernel; otherwise its plain form
  auto kkv = [] {
    if constexpr (D == DV) return sparse_attn_bwd_dkdv_kernel<D>;
    else return sparse_attn_bwd_dkdv_dv_kernel<D, DV>;
  }();
  constexpr int kv_lds = D == DV ? dkdv_lds<D>() : dkdv_dv_lds<D, DV>();
  constexpr int q_lds = dq_lds<D, DV>();
  if ((e = grant_lds(kq, q_lds, granted[dev][0])) != hipSuccess) return e;
  if ((e = grant_lds(kkv, kv_lds, granted[dev][1])) != hipSuccess) return e;
  hipLaunchKernelGGL(kq, dim3((unsigned)total_cubes), dim3(kThreads), q_lds, s, (const __bf16*)q,
                     (const __bf16*)k, (const __bf16*)v, (const __bf16*)dout, lut, valid, max_kv,
                     (const float2*)ld, dq, Nc, total_cubes, c_log2, scale, g.group);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(kkv, dim3((unsigned)total_kv_cubes), dim3(kThreads), kv_lds, s, (const __bf16*)q,
                     (const __bf16*)k, (const __bf16*)v, (const __bf16*)dout, (const int32_t*)coloff,
                     (const int32_t*)csr, max_kv, (const float2*)ld, dk, dv, Nc, total_kv_cubes, c_log2, scale,
                     g.group);
  return hipGetLastError();
}

static_assert(dq_lds<128>() <= kLdsMax && dkdv_lds<128>() <= kLdsMax, "LDS budget");

}  // namespace

size_t sparse_attn_bwd_workspace(const Geom& g, int max_kv) { return ws_layout(g, max_kv).total; }

bool sparse_attn_bwd_fits(const Geom& g, int max_kv) {
  // LDS counters of the transposed-list build hold one int per key cube;
  // every launch grid stays below 2^31 workgroups, and a key/value head's
  // list offsets (group * Nc * max_kv entries) fit in int32.
  return g.Nc >= 1 && g.Nc <= kMaxBwdCubes && g.BH * g.Nc < ((int64_t)1 << 31) &&
         (int64_t)g.group * g.Nc * max_kv < ((int64_t)1 << 31);
}

hipError_t launch_sparse_attn_bwd(const Geom& g, const void* q, const void* k, const void* v, const int32_t* lut,
                                  const int32_t* valid, int max_kv, const void* o, const float* lse,
                                  const void* dout, float* dq, float* dk, float* dv, void* workspace,
                                  hipStream_t s) {
  char* ws = static_cast<char*>(workspace);
  if (g.D == 128 && g.Dv == 128)
    return launch_d<128, 128>(g, q, k, v, lut, valid, max_kv, o, lse, dout, dq, dk, dv, ws, s);
  if (g.D == 64 && g.Dv == 64)
    return launch_d<64, 64>(g, q, k, v, lut, valid, max_kv, o, lse, dout, dq, dk, dv, ws, s);
  if (g.D == 128 && g.Dv == 64)
    return launch_d<128, 64>(g, q, k, v, lut, valid, max_kv, o, lse, dout, dq, dk, dv, ws, s);
  if (g.D == 64 && g.Dv == 128)
    return launch_d<64, 128>(g, q, k, v, lut, valid, max_kv, o, lse, dout, dq, dk, dv, ws, s);
  return hipErrorInvalidValue;
}

}  // namespace vsa
