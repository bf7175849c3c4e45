// Fine block-sparse attention with the gated combination, for gfx950.
//
// "VSA: Accelerating Video Diffusion Inference with Sparse Attention on AMD
// GPUs": §Two-Stage Architecture (Stage 2 computes token-level attention only
// over the key/value cubes the coarse stage selected; the output combines the
// coarse and fine outputs through gates), §Block-Sparse Encoding (index list
// plus valid count per query block), §Kernel Architecture (QK^T product,
// online softmax with running max M and sum L, PV product, double buffering)
// and §Sparse Traversal (loop over the valid count, jumping to the listed
// key/value block).  "VSA: Faster Video Diffusion with Trainable Sparse
// Attention", Abstract.  Softmax(QK^T / sqrt(d)) V as in §The Attention
// Bottleneck in Video Diffusion.
//
// Work decomposition:
//   * One workgroup (512 threads, 8 wavefronts) per CU, persistent.  Each
//     workgroup takes a PAIR of neighbouring query cubes (2p, 2p+1) of one
//     (batch, head): waves 0-3 serve cube A, waves 4-7 cube B.  Each XCD owns
//     one contiguous range of pairs and its workgroups walk it in rounds, so
//     neighbouring pairs sweep similar key cubes at the same time (L2 reuse).
//   * Step schedule.  Neighbouring query cubes select largely the same key
//     cubes.  The two LUT rows are turned into one list of steps: first every
//     key cube both rows list (loaded once, used by both halves), then the
//     remaining cubes of A paired with the remaining cubes of B (two tiles
//     per step).  Every step keeps all 8 waves busy whenever the rows have
//     equal counts, and K/V tiles are fetched once per pair instead of once
//     per cube for the shared part.  Attention sums over its key set, so the
//     visiting order only changes fp32 rounding.  Rows that list a cube twice
//     (allowed: each listing is attended) fall back to positional pairing.
//   * Within a half, wave w owns query half qh = w & 1 (32 of the cube's 64
//     query tokens) and key half kh = (w >> 1) & 1 (32 of the 64 tokens of
//     each key cube); the two key halves keep separate online-softmax states,
//     merged once per query cube.
//   * Scores are formed transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x16_bf16: K rows from LDS as the A operand, Q in
//     registers as the B operand.  In the accumulator layout each lane owns
//     one query (lane % 32) and 16 of its keys, so the row max is a local max
//     plus one v_permlane32_swap and all softmax state is lane-local.
//   * O^T += V^T P^T: P (bf16) is already in B-operand layout; V^T is read
//     from the V tile in its natural [key][d] order with ds_read_b64_tr_b16.
//   * Software pipeline, one barrier per step: each wave overlaps the QK
//     MFMAs of step p with the exponentials of step p - 1, and the PV MFMAs
//     of step p - 1 with the row max of step p.  The step loop is unrolled by
//     two so the two score tiles swap roles without register copies, and the
//     step schedule is read with one readlane from a 64-entry register
//     window that slides every 32 steps.
//   * Tiles arrive by direct global->LDS loads (16 bytes per lane, no
//     registers).  K and V have separate rings (4 + 4 tiles at d = 128;
//     10 + 8 at d = 64 when the schedule fits beside them, else 8 + 8)
//     because V is consumed one step after K.  A half with no tile in a step
//     reads a tile of zeros kept at the top of LDS instead of branching
//     around its operand reads.  Ring positions and, for
//     every step, the last load group the rings can take are computed once
//     per pair; the four waves of half A issue all loads right after the step
//     barrier, as far ahead as the rings allow, and wait for them with a
//     short chain of vmcnt waits.  Tiles are unpadded; 16-byte chunks are XOR
//     swizzled per row so every LDS read pattern is bank-conflict free.
//   * Rescaling of O is lazy: the exponent offset only moves when a block's
//     max exceeds it by more than 8 (log2 units), keeping every exp2 <= 256;
//     exact, because numerator and denominator share the offset.
//   * Epilogue per query cube: key halves merged through LDS, O normalised,
//     staged in LDS, combined with the gates and the broadcast coarse output
//     and written with coalesced 16-byte stores.
//   * What bounds it: on the 32K-token workload neither the tile bytes nor
//     the MFMAs alone.  Cutting the bytes a workgroup fetches by a quarter
//     gains about 5%; the per-step barrier and the scalar bookkeeping of the
//     schedule (slot, offset and wait arithmetic) cost more, because every
//     wave issues them between its MFMAs.
#include <mutex>
#include <type_traits>

#include "mfma_util.h"
#include "token_map.h"
#include "vsa_internal.h"

namespace vsa {
namespace {

constexpr int kBlk = 64;          // tokens per cube: query tile and key tile
constexpr int kThreads = 512;     // two query cubes x 4 wavefronts
constexpr int kIssueThreads = 256;   // the four wavefronts of half A issue every tile load
constexpr float kTau = 8.0f;      // lazy-rescale threshold (log2 units)
constexpr float kNegBig = -1.0e30f;   // initial exponent offset
constexpr int kLdsMax = 160 * 1024;   // LDS of one CU

template <int D>
struct Cfg {
  static constexpr int ROWB = D * 2;                 // bytes per token row
  static constexpr int CPR = D / 8;                  // 16-byte chunks per row
  static constexpr int TILE = kBlk * ROWB;           // one K or V cube tile
  static constexpr int LOADS = TILE / (kIssueThreads * 16);  // 16-byte loads per issuing wave per tile
  static constexpr int OT = D / 32;                  // 32-row tiles of O^T
  static constexpr int NOV = OT * 16;                // O^T accumulators per lane
  static constexpr int MERGE_G = 2 * (NOV + 4) * 64 * 4;   // merge buffer of one half
  static constexpr int OSTR = D + 4;                 // fp32 staging row stride
  static constexpr int OST_G = kBlk * OSTR * 4;      // staging of one half
  static constexpr int EPI_BYTES = 2 * (MERGE_G + OST_G);
  // Chunk swizzles: the logical 16-byte chunk c of row r sits at c ^ f(r).
  __device__ static constexpr int kswz(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
  __device__ static constexpr int vswz(int r) { return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); }
};

__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ uint32_t pack_step(int ta, int tb) {
  return (uint32_t)(ta < 0 ? 0xffff : ta) | ((uint32_t)(tb < 0 ? 0xffff : tb) << 16);
}


// Wait until at most `parts` K or V tiles' worth of this wave's loads (L load
// instructions per tile) are still pending.  The waits run from the loosest
// to the tightest and stop at `parts`: a wait that is already satisfied costs
// almost nothing, and the chain has no taken branch before its exit.  Counts
// beyond MAXP (or the field width) wait for fewer pending loads, which is
// merely conservative.
template <int N>
__device__ __forceinline__ void wait_vmem_capped() {
  wait_vmem<(N < 63 ? N : 63)>();
}

template <int L, int K>
__device__ __forceinline__ void wait_chain(int parts) {
  wait_vmem_capped<K * L>();
  if constexpr (K > 0) {
    if (parts < K) wait_chain<L, K - 1>(parts);
  }
}

template <int L, int MAXP>
__device__ __forceinline__ void wait_parts(int parts) {
  wait_chain<L, MAXP>(parts);
}

// RK / RV: positions of the K and V tile rings.
// PAD: the grid was padded up to whole cubes (the key masking of partial
// tiles is compiled only into this variant, so the divisible case keeps its
// loop as it is).
// ZT: the last TILE bytes of the CU's LDS hold a tile of zeros (beyond the
// ring, the schedule and the epilogue's buffers), read as the operands of a
// half that has no tile in a step.  The operands are then the same zeros as
// in the variant without it, which branches around its operand reads.
template <int D, int RK, int RV, bool PAD, bool ZT>
__global__ __launch_bounds__(kThreads, 1) void sparse_attn_fwd_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    const int32_t* __restrict__ lut, const int32_t* __restrict__ valid, int max_kv,
    const float* __restrict__ oc, const __bf16* __restrict__ gate_c, const __bf16* __restrict__ gate_f,
    __bf16* __restrict__ out, float* __restrict__ lse, int Nc, int64_t total_pairs, float c_log2,
    TokenMap tmap, int group, int gather_arg) {
  using C = Cfg<D>;
  // q, k, v in raster order, cube tiles gathered by the loads (only the
  // divisible d = 128 variants are ever launched that way)
  const bool gather = !PAD && D == 128 && gather_arg != 0;
  // The load plan issues group p (K tiles of step p, V tiles of step p - 1)
  // by barrier p - 1, while the tiles of the two steps before it are still
  // held; a step has up to two tiles, so each ring needs four positions
  // (with three, two consecutive two-tile steps leave no room for group p).
  static_assert(RK >= 4 && RV >= 4, "each ring holds two steps of up to two tiles");
  constexpr int V_BASE = RK * C::TILE;           // V ring after the K ring
  constexpr int RING = (RK + RV) * C::TILE;
  constexpr int ZERO_OFF = kLdsMax - C::TILE;    // the zero tile (ZT)
  static_assert(!ZT || (C::EPI_BYTES <= ZERO_OFF && RING < ZERO_OFF), "zero tile clear of the ring and epilogue");
  extern __shared__ __attribute__((aligned(16))) char smem[];
  // schedule after the ring: sched[s] packs the key cube of half A (low 16
  // bits) and of half B (high 16 bits) of step s; 0xffff = none.
  uint32_t* sched = reinterpret_cast<uint32_t*>(smem + RING);
  // plan[s] = kpos(s) | F(s) << 16, s = 0..S+1 (see the load plan below)
  uint32_t* plan = sched + max_kv;
  // dsc[p] = what step p needs (slots, presence, wait and issue counts) and
  // tlist = every tile load of the pair in issue order (see below)
  uint32_t* dsc = plan + max_kv + 2;
  uint32_t* tlist = dsc + max_kv + 1;
  int* flags = reinterpret_cast<int*>(tlist + 4 * max_kv);   // [0] duplicate, [1] unsorted, [2] shared count
  uint32_t* bmA = reinterpret_cast<uint32_t*>(flags + 4);               // Nc-bit membership maps
  const int nwords = (Nc + 31) >> 5;
  uint32_t* bmB = bmA + nwords;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;                  // 0: cube A, 1: cube B
  const int w4 = wave & 3;
  const int qh = w4 & 1, kh = w4 >> 1;
  const int n32 = lane & 31, g = lane >> 5;
  const int l16 = lane & 15, h16 = (lane >> 4) & 1;

  // ---- per-lane constant offsets ------------------------------------------
  // Direct loads (issued by half A only): lane i of load n of wave w fills
  // LDS chunk L = (w*LOADS+n)*64+i of a tile, which holds logical chunk
  // (L % CPR) ^ f(row) of row L / CPR.  Load n of wave w is one 1 KiB piece
  // P = w*LOADS + n of the tile: its rows 1024/ROWB * P onward.  In
  // cube-major order the piece starts P * 1024 bytes after the tile's first
  // row; with gather set the tensors are in raster order and a piece, one
  // run of cw = 1024/ROWB tokens along w, starts (lt*H + lh)*W rows after
  // the cube's first token (lt, lh: the piece's frame and row in the cube).
  // The load's instruction offset adds n * 1024 to both the source and the
  // LDS destination, so source offsets are taken relative to it.
  auto piece_off = [&](int P) -> int64_t {
    if (!gather) return (int64_t)P * 1024;
    const int lt = P / tmap.ch, lh = P - lt * tmap.ch;
    return ((int64_t)lt * tmap.H * tmap.W + (int64_t)lh * tmap.W) * C::ROWB;
  };
  // K: the swizzle depends on the row mod 16, so each load has its own
  // lane offset (and absorbs its piece's offset).  V: the swizzle depends on
  // the row mod 4 only and a piece spans whole groups of 4 rows (4 rows at
  // d = 128, 8 at d = 64), so one lane offset serves every piece and the
  // piece offsets vpd[n] are wave-uniform.
  uint32_t kg_off[C::LOADS];
  int64_t vpd[C::LOADS];
#pragma unroll
  for (int n = 0; n < C::LOADS; ++n) {
    const int P = (wave & 3) * C::LOADS + n;
    const int L = P * 64 + lane;
    const int r = L / C::CPR, x = L % C::CPR;
    kg_off[n] = (uint32_t)(piece_off(P) + (r - P * (1024 / C::ROWB)) * C::ROWB + ((x ^ C::kswz(r)) * 16) - n * 1024);
    vpd[n] = piece_off(P) - n * 1024;
  }
  uint32_t vg;
  {
    const int r = lane / C::CPR, x = lane % C::CPR;   // row within the piece (a multiple of 4 rows in)
    vg = (uint32_t)(r * C::ROWB + ((x ^ C::vswz(r)) * 16));
  }
  // first token row of cube c in the token tensors (tile rows follow it at
  // the piece offsets above)
  auto cube_row = [&](int c) -> uint32_t {
    if (!gather) return (uint32_t)c * kBlk;
    const CubeAt a = cube_at(tmap, c);
    if (!a.ok) return 0u;   // a table entry outside the grid: stay inside the tensors (no output is written for it)
    return (uint32_t)(((a.t * tmap.ct) * tmap.H + a.h * tmap.ch) * tmap.W + a.w * tmap.cw);
  };
  const uint32_t lds_ring = __builtin_amdgcn_readfirstlane(lds_addr(smem) + (uint32_t)((wave & 3) * C::LOADS * 1024));
  // K A-operand reads: key row 32*kh + n32, logical chunk 2*ks + g.
  int k_off[D / 16];
  {
    const int r = 32 * kh + n32;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) k_off[ks] = r * C::ROWB + (((2 * ks + g) ^ C::kswz(r)) * 16);
  }
  // V^T A-operand transposing reads: source lane l16 addresses key row
  // 32*kh + 16*j + 8*hi + 4*g + l16/4 and d columns 32*t + 16*h16 + 4*(l16%4).
  // The swizzle depends on the row only through bits that the +16*j + 8*hi
  // row steps (added as immediates) do not change.
  int v_off[C::OT];
  {
    const int r = 32 * kh + 4 * g + (l16 >> 2);
    const int byte_base = 32 * h16 + 8 * (l16 & 3);
#pragma unroll
    for (int t = 0; t < C::OT; ++t) {
      const int b = 64 * t + byte_base;
      v_off[t] = V_BASE + r * C::ROWB + ((((b >> 4) ^ C::vswz(r)) << 4) | (b & 15));
    }
  }

  if constexpr (ZT) {
    // written once; nothing else writes there (the first pair's schedule
    // build passes several barriers before the first operand read)
    for (int i = tid; i < C::TILE / 16; i += kThreads)
      *reinterpret_cast<uint4*>(smem + ZERO_OFF + 16 * i) = make_uint4(0u, 0u, 0u, 0u);
  }
  const int pairs_per_head = (Nc + 1) >> 1;
  const int64_t per_xcd = (total_pairs + 7) / 8;
  const int xcd = blockIdx.x % 8;
  const int64_t lo = (int64_t)xcd * per_xcd;
  const int64_t end = lo + per_xcd < total_pairs ? lo + per_xcd : total_pairs;
  const int64_t stride = gridDim.x / 8;

  for (int64_t pid = lo + blockIdx.x / 8; pid < end; pid += stride) {
    const int64_t bh = pid / pairs_per_head;
    const int cubeA = (int)(pid - bh * pairs_per_head) * 2;
    const bool hasB = cubeA + 1 < Nc;
    const int64_t rowA = bh * Nc + cubeA;
    const int64_t head_off = bh * (int64_t)Nc * kBlk * D;   // element offset of this (b, h)
    const int64_t kv_off = (bh / group) * (int64_t)Nc * kBlk * D;   // its key/value head
    const char* k_head = reinterpret_cast<const char*>(k + kv_off);
    const char* v_head = reinterpret_cast<const char*>(v + kv_off);

    // Q of this half's cube as the B operand: query 32*qh + n32, d = 16*s + 8*g
    // + 0..7.  Issued before the schedule is built, so that its latency
    // overlaps that of the index rows and the build itself.
    const int my_cube = cubeA + grp;
    const bool my_valid = grp == 0 || hasB;
    bf16x8 qf[D / 16];
    if (my_valid) {
      const int rq = 32 * qh + n32;   // token rq of the cube
      int64_t qr = (int64_t)my_cube * kBlk + rq;
      if (gather) {
        const int lt = small_div(rq, tmap.mag_plane), rem = rq - lt * (tmap.ch * tmap.cw);
        const int lh = small_div(rem, tmap.mag_cw), lw = rem - lh * tmap.cw;
        qr = (int64_t)cube_row(my_cube) + ((int64_t)lt * tmap.H + lh) * tmap.W + lw;
      }
      const __bf16* qrow = q + head_off + qr * D + 8 * g;
#pragma unroll
      for (int s = 0; s < D / 16; ++s) qf[s] = *reinterpret_cast<const bf16x8*>(qrow + 16 * s);
    }
    auto count_of = [&](int64_t row) {
      const int n = valid[row];
      return n < 0 ? 0 : (n > max_kv ? max_kv : n);
    };
    const int nA = count_of(rowA);
    const int nB = hasB ? count_of(rowA + 1) : 0;
    const int32_t* lrowA = lut + rowA * (int64_t)max_kv;
    const int32_t* lrowB = lrowA + max_kv;
    auto clampc = [&](int b) { return b < 0 ? 0 : (b >= Nc ? Nc - 1 : b); };   // memory-safety clamp
    const int S = nA > nB ? nA : nB;   // steps

    // ---- build the step schedule -------------------------------------------
    // Scratch for the build lives in the ring, which is idle until the first
    // tile load below: SH = cubes both rows list, EXA / EXB = cubes only one
    // row lists, PK = the sort key of each exclusive pair.
    int* SH = reinterpret_cast<int*>(smem);
    int* EXA = SH + max_kv;
    int* EXB = EXA + max_kv;
    int* PK = EXB + max_kv;
    for (int i = tid; i < 2 * nwords; i += kThreads) bmA[i] = 0u;
    if (tid < 4) flags[tid] = 0;
    __syncthreads();
    for (int i = tid; i < nA + nB; i += kThreads) {
      const bool inA = i < nA;
      const int c = clampc(inA ? lrowA[i] : lrowB[i - nA]);
      uint32_t* bm = inA ? bmA : bmB;
      const uint32_t bit = 1u << (c & 31);
      if (atomicOr(&bm[c >> 5], bit) & bit) flags[0] = 1;   // a row lists a cube twice
      const int nrow = inA ? nA : nB;
      const int idx = inA ? i : i - nA;
      if (idx + 1 < nrow && clampc(inA ? lrowA[i + 1] : lrowB[idx + 1]) <= c) flags[1] = 1;   // not ascending
    }
    __syncthreads();
    const bool dup = flags[0] != 0;
    const bool sorted = flags[1] == 0;
    if (dup) {
      // positional pairing: step s = (A[s], B[s])
      for (int s = tid; s < S; s += kThreads)
        sched[s] = pack_step(s < nA ? clampc(lrowA[s]) : -1, s < nB ? clampc(lrowB[s]) : -1);
    } else {
      // wave 0 splits row A into shared / A-only cubes, wave 1 row B into
      // B-only cubes (row order kept; ranks from wavefront ballots).
      if (wave < 2) {
        const int n_me = wave == 0 ? nA : nB;
        const int32_t* row = wave == 0 ? lrowA : lrowB;
        const uint32_t* other = wave == 0 ? bmB : bmA;
        int* ex = wave == 0 ? EXA : EXB;
        const uint64_t lt = lane == 0 ? 0ull : (~0ull >> (64 - lane));
        int sh_seen = 0, ex_seen = 0;
        for (int base = 0; base < n_me; base += 64) {
          const int i = base + lane;
          const bool in = i < n_me;
          int c = 0;
          bool sh = false;
          if (in) {
            c = clampc(row[i]);
            sh = (other[c >> 5] >> (c & 31)) & 1u;
          }
          const uint64_t msh = __ballot(in && sh), mex = __ballot(in && !sh);
          if (in) {
            if (!sh) ex[ex_seen + __popcll(mex & lt)] = c;
            else if (wave == 0) SH[sh_seen + __popcll(msh & lt)] = c;
          }
          sh_seen += __popcll(msh);
          ex_seen += __popcll(mex);
        }
        if (lane == 0 && wave == 0) flags[2] = sh_seen;
      }
      __syncthreads();
      const int nS = flags[2];
      const int nExA = nA - nS, nExB = nB - nS;
      const int nP = nExA > nExB ? nExA : nExB;   // exclusive steps; nS + nP == S
      for (int i = tid; i < nP; i += kThreads) {
        const int ka = i < nExA ? EXA[i] : 0x7fffffff;
        const int kb = i < nExB ? EXB[i] : 0x7fffffff;
        PK[i] = ka < kb ? ka : kb;
      }
      __syncthreads();
      if (sorted) {
        // Merge the shared cubes and the exclusive pairs into one ascending
        // order of key cube index, so that the workgroups of an XCD sweep the
        // key cubes together.  Both lists are ascending and never share a
        // value, so rank-by-binary-search gives a bijection onto [0, S).
        auto count_below = [](const int* a, int n, int x) {   // #{a[j] < x}, a ascending
          int lo = 0, hi = n;
          while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (a[mid] < x) lo = mid + 1; else hi = mid;
          }
          return lo;
        };
        for (int g2 = tid; g2 < nS; g2 += kThreads) {
          const int pos = g2 + count_below(PK, nP, SH[g2]);
          sched[pos] = pack_step(SH[g2], SH[g2]);
        }
        for (int i = tid; i < nP; i += kThreads) {
          const int pos = i + count_below(SH, nS, PK[i]);
          sched[pos] = pack_step(i < nExA ? EXA[i] : -1, i < nExB ? EXB[i] : -1);
        }
      } else {
        // any order is exact: shared cubes first, then the exclusive pairs
        for (int g2 = tid; g2 < nS; g2 += kThreads) sched[g2] = pack_step(SH[g2], SH[g2]);
        for (int i = tid; i < nP; i += kThreads)
          sched[nS + i] = pack_step(i < nExA ? EXA[i] : -1, i < nExB ? EXB[i] : -1);
      }
    }

    wait_vmem<0>();    // Q has landed (issued at the top of the pair)
    __syncthreads();   // schedule complete; bitmaps no longer needed

    // ---- load plan ----------------------------------------------------------
    // Ring positions are assigned to tiles in step order: step s owns
    // positions kpos(s) .. kpos(s + 1) - 1, its A tile (if any) first, then
    // its B tile if that differs.  kpos(s) = tiles of steps < s, for
    // s = 0..S + 1 (kpos(S + 1) = kpos(S)).
    if (wave == 0) {
      const uint64_t lt = lane == 0 ? 0ull : (~0ull >> (64 - lane));
      int carry = 0;
      for (int base = 0; base <= S; base += 64) {
        const int st = base + lane;
        int n = 0;
        if (st < S) {
          const uint32_t e = sched[st];
          const uint32_t a = e & 0xffffu, b = e >> 16;
          n = (a != 0xffffu ? 1 : 0) + ((b != 0xffffu && b != a) ? 1 : 0);
        }
        const uint64_t b1 = __ballot(n >= 1), b2 = __ballot(n == 2);
        if (st <= S) plan[st] = (uint32_t)(carry + __popcll(b1 & lt) + __popcll(b2 & lt));
        carry += __popcll(b1) + __popcll(b2);
      }
      if (lane == 0) plan[S + 1] = (uint32_t)carry;
    }
    __syncthreads();
    // Load group g = the K tiles of step g and the V tiles of step g - 1 (V
    // is consumed one step after K).  At step barrier p the K positions of
    // steps < p and the V positions of steps < p - 1 are free, so group g
    // may be in flight once kpos(g + 1) <= kpos(p) + RK and
    // kpos(g) <= kpos(p - 1) + RV.  F(p) = the last such group (<= S);
    // F(p - 1) >= p, so group p is always in flight by barrier p.
    {
      int* fscr = reinterpret_cast<int*>(smem);   // the ring is idle until the first load
      for (int pp = tid; pp <= S; pp += kThreads) {
        const int kcap = (int)plan[pp] + RK;
        const int vcap = (pp > 0 ? (int)plan[pp - 1] : 0) + RV;
        int glo = 0, ghi = S;   // group 0 always fits
        while (glo < ghi) {
          const int mid = (glo + ghi + 1) >> 1;
          if ((int)plan[mid + 1] <= kcap && (int)plan[mid] <= vcap) glo = mid; else ghi = mid - 1;
        }
        fscr[pp] = glo;
      }
      __syncthreads();
      for (int pp = tid; pp <= S; pp += kThreads) plan[pp] |= (uint32_t)fscr[pp] << 16;
      __syncthreads();
    }

    // ---- per-step descriptors and the tile list --------------------------
    // Loads are issued group by group (group g = the K tiles of step g, then
    // the V tiles of step g - 1), so the tiles of group g occupy list entries
    // kpos(g) + kpos(g - 1) onward.  tlist[i] = ring slot | (1 if V) << 4 |
    // the cube's first token row (cube_row) << 5.  Before the loop groups 0..F(0) are issued; after
    // barrier p, groups F(p - 1) + 1 .. F(p).  issued(p) = the list length
    // issued before barrier p; at barrier p the wave waits until only the
    // tiles after group p, issued(p) - kpos(p + 1) - kpos(p), remain in
    // flight.  dsc[p]:
    //   bits 0-3 / 4-7    K ring slot of half A's / half B's tile of step p
    //   bits 8-11 / 12-15 V ring slot of half A's / half B's tile of step p-1
    //   bits 16 / 17      half A / half B has a tile in step p
    //   bits 18 / 19      half A / half B had a tile in step p - 1
    //   bits 20-24        tiles to leave in flight at barrier p
    //   bits 25-29        tiles to issue after barrier p
    //   bits 30 / 31      half A's / half B's tile of step p holds padded positions
    {
      auto kpos = [&](int st) { return st < 0 ? 0 : (int)(plan[st] & 0xffffu); };
      auto fr = [&](int st) { return (int)(plan[st] >> 16); };
      auto issued_through = [&](int grpi) { return kpos(grpi + 1) + kpos(grpi); };
      for (int pp = tid; pp <= S; pp += kThreads) {
        uint32_t d = 0;
        if (pp < S) {
          const uint32_t e = sched[pp];
          const uint32_t a = e & 0xffffu, b = e >> 16;
          const int k0 = kpos(pp);
          const int kb = k0 + ((a != 0xffffu && b != a) ? 1 : 0);
          d |= (uint32_t)(k0 % RK) | ((uint32_t)(kb % RK) << 4);
          d |= (a != 0xffffu ? 1u << 16 : 0u) | (b != 0xffffu ? 1u << 17 : 0u);
          if constexpr (PAD) {
            if (a != 0xffffu && cube_partial(tmap, cube_at(tmap, (int)a))) d |= 1u << 30;
            if (b != 0xffffu && cube_partial(tmap, cube_at(tmap, (int)b))) d |= 1u << 31;
          }
        }
        if (pp > 0) {
          const uint32_t e = sched[pp - 1];
          const uint32_t a = e & 0xffffu, b = e >> 16;
          const int v0 = kpos(pp - 1);
          const int vb = v0 + ((a != 0xffffu && b != a) ? 1 : 0);
          d |= ((uint32_t)(v0 % RV) << 8) | ((uint32_t)(vb % RV) << 12);
          d |= (a != 0xffffu ? 1u << 18 : 0u) | (b != 0xffffu ? 1u << 19 : 0u);
        }
        const int before = issued_through(fr(pp > 0 ? pp - 1 : 0));   // issued before barrier pp
        const int after = issued_through(fr(pp));                     // ... after it
        d |= (uint32_t)(before - issued_through(pp)) << 20;
        d |= (uint32_t)(after - before) << 25;
        dsc[pp] = d;
      }
      for (int gg = tid; gg <= S; gg += kThreads) {
        int i = kpos(gg) + kpos(gg - 1);
        if (gg < S) {
          const uint32_t e = sched[gg];
          const uint32_t a = e & 0xffffu, b = e >> 16;
          const int k0 = kpos(gg), nk = kpos(gg + 1) - k0;
          if (nk >= 1) tlist[i++] = (cube_row((int)(a != 0xffffu ? a : b)) << 5) | (uint32_t)(k0 % RK);
          if (nk == 2) tlist[i++] = (cube_row((int)b) << 5) | (uint32_t)((k0 + 1) % RK);
        }
        if (gg > 0) {
          const uint32_t e = sched[gg - 1];
          const uint32_t a = e & 0xffffu, b = e >> 16;
          const int v0 = kpos(gg - 1), nv = kpos(gg) - v0;
          if (nv >= 1) tlist[i++] = (cube_row((int)(a != 0xffffu ? a : b)) << 5) | (uint32_t)(v0 % RV) | 16u;
          if (nv == 2) tlist[i++] = (cube_row((int)b) << 5) | (uint32_t)((v0 + 1) % RV) | 16u;
        }
      }
      __syncthreads();
    }
    const int n_init = (int)(plan[(int)(plan[0] >> 16) + 1] & 0xffffu) + (int)(plan[(int)(plan[0] >> 16)] & 0xffffu);

    // Descriptors and list entries are read from registers: lane j of dw
    // holds dsc[dwin + j], lane j of tw holds tlist[twin + j].  Each window
    // slides by 32 entries when its reads would leave the first half (a step
    // issues at most RK + RV < 32 tiles), and the next window is read from
    // LDS one slide ahead.
    int dwin = 0, twin = 0;
    uint32_t dw = lane <= S ? dsc[lane] : 0u;
    uint32_t ndw = 32 + lane <= S ? dsc[32 + lane] : 0u;
    const int n_list = 2 * (int)(plan[S] & 0xffffu);
    uint32_t tw = lane < n_list ? tlist[lane] : 0u;
    uint32_t ntw = 32 + lane < n_list ? tlist[32 + lane] : 0u;
    int i_tile = 0;   // next list entry to issue (half A)
    auto issue = [&](int count) {
      if (i_tile - twin >= 32) {
        twin += 32;
        tw = ntw;
        ntw = twin + 32 + lane < n_list ? tlist[twin + 32 + lane] : 0u;
      }
      for (int c = 0; c < count; ++c, ++i_tile) {
        const uint32_t e = (uint32_t)__builtin_amdgcn_readlane((int)tw, i_tile - twin);
        const uint32_t row = e >> 5, slot = e & 15u;
        if (e & 16u) {
          dma_pieces(uniform_ptr(v_head + (int64_t)row * C::ROWB), vpd, vg, lds_ring + V_BASE + slot * C::TILE);
        } else {
          dma_tile(uniform_ptr(k_head + (int64_t)row * C::ROWB), kg_off, lds_ring + slot * C::TILE);
        }
      }
    };
    if (grp == 0) issue(n_init);

    f32x16 o[C::OT];
#pragma unroll
    for (int t = 0; t < C::OT; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[t][r] = 0.f;
    // Exponent offset (log2 units).  It starts at a large finite negative
    // value rather than -inf so that offset arithmetic never forms inf - inf;
    // the first real block always moves it (exp2 of the difference is 0).
    float m_used = kNegBig;
    float l_part = 0.f;        // this lane's partial row sum
    f32x16 sc;                 // scores of the previous step: keys 32*kh + 8*(r/4) + 4*g + r%4, query n32
#pragma unroll
    for (int r = 0; r < 16; ++r) sc[r] = 0.f;
    float mx_prev = kNegBig;   // their row max (log2 units)

    // Step barrier p: every wave has finished iteration p - 1.  Half A waits
    // for its loads of group p (K of step p, V of step p - 1), the barrier
    // publishes them, and half A issues the groups that became free.
    uint32_t d_c = 0;   // dsc of the current step
    auto step_barrier = [&](int p) {
      if (p - dwin == 32) {   // slide the descriptor window by 32 entries
        dwin += 32;
        dw = ndw;
        ndw = dwin + 32 + lane <= S ? dsc[dwin + 32 + lane] : 0u;
      }
      d_c = (uint32_t)__builtin_amdgcn_readlane((int)dw, p - dwin);
      if (grp == 0) wait_parts<C::LOADS, RK + RV>((int)((d_c >> 20) & 31u));
      __syncthreads();
      if (grp == 0) issue((int)((d_c >> 25) & 31u));
    };

    // Iteration p, software pipelined within each wave: QK of step p runs on
    // the matrix cores while the exponentials of step p - 1 run on the vector
    // ALU, then PV of step p - 1 runs while the row max of step p is formed.
    // The MFMAs are unconditional (one code path keeps every accumulator in
    // one register set): a missing tile has zero operands, and a missing
    // previous step is exponentiated with an infinite offset, giving P = 0.
    // sc holds the scores of step p - 1, sn receives those of step p; the
    // loop is unrolled by two so the two score tiles swap roles instead of
    // being copied.
    auto iter = [&](int p, const f32x16& sc, f32x16& sn) {
      step_barrier(p);
      const bool has_c = (d_c >> (16 + grp)) & 1u;   // this half has a tile in step p
      const bool has_p = (d_c >> (18 + grp)) & 1u;   // ... in step p - 1
      const uint32_t kslot = (d_c >> (4 * grp)) & 15u;
      const uint32_t vslot = (d_c >> (8 + 4 * grp)) & 15u;
      bf16x8 ka[D / 16];
      bf16x8 va[C::OT][2];
      if constexpr (ZT) {
        // a half without a tile reads the zero tile: no branch
        const char* kbase = smem + (has_c ? kslot * C::TILE : (uint32_t)ZERO_OFF);
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) ka[ks] = *reinterpret_cast<const bf16x8*>(kbase + k_off[ks]);
        // v_off includes the V ring base
        const char* vbase = smem + (has_p ? vslot * C::TILE : (uint32_t)(ZERO_OFF - V_BASE));
#pragma unroll
        for (int t = 0; t < C::OT; ++t)
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const i16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_i16x4*)(vbase + v_off[t] + (16 * j) * C::ROWB));
            const i16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_i16x4*)(vbase + v_off[t] + (16 * j + 8) * C::ROWB));
            va[t][j] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
          }
      } else if (has_c) {
        const char* base = smem + kslot * C::TILE;
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) ka[ks] = *reinterpret_cast<const bf16x8*>(base + k_off[ks]);
      } else {
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks)
#pragma unroll
          for (int e = 0; e < 8; ++e) ka[ks][e] = (__bf16)0.f;
      }
      if (ZT) {
      } else if (has_p) {
        // For k-step j the A operand of lane (g, d-row) holds keys base +
        // 0..3 and base + 8..11 with base = 32*kh + 16*j + 4*g: exactly the
        // keys of pb[j]'s slots.
        const char* base = smem + vslot * C::TILE;   // v_off includes the V ring base
#pragma unroll
        for (int t = 0; t < C::OT; ++t)
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const i16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_i16x4*)(base + v_off[t] + (16 * j) * C::ROWB));
            const i16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_i16x4*)(base + v_off[t] + (16 * j + 8) * C::ROWB));
            va[t][j] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
          }
      } else {
#pragma unroll
        for (int t = 0; t < C::OT; ++t)
#pragma unroll
          for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 8; ++e) va[t][j][e] = (__bf16)0.f;
      }
      // Lazy rescale for step p - 1: the offset only moves when the block max
      // exceeds it by more than kTau.  o already holds PV of step p - 2.
      if (has_p && __ballot(mx_prev > m_used + kTau) != 0ull) {
        const float m_new = fmaxf(m_used, mx_prev);
        const float alpha = __builtin_amdgcn_exp2f(m_used - m_new);
        l_part *= alpha;
#pragma unroll
        for (int t = 0; t < C::OT; ++t)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[t][r] *= alpha;
        m_used = m_new;
      }
      const float m_off = has_p ? m_used : INFINITY;

      // QK(p) with the exponentials of step p - 1.  P^T is the B operand:
      // k-step j covers registers 8j..8j+7, i.e. keys 16j + 8*(e/4) + 4*g +
      // e%4 for slot e.  The row sum is kept in fp32 from the unrounded
      // probabilities (accurate log-sum-exp).
      constexpr int NQK = D / 16;          // QK MFMAs per step
      constexpr int EPM = 16 / NQK;        // exponentials per MFMA
#pragma unroll
      for (int r = 0; r < 16; ++r) sn[r] = 0.f;
      bf16x8 pb[2];
#pragma unroll
      for (int i = 0; i < NQK; ++i) {
        sn = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[i], qf[i], sn, 0, 0, 0);
#pragma unroll
        for (int u = 0; u < EPM; ++u) {
          const int e = i * EPM + u;
          const float pr = __builtin_amdgcn_exp2f(fmaf(sc[e], c_log2, -m_off));
          l_part += pr;
          pb[e >> 3][e & 7] = (__bf16)pr;
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if constexpr (PAD) {
        // The masking branch below would otherwise let the compiler sink the
        // exponentials past it, next to the PV products that consume them,
        // where nothing overlaps them: keep them with the QK products.
        typedef int i32x4 __attribute__((ext_vector_type(4)));
        asm volatile("" ::"v"(__builtin_bit_cast(i32x4, pb[0])), "v"(__builtin_bit_cast(i32x4, pb[1])),
                     "v"(l_part));
      }
      // A key tile that reaches past the grid: its padded positions are not
      // keys (score -inf, so they add nothing to the row max or the sum).
      if (PAD && ((d_c >> (30 + grp)) & 1u)) {
        const uint32_t e = sched[p];
        const int32_t cube = __builtin_amdgcn_readfirstlane((int32_t)(grp == 0 ? (e & 0xffffu) : (e >> 16)));
        const uint64_t real = cube_mask(tmap, cube_at(tmap, cube));   // bit l: position l is a real token
        // this lane's keys 32*kh + 4*g + 8*q + j (q, j < 4) are bits 8*q + j of m
        const uint64_t m = real >> (32 * kh + 4 * g);
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (!((m >> (8 * (r >> 2) + (r & 3))) & 1ull)) sn[r] = -INFINITY;
      }
      // PV(p-1) with the row max of step p.
      float mx = kNegBig;
#pragma unroll
      for (int i = 0; i < 2 * C::OT; ++i) {
        const int t = i % C::OT, j = i / C::OT;
        o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[t][j], pb[j], o[t], 0, 0, 0);
        constexpr int MPM = 16 / (2 * C::OT);   // max inputs per MFMA
#pragma unroll
        for (int u = 0; u < MPM; ++u) mx = fmaxf(mx, sn[i * MPM + u]);
        __builtin_amdgcn_sched_barrier(0);
      }
      mx_prev = pair_max(mx) * c_log2;
    };
    f32x16 sc2;
    for (int p = 0; p <= S; p += 2) {
      iter(p, sc, sc2);
      if (p + 1 > S) break;
      iter(p + 1, sc2, sc);
    }
    __syncthreads();   // every wave is done with the ring before it is reused

    // ---- merge the two key halves, normalise, combine, store ----
    // Each key half finishes half of the d tiles (kh 0 the first OT / 2, kh 1
    // the rest): it hands the other half's tiles over through LDS with its
    // (offset, row sum), then merges both halves' partials of its own tiles.
    // Either wave forms the merged value as fma(x0, a0, x1 * a1) * inv with
    // x0, x1 the partials of key halves 0 and 1, so every tile is merged the
    // same way whichever half finishes it.
    const float l_row = pair_sum(l_part);
    constexpr int HT = C::OT / 2;    // d tiles each key half finishes
    constexpr int HV = HT * 16;      // their accumulators per lane
    float* mbuf = reinterpret_cast<float*>(smem + grp * C::MERGE_G);                 // [qh][4 + NOV][64]
    float* ost = reinterpret_cast<float*>(smem + 2 * C::MERGE_G + grp * C::OST_G);   // [64][OSTR]
    float* b = mbuf + qh * (C::NOV + 4) * 64;   // rows 0-3: (offset, sum) of kh 0, of kh 1; then kh 0's, kh 1's hand-over
    auto hand_over = [&](auto khc) {
      constexpr int KH = decltype(khc)::value;
#pragma unroll
      for (int u = 0; u < HT; ++u)
#pragma unroll
        for (int r = 0; r < 16; ++r) b[(4 + KH * HV + u * 16 + r) * 64 + lane] = o[(1 - KH) * HT + u][r];
    };
    b[(2 * kh) * 64 + lane] = m_used;
    b[(2 * kh + 1) * 64 + lane] = l_row;
    if (kh == 0) hand_over(std::integral_constant<int, 0>{}); else hand_over(std::integral_constant<int, 1>{});
    __syncthreads();
    {
      const float m0 = b[lane], l0 = b[64 + lane], m1 = b[128 + lane], l1 = b[192 + lane];
      const float m = fmaxf(m0, m1);
      const float a0 = (m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m0 - m);
      const float a1 = (m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m1 - m);
      const float l = fmaf(l0, a0, l1 * a1);
      const float inv = l > 0.f ? 1.f / l : 0.f;
      float* orow = ost + (32 * qh + n32) * C::OSTR;
      auto finish = [&](auto khc) {
        constexpr int KH = decltype(khc)::value;
        const float* other = b + (4 + (1 - KH) * HV) * 64;   // the other half's partials of these tiles
#pragma unroll
        for (int u = 0; u < HT; ++u)
#pragma unroll
          for (int rq = 0; rq < 4; ++rq) {
            float w[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float own = o[KH * HT + u][4 * rq + e];
              const float oth = other[(u * 16 + 4 * rq + e) * 64 + lane];
              const float x0 = KH == 0 ? own : oth, x1 = KH == 0 ? oth : own;
              w[e] = fmaf(x0, a0, x1 * a1) * inv;
            }
            // d = 32*t + 8*rq + 4*g + 0..3
            *reinterpret_cast<float4*>(orow + 32 * (KH * HT + u) + 8 * rq + 4 * g) = make_float4(w[0], w[1], w[2], w[3]);
          }
      };
      if (kh == 0) finish(std::integral_constant<int, 0>{}); else finish(std::integral_constant<int, 1>{});
      const int32_t my_tok = 32 * qh + n32;
      const CubeAt mq = tmap.on ? cube_at(tmap, my_cube) : CubeAt{0, 0, 0, true};
      if (kh == 0 && lse != nullptr && g == 0 && my_valid && mq.ok &&
          (!PAD || !tmap.on || token_real(tmap, mq, my_tok))) {
        const float val = (l > 0.f) ? (m + __log2f(l)) * 0.69314718055994531f : -INFINITY;
        lse[bh * (int64_t)(tmap.on ? tmap.N : tmap.Np) + token_pos(tmap, my_cube, mq, my_tok)] = val;
      }
    }
    __syncthreads();

    const CubeAt mq = tmap.on ? cube_at(tmap, my_cube) : CubeAt{0, 0, 0, true};
    if (my_valid && mq.ok) {
      const int64_t my_row = rowA + grp;
      const float* ocrow = oc ? oc + my_row * (int64_t)D : nullptr;
      // thread index within the half, as an opaque copy: the rows and
      // columns below are then derived here, instead of once before the pair
      // loop and held (spilled) through the step loop
      int gt = tid & 255;
      asm volatile("" : "+v"(gt));
      // Without gates (and without padding) the rows are written by a loop
      // with no branch, so that its staging reads can all be issued before
      // the first store; the general loop below tests the gates per row.
      if (!PAD && gate_f == nullptr && gate_c == nullptr) {
#pragma unroll
        for (int u = 0; u < kBlk * C::CPR / 256; ++u) {
          const int c = gt + u * 256;
          const int row = c / C::CPR, col = c % C::CPR;
          const int64_t gidx = token_elem(tmap, bh, my_cube, mq, row, D) + col * 8;
          const float4 v0 = *reinterpret_cast<const float4*>(ost + row * C::OSTR + col * 8);
          const float4 v1 = *reinterpret_cast<const float4*>(ost + row * C::OSTR + col * 8 + 4);
          uint4 packed;
          packed.x = pack_bf16x2(v0.x, v0.y);
          packed.y = pack_bf16x2(v0.z, v0.w);
          packed.z = pack_bf16x2(v1.x, v1.y);
          packed.w = pack_bf16x2(v1.z, v1.w);
          *reinterpret_cast<uint4*>(out + gidx) = packed;
        }
      } else {
#pragma unroll
        for (int u = 0; u < kBlk * C::CPR / 256; ++u) {
          const int c = gt + u * 256;
          const int row = c / C::CPR, col = c % C::CPR;
          if (PAD && tmap.on && !token_real(tmap, mq, row)) continue;   // padding: no raster row
          const int64_t gidx = token_elem(tmap, bh, my_cube, mq, row, D) + col * 8;
          float val[8];
          const float4 v0 = *reinterpret_cast<const float4*>(ost + row * C::OSTR + col * 8);
          const float4 v1 = *reinterpret_cast<const float4*>(ost + row * C::OSTR + col * 8 + 4);
          val[0] = v0.x; val[1] = v0.y; val[2] = v0.z; val[3] = v0.w;
          val[4] = v1.x; val[5] = v1.y; val[6] = v1.z; val[7] = v1.w;
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
    }
    __syncthreads();   // staging reads done before the next pair reuses LDS
  }
}

// Per-device launch state: the CU count and the dynamic-LDS limit already
// granted to each instantiation.
struct DevState {
  int cus = 0;
  int lds_granted[16] = {};
};

std::mutex dev_state_mutex;

template <int D, int RK, int RV, bool PAD, bool ZT>
hipError_t launch_ring(const Geom& g, const void* q, const void* k, const void* v, const int32_t* lut,
                       const int32_t* valid, int max_kv, const float* oc, const void* gate_c,
                       const void* gate_f, void* out, float* lse, hipStream_t s, size_t sched_bytes, int slot,
                       const TokenMap& tmap, bool gather) {
  using C = Cfg<D>;
  static DevState dev_state[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  DevState& st = dev_state[dev];
  auto kern = sparse_attn_fwd_kernel<D, RK, RV, PAD, ZT>;
  size_t lds = (size_t)(RK + RV) * C::TILE + sched_bytes;
  if (lds < (size_t)C::EPI_BYTES) lds = C::EPI_BYTES;
  if (ZT) {
    if (lds > (size_t)(kLdsMax - C::TILE)) return hipErrorInvalidValue;
    lds = kLdsMax;   // the zero tile is the last TILE bytes
  }
  if (lds > (size_t)kLdsMax) return hipErrorInvalidValue;
  int cus = 0;
  {
    // host threads may launch concurrently: grant and record under one lock
    std::lock_guard<std::mutex> lock(dev_state_mutex);
    if (st.lds_granted[slot] < (int)lds) {
      hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return e;
      st.lds_granted[slot] = (int)lds;
    }
    if (st.cus == 0) {
      hipError_t e = hipDeviceGetAttribute(&st.cus, hipDeviceAttributeMultiprocessorCount, dev);
      if (e != hipSuccess || st.cus <= 0) {
        st.cus = 0;
        return e != hipSuccess ? e : hipErrorInvalidDevice;
      }
    }
    cus = st.cus;
  }
  const int64_t total_pairs = g.BH * ((g.Nc + 1) / 2);
  // persistent grid: one workgroup per CU, a multiple of 8 (one share per XCD)
  int64_t grid = ((int64_t)cus + 7) / 8 * 8;
  const int64_t need = (total_pairs + 7) / 8 * 8;
  if (grid > need) grid = need;
  const float c_log2 = 1.4426950408889634f / sqrtf((float)D);
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kThreads), lds, s, (const __bf16*)q, (const __bf16*)k,
                     (const __bf16*)v, lut, valid, max_kv, oc, (const __bf16*)gate_c, (const __bf16*)gate_f,
                     (__bf16*)out, lse, (int)g.Nc, total_pairs, c_log2, tmap, g.group, gather ? 1 : 0);
  return hipGetLastError();
}

// LDS after the tile ring: step list, load plan, step descriptors, tile
// list, flags and two Nc-bit maps.
size_t sched_bytes(const Geom& g, int max_kv) {
  const size_t nwords = (size_t)(g.Nc + 31) / 32;
  const size_t m = (size_t)max_kv;
  return 4 * m + 4 * (m + 2) + 4 * (m + 1) + 16 * m + 16 + 2 * 4 * nwords;
}

constexpr size_t kBaseRingBytes = 128 * 1024;   // 4 + 4 tiles at d = 128, 8 + 8 at d = 64

// Ring shapes: at d = 128 four K and four V positions (measured as fast as
// five and four); at d = 64 ten and eight whenever the schedule fits beside
// them, else eight and eight.  The zero tile (ZT) takes the last tile of LDS
// whenever the ring and the schedule leave it free (not with padded grids at
// d = 128).
template <int D, bool PAD>
hipError_t launch_d(const Geom& g, const void* q, const void* k, const void* v, const int32_t* lut,
                    const int32_t* valid, int max_kv, const float* oc, const void* gate_c,
                    const void* gate_f, void* out, float* lse, hipStream_t s, const TokenMap& tmap,
                    bool gather) {
  using C = Cfg<D>;
  constexpr int RK_DEEP = D == 128 ? 4 : 10, RV_DEEP = D == 128 ? 4 : 8;
  constexpr int R_BASE = D == 128 ? 4 : 8;
  static_assert((size_t)2 * R_BASE * C::TILE == kBaseRingBytes, "base ring size");
  if (!sparse_attn_fwd_fits(g, max_kv)) return hipErrorInvalidValue;
  const size_t sched = sched_bytes(g, max_kv);
  const size_t build_scratch = 16 * (size_t)max_kv;   // SH, EXA, EXB, PK
  const size_t zfree = (size_t)kLdsMax - C::TILE;     // LDS below the zero tile
  const int slot0 = (D == 128 ? 3 : 0) + (PAD ? 6 : 0);
  constexpr size_t DEEP = (size_t)(RK_DEEP + RV_DEEP) * C::TILE;
  if constexpr (RK_DEEP != R_BASE) {
    if (DEEP + sched <= zfree && build_scratch <= DEEP)
      return launch_ring<D, RK_DEEP, RV_DEEP, PAD, true>(g, q, k, v, lut, valid, max_kv, oc, gate_c, gate_f, out,
                                                        lse, s, sched, slot0, tmap, gather);
  }
  if (build_scratch > kBaseRingBytes) return hipErrorInvalidValue;
  // (the padded d = 128 variant keeps its branches: with the zero tile it
  // spills a register)
  if (!(PAD && D == 128) && kBaseRingBytes + sched <= zfree)
    return launch_ring<D, R_BASE, R_BASE, PAD, !(PAD && D == 128)>(g, q, k, v, lut, valid, max_kv, oc, gate_c, gate_f, out, lse, s,
                                                    sched, slot0 + 1, tmap, gather);
  return launch_ring<D, R_BASE, R_BASE, PAD, false>(g, q, k, v, lut, valid, max_kv, oc, gate_c, gate_f, out, lse, s,
                                                   sched, slot0 + 2, tmap, gather);
}

}  // namespace

// Cube ids and ring positions are 16-bit fields of the step list and the
// load plan, and the per-pair schedule must fit in LDS beside the base ring
// (its build scratch, 16 bytes per entry, lives in the ring).
static bool pair_fits(const Geom& g, int max_kv) {
  if (g.Nc < 1 || g.Nc > 0xfffe || max_kv < 1 || max_kv > 0x7fff) return false;
  if (kBaseRingBytes + sched_bytes(g, max_kv) > (size_t)kLdsMax) return false;
  return 16 * (size_t)max_kv <= kBaseRingBytes;
}

bool sparse_attn_fwd_fits(const Geom& g, int max_kv) {
  return sparse_attn_fwd_quad_fits(g, max_kv) || pair_fits(g, max_kv);
}

// The gathering pair kernel reads each 1 KiB piece of a cube tile as one run
// of tokens along w: at d = 128 that is cw = 4 tokens.  Grids padded up to
// whole cubes have positions with no raster row, so they are not gathered;
// token rows are 27-bit fields of the tile list.
bool sparse_attn_fwd_gather_fits(const Geom& g, int max_kv) {
  return g.D == 128 && g.Dv == 128 && g.cw * 128 * 2 == 1024 && !g.padded && g.vol == kBlk &&
         g.N < ((int64_t)1 << 27) && pair_fits(g, max_kv);
}

hipError_t launch_sparse_attn_fwd(const Geom& g, const void* q, const void* k, const void* v,
                                  const int32_t* lut, const int32_t* valid, int max_kv,
                                  const float* oc, const void* gate_c, const void* gate_f,
                                  void* out, float* lse, int out_order, hipStream_t s, bool gather) {
  if (gather) {   // q, k, v in raster order: the pair kernel gathers their cube tiles
    if (!sparse_attn_fwd_gather_fits(g, max_kv) || out_order != 1) return hipErrorInvalidValue;
    return launch_d<128, false>(g, q, k, v, lut, valid, max_kv, oc, gate_c, gate_f, out, lse, s,
                                make_token_map(g, out_order), true);
  }
  // Quads of query cubes when the rows list at least half of the cubes
  // (measured on the 32K-token layer: Top-256 3.62 ms against 3.7, all 512
  // cubes 6.17 against 6.5); below that, neighbouring quads' key sets cover
  // more cubes than an XCD's L2 holds and the pair kernel is faster (Top-154
  // 2.20 vs 2.20, the 1,920-cube layer at Top-192 46.6 vs 42.1 ms).
  if (2 * (int64_t)max_kv >= g.Nc && sparse_attn_fwd_quad_fits(g, max_kv))
    return launch_sparse_attn_fwd_quad(g, q, k, v, lut, valid, max_kv, oc, gate_c, gate_f, out, lse, out_order, s);
  const TokenMap m = make_token_map(g, out_order);
  if (g.D == 128 && g.padded)
    return launch_d<128, true>(g, q, k, v, lut, valid, max_kv, oc, gate_c, gate_f, out, lse, s, m, false);
  if (g.D == 128) return launch_d<128, false>(g, q, k, v, lut, valid, max_kv, oc, gate_c, gate_f, out, lse, s, m, false);
  if (g.D == 64 && g.padded)
    return launch_d<64, true>(g, q, k, v, lut, valid, max_kv, oc, gate_c, gate_f, out, lse, s, m, false);
  if (g.D == 64) return launch_d<64, false>(g, q, k, v, lut, valid, max_kv, oc, gate_c, gate_f, out, lse, s, m, false);
  return hipErrorInvalidValue;
}

}  // namespace vsa
