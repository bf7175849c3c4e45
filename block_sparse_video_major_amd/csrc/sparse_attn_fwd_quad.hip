// Fine block-sparse attention with the gated combination, four query cubes
// per workgroup, for gfx950.
//
// "VSA: Accelerating Video Diffusion Inference with Sparse Attention on AMD
// GPUs": §Two-Stage Architecture (Stage 2 attends each query cube's tokens to
// the tokens of the key/value cubes the coarse stage selected; the output
// combines the coarse and fine outputs through gates), §Block-Sparse Encoding
// (an index list plus a valid count per query block), §Kernel Architecture
// (QK^T, online softmax with running max and sum, PV) and §Sparse Traversal
// (the loop over the listed key/value blocks).  "VSA: Faster Video Diffusion
// with Trainable Sparse Attention", Abstract.  The attention is
// softmax(QK^T / sqrt(d)) V as in §The Attention Bottleneck in Video
// Diffusion.
//
// Work decomposition:
//   * One workgroup of 8 wavefronts per CU, persistent.  A workgroup takes a
//     QUAD of neighbouring query cubes (4i .. 4i+3) of one (batch, head).
//     Wave w serves cube w >> 1 and its queries 32*(w & 1) .. +31, over all
//     64 keys of every key cube it visits, so its softmax state never needs
//     merging with another wave.  Each XCD owns one contiguous range of quads.
//   * Step schedule.  Neighbouring query cubes select largely the same key
//     cubes; the quad visits the union of its four lists in steps, a step
//     giving each cube at most one key cube, and a key cube listed by several
//     cubes of the quad is visited by all of them in the same step, so its
//     K/V tiles are fetched once.  Key cubes are grouped by the set of query
//     cubes that list them: the cubes all four list first, then one block per
//     three-cube set, then the two-cube sets in complementary pairs side by
//     side ({0,1} with {2,3}, {0,2} with {1,3}, {0,3} with {1,2}), and every
//     cube's remaining (own) key cubes fill its idle slots in that order,
//     then run side by side.  On the 32K-token Top-154 workload this takes
//     154.3 steps for 154 cubes per row and fetches 1.84 tiles per step for
//     four query cubes (pairs of cubes: 1.36 per step for two).  Attention
//     sums over each cube's own key set, so the visiting order only changes
//     fp32 rounding.  Quads with a row that lists a cube twice (each listing
//     is attended) visit the lists position by position instead.
//   * Scores are formed transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x16_bf16: K rows from LDS as the A operand, Q in
//     registers as the B operand.  Each lane owns one query and 32 of its 64
//     keys; the row max is a lane-local max plus one v_permlane32_swap.
//   * O^T += V^T P^T: P (bf16) is already in B-operand layout; V^T is read
//     from the V tile in its natural [key][d] order with ds_read_b64_tr_b16.
//   * Software pipeline per wave, one barrier per step: the QK MFMAs of step
//     p run beside the exponentials of step p - 1, the PV MFMAs of step p - 1
//     beside the row max of step p.
//   * Tiles arrive by direct global->LDS loads into one FIFO ring of R tile
//     slots.  Load group g holds the K tiles of step g and the V tiles of
//     step g - 1 (V is consumed one step after K), so every tile of group g
//     is dead once step g is done: at barrier p groups < p are free, and the
//     groups that then fit are issued.  The tile list is built once per
//     quad; waves 0-3 (one per SIMD) move a quarter of every tile each, in
//     one burst right after the barrier, while waves 4-7 go straight to
//     their products.  Direct loads of one CU pass its address unit one
//     1 KiB piece at a time, so a burst over all eight waves would hold all
//     of them; measured on the 32K-token Top-154 workload, loading only the
//     K tiles takes 1.99 ms instead of 2.34, loading into registers instead
//     of LDS 1.94, and no loads at all 1.50.  16-byte chunks are XOR swizzled
//     per row so every LDS read pattern is conflict free.
//   * Lazy rescaling: the exponent offset only moves when a block's max
//     exceeds it by more than 8 (log2 units), keeping every exp2 <= 256.
//   * Epilogue: O normalised, staged in LDS, combined with the gates and the
//     broadcast coarse output and written with coalesced 16-byte stores in
//     the requested token order.
#include <mutex>

#include "mfma_util.h"
#include "token_map.h"
#include "vsa_internal.h"

namespace vsa {
namespace {

constexpr int kBlk = 64;              // tokens per cube
constexpr int kThreads = 512;         // 8 wavefronts: 4 cubes x 2 query halves
constexpr int kQuad = 4;              // query cubes per workgroup
constexpr float kTau = 8.0f;          // lazy-rescale threshold (log2 units)
constexpr float kNegBig = -1.0e30f;   // initial exponent offset
constexpr uint32_t kNone = 0xffffu;   // no key cube in this step for this cube
constexpr int kMaxRing = 15;          // ring slots fit a 4-bit field; 15 = none
constexpr int kMinRing = 8;           // one load group holds up to 8 tiles

template <int D>
struct QCfg {
  static constexpr int ROWB = D * 2;                 // bytes per token row
  static constexpr int CPR = D / 8;                  // 16-byte chunks per row
  static constexpr int TILE = kBlk * ROWB;           // one K or V cube tile
  static constexpr int PIECES = TILE / 1024;         // 1 KiB direct-load pieces per tile
  static constexpr int PPW = PIECES / 8;             // pieces per wave per tile
  static constexpr int OT = D / 32;                  // 32-row tiles of O^T
  static constexpr int KS = D / 16;                  // k-steps of the QK contraction
  static constexpr int OSTR = D + 4;                 // fp32 staging row stride
  static constexpr int OST = kBlk * OSTR * 4;        // staging of one cube
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

// Four 1 KiB pieces: for piece j = 0..3 lane i moves the 16 bytes at
// base + o_j + 1024 j to LDS byte address m0 + 1024 j + 16 i (the
// instruction offset moves both the source and the LDS destination).
// Issued through inline assembly so that the compiler does not track these
// LDS writes; completion is enforced explicitly (vmcnt wait + barrier)
// before any wave reads the slot.
// One 1 KiB piece: lane i moves the 16 bytes at base + voff to LDS byte
// address m0 + 16 i.
__device__ __forceinline__ void dma_piece(const char* base, uint32_t voff, uint32_t m0) {
  asm volatile(
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, %2"
      :
      : "v"(voff), "s"(m0), "s"(base)
      : "memory", "m0");
}

__device__ __forceinline__ void dma_pair(const char* base, uint32_t o0, uint32_t o1, uint32_t m0) {
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, %3\n\t"
      "global_load_lds_dwordx4 %1, %3 offset:1024"
      :
      : "v"(o0), "v"(o1), "s"(m0), "s"(base)
      : "memory", "m0");
}

__device__ __forceinline__ void dma_quad(const char* base, uint32_t o0, uint32_t o1, uint32_t o2, uint32_t o3,
                                         uint32_t m0) {
  asm volatile(
      "s_mov_b32 m0, %4\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, %5\n\t"
      "global_load_lds_dwordx4 %1, %5 offset:1024\n\t"
      "global_load_lds_dwordx4 %2, %5 offset:2048\n\t"
      "global_load_lds_dwordx4 %3, %5 offset:3072"
      :
      : "v"(o0), "v"(o1), "v"(o2), "v"(o3), "s"(m0), "s"(base)
      : "memory", "m0");
}

// Wait until at most n (0..15) tiles' worth of this wave's direct loads (P
// pieces per tile) are still pending: a binary decision over n, four
// scalar branches deep, ending in one s_waitcnt with a constant count.
template <int P, int LO, int HI>
__device__ __forceinline__ void wait_tiles(int n) {
  if constexpr (LO == HI) {
    wait_vmem<LO * P>();
  } else {
    constexpr int MID = (LO + HI + 1) / 2;
    if (n >= MID) wait_tiles<P, MID, HI>(n);
    else wait_tiles<P, LO, MID - 1>(n);
  }
}

// Layout of the LDS after the tile ring (kept for the whole quad):
//   sched[s]  (uint2)  the key cube of each of the 4 query cubes in step s
//                      (16 bits each, kNone = none)
//   dsc[p]    (uint4)  what iteration p needs:
//     .x  bits 4c..4c+3 = ring slot of cube c's K tile of step p (15 =
//         none); bits 16+4c.. = ring slot of cube c's V tile of step p-1
//     .y  the list index up to which tiles are issued by the end of barrier
//         p (the groups that fit in the ring once groups < p are dead)
//     .z  the list index where the tiles of groups > p begin (everything
//         below it must have landed by barrier p)
//     .w  bit 0: the step's own group is only issued after barrier p (then
//         a second wait and barrier); bits 1-4: cube c's K tile of step p
//         reaches past the grid (padded grids)
//   tlist[i]  (uint32) every tile load of the quad in issue order: group g =
//         the distinct key cubes of step g (K tiles), then those of step
//         g - 1 (V tiles), each in the order of first appearance over cubes
//         0..3; entry = cube | (1 if V) << 16.  Tile i sits in ring slot
//         i % R.
struct QuadMeta {
  int s_max;       // steps a quad can need
  int t_max;       // tile loads a quad can need
  size_t sched_off, dsc_off, tlist_off, bytes;
};

// A quad needs at most min(2 max_kv, Nc) steps when no row lists a cube
// twice (every step holds a distinct key cube, and the blocks before the
// own-cube tail hold at most half of the four rows' entries), and max_kv
// steps when one does (position by position; max_kv <= Nc).  Each step
// loads each of its distinct key cubes twice (K and V): at most
// 2 * min(4 max_kv, Nc) tiles without repeats, 8 max_kv with them.
__host__ __device__ inline QuadMeta quad_meta(int64_t Nc, int max_kv, size_t ring_bytes) {
  QuadMeta m;
  const int64_t s2 = 2 * (int64_t)max_kv;
  int64_t s = s2 < Nc ? s2 : Nc;
  if (s < max_kv) s = max_kv;
  m.s_max = (int)s;
  m.t_max = 8 * max_kv;
  m.sched_off = ring_bytes;
  m.dsc_off = m.sched_off + 8 * (size_t)m.s_max;
  m.tlist_off = m.dsc_off + 16 * ((size_t)m.s_max + 1);
  m.bytes = 8 * (size_t)m.s_max + 16 * ((size_t)m.s_max + 1) + 4 * (size_t)m.t_max;
  return m;
}

// Scratch for the schedule build, inside the ring (idle until the first
// tile load of the quad): 4 membership bitmaps, per-chunk class counts,
// group positions and the last group each barrier may issue.
struct BuildScratch {
  uint2* tmp;        // [s_max] steps in block order, before sorting
  uint32_t* bm;      // [4][nwords] membership bitmaps
  int* cc;           // [nchunks][16] class counts of each 64-cube chunk, then exclusive prefixes
  int* info;         // [32]: 0 duplicate flag, 16..31 class sizes
  int* gpos;         // [s_max + 2] first tile index of each load group
  int* last;         // [s_max + 1] last group issued by barrier p
  uint32_t* mk;      // [nwords] bitmap of the steps' smallest key cubes
  int* wpre;         // [nwords] exclusive prefix of its popcounts
};

__device__ __forceinline__ BuildScratch build_scratch(char* smem, int nwords, int nchunks, int s_max) {
  BuildScratch b;
  b.tmp = reinterpret_cast<uint2*>(smem);
  b.bm = reinterpret_cast<uint32_t*>(b.tmp + s_max);
  b.cc = reinterpret_cast<int*>(b.bm + 4 * nwords);
  b.info = b.cc + 16 * nchunks;
  b.gpos = b.info + 32;
  b.last = b.gpos + s_max + 2;
  b.mk = reinterpret_cast<uint32_t*>(b.last + s_max + 1);
  b.wpre = reinterpret_cast<int*>(b.mk + nwords);
  return b;
}

__host__ __device__ inline size_t build_scratch_bytes(int64_t Nc, int s_max) {
  const int64_t nwords = (Nc + 31) / 32, nchunks = (Nc + 63) / 64;
  return 8 * (size_t)s_max + 4 * (4 * nwords + 16 * nchunks + 32 + (s_max + 2) + (s_max + 1) + 2 * nwords);
}

// Members of each cube class: bit c set = query cube c lists the key cube.
// Steps: class 15, then 7, 11, 13, 14, then the complementary pairs
// (3,12), (5,10), (6,9) side by side, then every cube's own cubes.
__device__ __forceinline__ int class_base(const int* n, int m, int* len_out) {
  // running bases in the fixed block order
  const int b7 = n[15], b11 = b7 + n[7], b13 = b11 + n[11], b14 = b13 + n[13];
  const int p1 = b14 + n[14];
  const int l1 = max(n[3], n[12]);
  const int p2 = p1 + l1;
  const int l2 = max(n[5], n[10]);
  const int p3 = p2 + l2;
  const int l3 = max(n[6], n[9]);
  if (len_out) *len_out = p3 + l3;   // B: steps before the own-cube tail
  switch (m) {
    case 15: return 0;
    case 7: return b7;
    case 11: return b11;
    case 13: return b13;
    case 14: return b14;
    case 3: case 12: return p1;
    case 5: case 10: return p2;
    case 6: case 9: return p3;
    default: return 0;
  }
}

// Step of the j-th own (single-cube) key cube of cube c: its holes in the
// blocks above in step order, then the tail from B on.
__device__ __forceinline__ int single_pos(const int* n, int c, int j) {
  int B;
  (void)class_base(n, 15, &B);
  const int m3 = 15 ^ (1 << c);               // the three-cube block without c
  int lo = class_base(n, m3, nullptr), len = n[m3];
  if (j < len) return lo + j;
  j -= len;
  // complementary pair blocks: c sits in exactly one class of each pair
  const int pa[3] = {3, 5, 6}, pb[3] = {12, 10, 9};
  for (int i = 0; i < 3; ++i) {
    const int mine = ((pa[i] >> c) & 1) ? pa[i] : pb[i];
    const int base = class_base(n, pa[i], nullptr);
    const int blen = max(n[pa[i]], n[pb[i]]);
    const int holes = blen - n[mine];
    if (j < holes) return base + n[mine] + j;
    j -= holes;
  }
  return B + j;
}

__device__ __forceinline__ uint32_t step_cube(const uint2 w, int c) {
  const uint32_t x = c < 2 ? w.x : w.y;
  return (c & 1) ? (x >> 16) : (x & 0xffffu);
}

// Distinct key cubes of a step; first_idx[c] = the index of cube c's key
// cube among them in order of first appearance (-1: none).
__device__ __forceinline__ int step_distinct(const uint2 w, int* first_idx) {
  uint32_t e[kQuad];
#pragma unroll
  for (int c = 0; c < kQuad; ++c) e[c] = step_cube(w, c);
  int n = 0;
#pragma unroll
  for (int c = 0; c < kQuad; ++c) {
    int idx = -1;
    if (e[c] != kNone) {
#pragma unroll
      for (int c2 = 0; c2 < c; ++c2)
        if (idx < 0 && e[c2] == e[c]) idx = first_idx ? first_idx[c2] : 0;
      if (idx < 0) idx = n++;
    }
    if (first_idx) first_idx[c] = idx;
  }
  return n;
}

// Builds the step list, the per-step descriptors and the tile list of the
// quad whose first query cube is cube0 (LUT row row0) in LDS; every thread
// of the workgroup (NT of them) takes part.  Returns the step count S and
// sets t_init (the tiles issued before the first step) and n_list (all of
// the quad's tiles).
template <bool PAD, int NT>
__device__ __forceinline__ int build_quad(const BuildScratch& bs, uint2* sched, uint4* dsc, uint32_t* tlist,
                                          const int32_t* __restrict__ lut, const int32_t* __restrict__ valid,
                                          int max_kv, int Nc, int64_t row0, int cube0, int R, const TokenMap& tmap,
                                          int tid, int lane, int wave, int& t_init, int& n_list) {
  const int nwords = (Nc + 31) >> 5, nchunks = (Nc + 63) >> 6;
  const uint64_t lt_mask = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  auto count_of = [&](int c) {
    if (cube0 + c >= Nc) return 0;
    const int n = valid[row0 + c];
    return n < 0 ? 0 : (n > max_kv ? max_kv : n);
  };
  int ncnt[kQuad];
#pragma unroll
  for (int c = 0; c < kQuad; ++c) ncnt[c] = count_of(c);
  const int ntot = ncnt[0] + ncnt[1] + ncnt[2] + ncnt[3];
  auto clampc = [&](int b) { return b < 0 ? 0 : (b >= Nc ? Nc - 1 : b); };   // memory-safety clamp
  auto entry = [&](int c, int j) { return clampc(lut[(row0 + c) * (int64_t)max_kv + j]); };

  // ---- step schedule -------------------------------------------------------
  for (int i = tid; i < 4 * nwords; i += NT) bs.bm[i] = 0u;
  if (tid < 32) bs.info[tid] = 0;
  __syncthreads();
  for (int i = tid; i < ntot; i += NT) {
    int c = 0, j = i;
    while (c < kQuad - 1 && j >= ncnt[c]) { j -= ncnt[c]; ++c; }
    const int u = entry(c, j);
    const uint32_t bit = 1u << (u & 31);
    if (atomicOr(&bs.bm[c * nwords + (u >> 5)], bit) & bit) bs.info[0] = 1;   // listed twice
  }
  __syncthreads();
  const bool dup = bs.info[0] != 0;
  int S;
  if (dup) {
    // position by position
    S = max(max(ncnt[0], ncnt[1]), max(ncnt[2], ncnt[3]));
    for (int s = tid; s < S; s += NT) {
      uint32_t e[kQuad];
#pragma unroll
      for (int c = 0; c < kQuad; ++c) e[c] = s < ncnt[c] ? (uint32_t)entry(c, s) : kNone;
      sched[s] = make_uint2(e[0] | (e[1] << 16), e[2] | (e[3] << 16));
    }
    __syncthreads();
  } else {
    // class of key cube u: bit c = cube c lists it.  Per 64-cube chunk the
    // class sizes (ballots), then exclusive prefixes over the chunks, then
    // every cube's rank within its class gives its step.
    auto cls = [&](int u) {
      if (u >= Nc) return 0;
      const int w = u >> 5, b = u & 31;
      return (int)(((bs.bm[w] >> b) & 1u) | (((bs.bm[nwords + w] >> b) & 1u) << 1) |
                   (((bs.bm[2 * nwords + w] >> b) & 1u) << 2) | (((bs.bm[3 * nwords + w] >> b) & 1u) << 3));
    };
    for (int ch = wave; ch < nchunks; ch += NT / 64) {
      const int m = cls(ch * 64 + lane);
      int mine = 0;
      for (int x = 1; x < 16; ++x) {
        const int cnt = __popcll(__ballot(m == x));
        if (lane == x) mine = cnt;
      }
      if (lane < 16) bs.cc[ch * 16 + lane] = lane == 0 ? 0 : mine;
    }
    __syncthreads();
    if (tid < 16) {
      // (the opaque copy keeps the compiler from holding this address
      // in a register across the whole kernel)
      int cls_id = tid;
      asm volatile("" : "+v"(cls_id));
      int run = 0;
      for (int ch = 0; ch < nchunks; ++ch) {
        const int x = bs.cc[ch * 16 + cls_id];
        bs.cc[ch * 16 + cls_id] = run;
        run += x;
      }
      bs.info[16 + cls_id] = cls_id == 0 ? 0 : run;
    }
    __syncthreads();
    const int* ncls = bs.info + 16;
    int B;
    (void)class_base(ncls, 15, &B);
    // holes of each cube before B, and its own cubes
    int tail = 0;
#pragma unroll
    for (int c = 0; c < kQuad; ++c) {
      int nonsingle = 0;
      for (int x = 1; x < 16; ++x)
        if (((x >> c) & 1) && x != (1 << c)) nonsingle += ncls[x];
      const int holes = B - nonsingle;
      const int own = ncls[1 << c];
      tail = max(tail, own - holes);
    }
    S = B + max(tail, 0);
    for (int s = tid; s < S; s += NT) bs.tmp[s] = make_uint2(kNone | (kNone << 16), kNone | (kNone << 16));
    for (int i = tid; i < nwords; i += NT) bs.mk[i] = 0u;
    __syncthreads();
    for (int ch = wave; ch < nchunks; ch += NT / 64) {
      const int u = ch * 64 + lane;
      const int m = cls(u);
      int rank = 0;
      for (int x = 1; x < 16; ++x) {
        const uint64_t b = __ballot(m == x);
        if (m == x) rank = bs.cc[ch * 16 + x] + __popcll(b & lt_mask);
      }
      if (m != 0) {
        int pos;
        if (__popc(m) == 1) pos = single_pos(ncls, __ffs(m) - 1, rank);
        else pos = class_base(ncls, m, nullptr) + rank;
        uint16_t* e = reinterpret_cast<uint16_t*>(&bs.tmp[pos]);
#pragma unroll
        for (int c = 0; c < kQuad; ++c)
          if ((m >> c) & 1) e[c] = (uint16_t)u;
      }
    }
    __syncthreads();
    // Steps in ascending order of their smallest key cube (each key cube
    // sits in one step, so these are distinct): the workgroups of an XCD
    // then sweep the key cubes of a head together, which keeps their
    // tiles in the XCD's L2 while several quads use them.
    auto step_min = [&](const uint2 w2) {
      uint32_t mn = kNone;
#pragma unroll
      for (int c = 0; c < kQuad; ++c) mn = min(mn, step_cube(w2, c));
      return mn;
    };
    for (int s = tid; s < S; s += NT) {
      const uint32_t mn = step_min(bs.tmp[s]);   // < Nc: every step holds a key cube
      if (mn < (uint32_t)Nc) atomicOr(&bs.mk[mn >> 5], 1u << (mn & 31));
    }
    __syncthreads();
    if (wave == 0) {
      int carry = 0;
      for (int base = 0; base < nwords; base += 64) {
        const int wi = base + lane;
        const int cnt = wi < nwords ? __popc(bs.mk[wi]) : 0;
        int x = cnt;   // inclusive scan over the wavefront
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const int y = __shfl_up(x, off);
          if (lane >= off) x += y;
        }
        if (wi < nwords) bs.wpre[wi] = carry + x - cnt;
        carry += __shfl(x, 63);
      }
    }
    __syncthreads();
    for (int s = tid; s < S; s += NT) {
      const uint2 w2 = bs.tmp[s];
      const uint32_t mn = step_min(w2);
      if (mn >= (uint32_t)Nc) continue;
      const int rank = bs.wpre[mn >> 5] + __popc(bs.mk[mn >> 5] & ((1u << (mn & 31)) - 1u));
      sched[rank] = w2;
    }
    __syncthreads();
  }

  // ---- load plan ------------------------------------------------------------
  // d(s) = distinct key cubes of step s.  Group g = the K tiles of step g,
  // then the V tiles of step g - 1: u(g) = d(g) + d(g - 1) tiles, the first
  // at running index gpos(g).
  if (wave == 0) {
    int carry = 0;
    for (int base = 0; base <= S; base += 64) {
      const int gi = base + lane;
      int u = 0;
      if (gi <= S) {
        if (gi < S) u += step_distinct(sched[gi], nullptr);
        if (gi > 0) u += step_distinct(sched[gi - 1], nullptr);
      }
      int x = u;   // inclusive scan over the wavefront
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(x, off);
        if (lane >= off) x += y;
      }
      if (gi <= S) bs.gpos[gi] = carry + x - u;
      carry += __shfl(x, 63);
    }
    if (lane == 0) bs.gpos[S + 1] = carry;
  }
  __syncthreads();
  // last(p) = the last group that fits in the ring at barrier p (groups < p
  // are dead then): gpos(g + 1) - gpos(p) <= R.  A group holds at most 8
  // tiles, so last(p) >= p.
  for (int pp = tid; pp <= S; pp += NT) {
    int glo = pp, ghi = S;
    const int cap = bs.gpos[pp] + R;
    while (glo < ghi) {
      const int mid = (glo + ghi + 1) >> 1;
      if (bs.gpos[mid + 1] <= cap) glo = mid; else ghi = mid - 1;
    }
    bs.last[pp] = glo;
  }
  __syncthreads();
  // descriptors and the tile list
  for (int pp = tid; pp <= S; pp += NT) {
    uint32_t x = 0xffffffffu, w = 0;
    const int gp = bs.gpos[pp];
    int fi[kQuad];
    int dk = 0;
    if (pp < S) {
      const uint2 w2 = sched[pp];
      dk = step_distinct(w2, fi);
#pragma unroll
      for (int c = 0; c < kQuad; ++c) {
        if (fi[c] < 0) continue;
        x = (x & ~(15u << (4 * c))) | ((uint32_t)((gp + fi[c]) % R) << (4 * c));
        bool first = true;
#pragma unroll
        for (int c2 = 0; c2 < c; ++c2)
          if (fi[c2] == fi[c]) first = false;
        if (first) tlist[gp + fi[c]] = step_cube(w2, c);
        if constexpr (PAD) {
          if (cube_partial(tmap, cube_at(tmap, (int)step_cube(w2, c)))) w |= 2u << c;
        }
      }
    }
    if (pp > 0) {
      const uint2 w2 = sched[pp - 1];
      (void)step_distinct(w2, fi);
#pragma unroll
      for (int c = 0; c < kQuad; ++c) {
        if (fi[c] < 0) continue;
        const int ti = gp + dk + fi[c];
        x = (x & ~(15u << (16 + 4 * c))) | ((uint32_t)(ti % R) << (16 + 4 * c));
        bool first = true;
#pragma unroll
        for (int c2 = 0; c2 < c; ++c2)
          if (fi[c2] == fi[c]) first = false;
        if (first) tlist[ti] = step_cube(w2, c) | (1u << 16);
      }
    }
    // Before barrier pp the groups <= last(pp - 1) are issued (before the
    // loop: groups <= last(0)); if that does not include group pp, it is
    // issued after the barrier and met at a second one.
    const int prev = pp == 0 ? bs.last[0] : bs.last[pp - 1];
    if (prev < pp) w |= 1u;
    dsc[pp] = make_uint4(x, (uint32_t)bs.gpos[bs.last[pp] + 1], (uint32_t)bs.gpos[pp + 1], w);
  }
  t_init = bs.gpos[bs.last[0] + 1];
  n_list = bs.gpos[S + 1];
  __syncthreads();   // descriptors and list done; the build scratch (the ring) is free
  return S;
}

template <int D, bool PAD>
__global__ __launch_bounds__(kThreads, 1) void sparse_attn_fwd_quad_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    const int32_t* __restrict__ lut, const int32_t* __restrict__ valid, int max_kv,
    const float* __restrict__ oc, const __bf16* __restrict__ gate_c, const __bf16* __restrict__ gate_f,
    __bf16* __restrict__ out, float* __restrict__ lse, int Nc, int64_t total_quads, float c_log2,
    TokenMap tmap, int group, int R) {
  using C = QCfg<D>;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const QuadMeta meta = quad_meta(Nc, max_kv, (size_t)R * C::TILE);
  uint2* sched = reinterpret_cast<uint2*>(smem + meta.sched_off);
  uint4* dsc = reinterpret_cast<uint4*>(smem + meta.dsc_off);
  uint32_t* tlist = reinterpret_cast<uint32_t*>(smem + meta.tlist_off);
  const int nwords = (Nc + 31) >> 5, nchunks = (Nc + 63) >> 6;
  const BuildScratch bs = build_scratch(smem, nwords, nchunks, meta.s_max);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int cq = wave >> 1;               // this wave's cube within the quad
  const int qh = wave & 1;                // its query half
  const int n32 = lane & 31, g = lane >> 5;
  const int l16 = lane & 15, h16 = (lane >> 4) & 1;
  const uint64_t lt_mask = lane == 0 ? 0ull : (~0ull >> (64 - lane));

  // ---- per-lane constant offsets ------------------------------------------
  // Direct loads: lane i of 1 KiB piece n of a tile fills LDS chunk
  // 64 n + i, which holds logical chunk (i % CPR) ^ f(row) of row
  // (64 n + i) / CPR.  Relative to the piece, the lane's source offset
  // depends on n only through n % 4 for K (d = 128: rows 4n .. 4n + 3, whose
  // swizzle is the row mod 16; d = 64: through n % 2) and not at all for V
  // (its swizzle only sees the row mod 4, resp. mod 8 / 2).
  // The K offsets are recomputed at each use (a few integer operations on
  // the lane id) rather than held in four registers through the loop.
  auto k_lane_off = [&](int j) {
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int L = j * 64 + ln;
    const int r = L / C::CPR, x = L % C::CPR;
    return (uint32_t)(r * C::ROWB + ((x ^ C::kswz(r)) * 16) - j * 1024);
  };
  uint32_t vg;
  {
    const int r = lane / C::CPR, x = lane % C::CPR;
    vg = (uint32_t)(r * C::ROWB + ((x ^ C::vswz(r)) * 16));
  }
  const uint32_t lds_base = __builtin_amdgcn_readfirstlane(lds_addr(smem));
  // K A-operand reads: key row 32*kt + n32, logical chunk 2*ks + g (kt adds
  // 32 rows, which leaves both swizzles unchanged).
  int k_off[C::KS];
  {
    const int r = n32;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) k_off[ks] = r * C::ROWB + (((2 * ks + g) ^ C::kswz(r)) * 16);
  }
  // V^T A-operand transposing reads: lane l16 of a 16-lane group addresses
  // key row 16*j + 8*hi + 4*g + l16/4 and d columns 32*t + 16*h16 + 4*(l16%4);
  // the swizzle depends on the row only through bits the 16*j + 8*hi steps
  // (immediates) leave alone.
  int v_off[C::OT];
  {
    const int r = 4 * g + (l16 >> 2);
    const int byte_base = 32 * h16 + 8 * (l16 & 3);
#pragma unroll
    for (int t = 0; t < C::OT; ++t) {
      const int b = 64 * t + byte_base;
      v_off[t] = r * C::ROWB + ((((b >> 4) ^ C::vswz(r)) << 4) | (b & 15));
    }
  }

  const int quads_per_head = (Nc + kQuad - 1) / kQuad;
  const int64_t per_xcd = (total_quads + 7) / 8;
  const int xcd = blockIdx.x % 8;
  const int64_t lo = (int64_t)xcd * per_xcd;
  const int64_t end = lo + per_xcd < total_quads ? lo + per_xcd : total_quads;
  const int64_t stride = gridDim.x / 8;

  for (int64_t qid = lo + blockIdx.x / 8; qid < end; qid += stride) {
    const int64_t bh = qid / quads_per_head;
    const int cube0 = (int)(qid - bh * quads_per_head) * kQuad;
    const int64_t row0 = bh * Nc + cube0;
    const int64_t head_off = bh * (int64_t)Nc * kBlk * D;
    const int64_t kv_off = (bh / group) * (int64_t)Nc * kBlk * D;
    const char* k_head = reinterpret_cast<const char*>(k + kv_off);
    const char* v_head = reinterpret_cast<const char*>(v + kv_off);
    int t_init = 0, n_list = 0;
    const int S = build_quad<PAD, kThreads>(bs, sched, dsc, tlist, lut, valid, max_kv, Nc, row0, cube0, R, tmap, tid,
                                            lane, wave, t_init, n_list);

    // Q of this wave's cube as the B operand: query 32*qh + n32, d = 16*s + 8*g + 0..7
    const int my_cube = cube0 + cq;
    const bool my_valid = my_cube < Nc;
    bf16x8 qf[C::KS];
    if (my_valid) {
      const __bf16* qrow = q + head_off + (int64_t)(my_cube * kBlk + 32 * qh + n32) * D + 8 * g;
#pragma unroll
      for (int s = 0; s < C::KS; ++s) qf[s] = *reinterpret_cast<const bf16x8*>(qrow + 16 * s);
    } else {
#pragma unroll
      for (int s = 0; s < C::KS; ++s)
#pragma unroll
        for (int e = 0; e < 8; ++e) qf[s][e] = (__bf16)0.f;
    }


    // The tile list is read from registers: lane j of tw holds
    // tlist[twin + j].  The window only slides at a step barrier (by 32
    // entries, once the next tile is past its first half), so no LDS read
    // of it is outstanding between the products; at most R <= 15 list
    // entries are issued per step.
    // Loads: the wavefronts w = 0..3 (one per SIMD) move every tile, wave w
    // its pieces 4w .. 4w + 3 (d = 128; 2w .. 2w + 1 at d = 64) as one
    // group of pieces under one M0; waves 4..7 only compute, so on every
    // SIMD one wave keeps the matrix cores busy while the other's loads
    // drain through the address unit.
    const bool loader = wave < 4;
    int twin = 0;
    uint32_t tw = lane < n_list ? tlist[lane] : 0u;
    int i_next = 0;            // next tile to load (loaders)
    int slot_next = 0;         // its ring slot (i_next % R)
    auto issue_to = [&](int bound) {   // every tile with index < bound
      if (!loader) {
        i_next = bound;
        return;
      }
      for (; i_next < bound; ++i_next) {
        const uint32_t e = (uint32_t)__builtin_amdgcn_readlane((int)tw, i_next - twin);
        const bool isv = (e >> 16) & 1u;
        const int off = wave * C::PIECES * 256;   // pieces PIECES / 4 * wave ..
        const char* src = (isv ? v_head : k_head) + (int64_t)(e & 0xffffu) * C::TILE + off;
        const uint32_t m0 = lds_base + (uint32_t)slot_next * C::TILE + off;
        if constexpr (C::PIECES == 16) {
          if (isv) dma_quad(src, vg, vg, vg, vg, m0);
          else dma_quad(src, k_lane_off(0), k_lane_off(1), k_lane_off(2), k_lane_off(3), m0);
        } else {
          if (isv) dma_pair(src, vg, vg, m0);
          else dma_pair(src, k_lane_off(0), k_lane_off(1), m0);
        }
        if (++slot_next == R) slot_next = 0;
      }
    };
    // this wave's tiles with index in [lo, hi)
    auto mine = [&](int lo, int hi) { return loader ? hi - lo : 0; };
    wait_vmem<0>();     // the Q loads: every later wait counts tile pieces only
    issue_to(t_init);

    f32x16 o[C::OT];
#pragma unroll
    for (int t = 0; t < C::OT; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[t][r] = 0.f;
    float m_used = kNegBig;    // exponent offset (log2 units)
    f32x16 sc[2];              // scores of the previous step: keys 32*kt + 8*(r/4) + 4*g + r%4, query n32
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) sc[kt][r] = 0.f;
    float mx_prev = kNegBig;   // their row max (log2 units)

    uint32_t dx = 0, dw = 0;   // descriptor of the current step
    uint4 dnext = dsc[0];      // ... and of the next (read a step ahead)
    int issued = t_init;       // list index up to which tiles are issued
    auto step_barrier = [&](int p) {
      if (i_next - twin >= 32) {
        twin += 32;
        tw = twin + lane < n_list ? tlist[twin + lane] : 0u;
      }
      dx = (uint32_t)__builtin_amdgcn_readfirstlane((int)dnext.x);
      const int bound = __builtin_amdgcn_readfirstlane((int)dnext.y);
      const int landed = __builtin_amdgcn_readfirstlane((int)dnext.z);
      dw = (uint32_t)__builtin_amdgcn_readfirstlane((int)dnext.w);
      if (dw & 1u) {
        wait_vmem<0>();
        __syncthreads();
        issue_to(bound);
        wait_tiles<C::PIECES / 4, 0, kMaxRing>(mine(landed, bound));
        __syncthreads();
      } else {
        wait_tiles<C::PIECES / 4, 0, kMaxRing>(mine(landed, issued));
        __syncthreads();
        issue_to(bound);   // in one burst: the compute waves (4-7) run meanwhile
      }
      issued = bound;
    };

    // Exponentials of the previous step's score element e (0..31: tile
    // e / 16, register e % 16) into the P^T operand: k-step j of the PV
    // product covers keys 16j + 8*(e'/4) + 4*g + e'%4, i.e. registers
    // 8*(j%2) + e' of score tile j/2.  The row sum is kept in fp32 from the
    // unrounded probabilities (an accurate log-sum-exp), in two partial sums.
    float l_acc[2] = {0.f, 0.f};
    auto expo2 = [&](const f32x16 (&sc)[2], bf16x8 (&pb)[4], int e, float m_off) {   // elements e, e + 1
      const float p0 = __builtin_amdgcn_exp2f(fmaf(sc[e >> 4][e & 15], c_log2, -m_off));
      const float p1 = __builtin_amdgcn_exp2f(fmaf(sc[(e + 1) >> 4][(e + 1) & 15], c_log2, -m_off));
      pb[e >> 3][e & 7] = (__bf16)p0;
      pb[(e + 1) >> 3][(e + 1) & 7] = (__bf16)p1;
      l_acc[0] += p0;
      l_acc[1] += p1;
    };
    auto iter = [&](int p, const f32x16 (&sc)[2], f32x16 (&sn)[2]) {
      step_barrier(p);
      const uint32_t kslot = (dx >> (4 * cq)) & 15u;
      const uint32_t vslot = (dx >> (16 + 4 * cq)) & 15u;
      const bool has_c = kslot != 15u;   // this cube has a key tile in step p
      const bool has_p = vslot != 15u;   // ... had one in step p - 1
      // Lazy rescale for step p - 1 (o holds PV of steps <= p - 2).
      if (has_p && __ballot(mx_prev > m_used + kTau) != 0ull) {
        const float m_new = fmaxf(m_used, mx_prev);
        const float alpha = __builtin_amdgcn_exp2f(m_used - m_new);
        l_acc[0] *= alpha;
        l_acc[1] *= alpha;
#pragma unroll
        for (int t = 0; t < C::OT; ++t)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[t][r] *= alpha;
        m_used = m_new;
      }
      const float m_off = has_p ? m_used : INFINITY;

      // Work per MFMA slot.  QK(p): key rows 0-31 (tile 0) in the first
      // half, rows 32-63 (tile 1) in the second, K operands read PF MFMAs
      // ahead.  Exponentials of step p - 1: all of tile 0 in the first half,
      // half of tile 1 in the second, the rest beside the first PV products
      // (their operand is needed from PV product 3*OT on).  Row max of step
      // p: tile 0 beside the last QK products (once its chain has settled),
      // tile 1 beside the remaining PV products.  The products always run
      // (one straight code path keeps this interleaving); without a key tile
      // they read ring slot 0, which from barrier 0 on always holds key or
      // value rows of this head.  Such scores and their max are never used:
      // the next step has no value tile for this cube, so its offset is
      // +inf and P is exactly 0, and the PV products add nothing.  (This
      // holds for finite key and value inputs: a non-finite score, or 0
      // times a non-finite value read this way, would not give 0.)
      constexpr int NQK = 2 * C::KS;       // QK MFMAs per step
      constexpr int H = NQK / 2;           // per score tile
      // first QK slot of the tile-0 max (none with padded grids: their
      // masking comes after the QK products)
      constexpr int M0 = PAD ? NQK : H + (H >= 8 ? 2 : 1);
      constexpr int NPV = 4 * C::OT;       // PV MFMAs per step
      constexpr int Q4 = NPV / 4;          // PV slots before pb[1] is first used
      constexpr int PF = PAD ? 2 : 4;      // operand reads in flight (the masking needs registers)
      bf16x8 pb[4];
      float mx = kNegBig;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) sn[kt][r] = 0.f;
      {
        const char* kbase = smem + (has_c ? kslot : 0u) * C::TILE;
        auto ldk = [&](int i) {   // i: tile i / H, k-step i % H
          return *reinterpret_cast<const bf16x8*>(kbase + (i / H) * 32 * C::ROWB + k_off[i % H]);
        };
        bf16x8 kb[PF];
#pragma unroll
        for (int i = 0; i < PF; ++i) kb[i] = ldk(i);
#pragma unroll
        for (int i = 0; i < NQK; ++i) {
          sn[i / H] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kb[i % PF], qf[i % H], sn[i / H], 0, 0, 0);
          if (i + PF < NQK) kb[i % PF] = ldk(i + PF);
          // exponentials two at a time: pairs [a, b) of elements 2q, 2q + 1
          if (i < H) {
#pragma unroll
            for (int q2 = i * 8 / H; q2 < (i + 1) * 8 / H; ++q2) expo2(sc, pb, 2 * q2, m_off);
          } else {
#pragma unroll
            for (int q2 = 8 + (i - H) * 4 / H; q2 < 8 + (i - H + 1) * 4 / H; ++q2) expo2(sc, pb, 2 * q2, m_off);
            if (i >= M0) {
              constexpr int NS = NQK - M0;
#pragma unroll
              for (int r = (i - M0) * 16 / NS; r < (i - M0 + 1) * 16 / NS; ++r) mx = fmaxf(mx, sn[0][r]);
              asm volatile("" : "+v"(mx));   // keep these max operations in this slot
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      if (PAD && ((dw >> (1 + cq)) & 1u)) {
        // A key tile that reaches past the grid: its padded positions are
        // not keys (score -inf: nothing added to the row max or the sum).
        const int32_t cube = __builtin_amdgcn_readfirstlane((int32_t)step_cube(sched[p], cq));
        const uint64_t real = cube_mask(tmap, cube_at(tmap, cube));   // bit l: position l is a real token
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          const uint64_t m = real >> (32 * kt + 4 * g);
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (!((m >> (8 * (r >> 2) + (r & 3))) & 1ull)) sn[kt][r] = -INFINITY;
        }
      }
      dnext = dsc[p < S ? p + 1 : S];
      // PV(p-1), products ordered by k-step j (i = OT*j + t), V operands
      // read PF MFMAs ahead.
      {
        const char* vbase = smem + (has_p ? vslot : 0u) * C::TILE;
        auto ldv = [&](int i) {
          const int t = i % C::OT, j = i / C::OT;
          const i16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_i16x4*)(vbase + v_off[t] + (16 * j) * C::ROWB));
          const i16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_i16x4*)(vbase + v_off[t] + (16 * j + 8) * C::ROWB));
          return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
        };
        bf16x8 vb[PF];
#pragma unroll
        for (int i = 0; i < PF; ++i) vb[i] = ldv(i);
#pragma unroll
        for (int i = 0; i < NPV; ++i) {
          const int t = i % C::OT, j = i / C::OT;
          o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vb[i % PF], pb[j], o[t], 0, 0, 0);
          if (i + PF < NPV) vb[i % PF] = ldv(i + PF);
          if (i < Q4) {
#pragma unroll
            for (int q2 = 12 + i * 4 / Q4; q2 < 12 + (i + 1) * 4 / Q4; ++q2) expo2(sc, pb, 2 * q2, m_off);
          } else {
            // padded grids: both tiles' max here
            constexpr int NS = NPV - Q4, NM = PAD ? 32 : 16;
#pragma unroll
            for (int r = (i - Q4) * NM / NS; r < (i - Q4 + 1) * NM / NS; ++r) {
              const int e = PAD ? r : 16 + r;
              mx = fmaxf(mx, sn[e >> 4][e & 15]);
            }
            asm volatile("" : "+v"(mx));
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      mx_prev = pair_max(mx) * c_log2;
    };
    // A quad with no listed key cube at all has no step and loads nothing:
    // its outputs are 0 and its LSE -inf.
    f32x16 sc2[2];
    for (int p = 0; S > 0 && p <= S; p += 2) {
      iter(p, sc, sc2);
      if (p + 1 > S) break;
      iter(p + 1, sc2, sc);
    }
    __syncthreads();   // every wave is done with the ring before it is reused

    // ---- normalise, stage, combine, store ----
    const float l_row = pair_sum(l_acc[0] + l_acc[1]);
    const float inv = l_row > 0.f ? 1.f / l_row : 0.f;
    float* ost = reinterpret_cast<float*>(smem + cq * C::OST);   // [64][OSTR]
    {
      float* orow = ost + (32 * qh + n32) * C::OSTR;
#pragma unroll
      for (int t = 0; t < C::OT; ++t)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          float4 w;
          w.x = o[t][4 * rq + 0] * inv;
          w.y = o[t][4 * rq + 1] * inv;
          w.z = o[t][4 * rq + 2] * inv;
          w.w = o[t][4 * rq + 3] * inv;
          *reinterpret_cast<float4*>(orow + 32 * t + 8 * rq + 4 * g) = w;   // d = 32t + 8rq + 4g + 0..3
        }
      const int32_t my_tok = 32 * qh + n32;
      const CubeAt mq = tmap.on && my_valid ? cube_at(tmap, my_cube) : CubeAt{0, 0, 0, true};
      if (lse != nullptr && g == 0 && my_valid && mq.ok && (!PAD || !tmap.on || token_real(tmap, mq, my_tok))) {
        const float val = (l_row > 0.f) ? (m_used + __log2f(l_row)) * 0.69314718055994531f : -INFINITY;
        lse[bh * (int64_t)(tmap.on ? tmap.N : tmap.Np) + token_pos(tmap, my_cube, mq, my_tok)] = val;
      }
    }
    __syncthreads();
    // 4 cubes x 64 rows x CPR chunks, 16 bytes each, over all 512 threads
    for (int cidx = tid; cidx < kQuad * kBlk * C::CPR; cidx += kThreads) {
      const int cc = cidx / (kBlk * C::CPR);
      const int rem = cidx - cc * kBlk * C::CPR;
      const int row = rem / C::CPR, col = rem % C::CPR;
      const int cube = cube0 + cc;
      if (cube >= Nc) continue;
      const CubeAt cqa = tmap.on ? cube_at(tmap, cube) : CubeAt{0, 0, 0, true};
      if (!cqa.ok) continue;
      if (PAD && tmap.on && !token_real(tmap, cqa, row)) continue;   // padding: no raster row
      const int64_t gidx = token_elem(tmap, bh, cube, cqa, row, D) + col * 8;
      const float* srow = reinterpret_cast<const float*>(smem + cc * C::OST) + row * C::OSTR + col * 8;
      float val[8];
      const float4 v0 = *reinterpret_cast<const float4*>(srow);
      const float4 v1 = *reinterpret_cast<const float4*>(srow + 4);
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
        const float* ocrow = oc + (row0 + cc) * (int64_t)D + col * 8;
        const float4 c0 = *reinterpret_cast<const float4*>(ocrow);
        const float4 c1 = *reinterpret_cast<const float4*>(ocrow + 4);
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
    __syncthreads();   // staging reads done before the next quad reuses LDS
  }
}

// Per-device launch state: the CU count and the dynamic-LDS limit already
// granted to each instantiation.
struct QuadDevState {
  int cus = 0;
  int lds_granted[4] = {0, 0, 0, 0};
};

constexpr int kLdsMax = 160 * 1024;
std::mutex quad_state_mutex;

// Ring slots for this problem: as many whole tiles as fit beside the
// quad's metadata, at most kMaxRing; 0 when fewer than kMinRing fit or the
// build scratch does not fit in the ring.
template <int D>
int quad_ring(const Geom& g, int max_kv) {
  using C = QCfg<D>;
  if (g.Nc < 1 || g.Nc > 0xfffe || max_kv < 1) return 0;
  const QuadMeta m = quad_meta(g.Nc, max_kv, 0);
  if (m.bytes >= (size_t)kLdsMax) return 0;
  int R = (int)(((size_t)kLdsMax - m.bytes) / C::TILE);
  if (R > kMaxRing) R = kMaxRing;
  if (R < kMinRing) return 0;
  if (build_scratch_bytes(g.Nc, m.s_max) > (size_t)R * C::TILE) return 0;
  return R;
}

template <int D, bool PAD>
hipError_t launch_quad(const Geom& g, const void* q, const void* k, const void* v, const int32_t* lut,
                       const int32_t* valid, int max_kv, const float* oc, const void* gate_c, const void* gate_f,
                       void* out, float* lse, hipStream_t s, const TokenMap& tmap, int slot) {
  using C = QCfg<D>;
  static QuadDevState dev_state[64];
  const int R = quad_ring<D>(g, max_kv);
  if (R == 0) return hipErrorInvalidValue;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  QuadDevState& st = dev_state[dev];
  auto kern = sparse_attn_fwd_quad_kernel<D, PAD>;
  size_t lds = (size_t)R * C::TILE + quad_meta(g.Nc, max_kv, 0).bytes;
  if (lds < (size_t)kQuad * C::OST) lds = (size_t)kQuad * C::OST;
  if (lds > (size_t)kLdsMax) return hipErrorInvalidValue;
  int cus = 0;
  {
    std::lock_guard<std::mutex> lock(quad_state_mutex);
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
  const int64_t total_quads = g.BH * ((g.Nc + kQuad - 1) / kQuad);
  int64_t grid = ((int64_t)cus + 7) / 8 * 8;
  const int64_t need = (total_quads + 7) / 8 * 8;
  if (grid > need) grid = need;
  const float c_log2 = 1.4426950408889634f / sqrtf((float)D);
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kThreads), lds, s, (const __bf16*)q, (const __bf16*)k,
                     (const __bf16*)v, lut, valid, max_kv, oc, (const __bf16*)gate_c, (const __bf16*)gate_f,
                     (__bf16*)out, lse, (int)g.Nc, total_quads, c_log2, tmap, g.group, R);
  return hipGetLastError();
}

}  // namespace

bool sparse_attn_fwd_quad_fits(const Geom& g, int max_kv) {
  if (g.D != g.Dv) return false;
  if (g.D == 128) return quad_ring<128>(g, max_kv) != 0;
  if (g.D == 64) return quad_ring<64>(g, max_kv) != 0;
  return false;
}

hipError_t launch_sparse_attn_fwd_quad(const Geom& g, const void* q, const void* k, const void* v,
                                       const int32_t* lut, const int32_t* valid, int max_kv, const float* oc,
                                       const void* gate_c, const void* gate_f, void* out, float* lse,
                                       int out_order, hipStream_t s) {
  const TokenMap m = make_token_map(g, out_order);
  if (g.D == 128 && g.padded) return launch_quad<128, true>(g, q, k, v, lut, valid, max_kv, oc, gate_c, gate_f, out, lse, s, m, 0);
  if (g.D == 128) return launch_quad<128, false>(g, q, k, v, lut, valid, max_kv, oc, gate_c, gate_f, out, lse, s, m, 1);
  if (g.D == 64 && g.padded) return launch_quad<64, true>(g, q, k, v, lut, valid, max_kv, oc, gate_c, gate_f, out, lse, s, m, 2);
  if (g.D == 64) return launch_quad<64, false>(g, q, k, v, lut, valid, max_kv, oc, gate_c, gate_f, out, lse, s, m, 3);
  return hipErrorInvalidValue;
}

}  // namespace vsa
