// Coarse stage: cube-to-cube scores, Top-K key-cube selection (the LUT) and
// the coarse attention output O_c.
//
// "VSA: Accelerating Video Diffusion Inference with Sparse Attention on AMD
// GPUs", §Two-Stage Architecture (Stage 1: coarse scores, Top-K cubes per
// query cube, coarse output kept for global context), §Block-Sparse Encoding
// (index list + valid count) and §Generating Sparsity Patterns (scores are
// the pooled-query / pooled-key inner products, Top-K per query row);
// "VSA: Faster Video Diffusion with Trainable Sparse Attention", Abstract.
//
// One workgroup = R query cubes of one (batch, head): R = 8 with eight
// wavefronts, or R = 4 with four when eight score rows do not fit in LDS.  Key and value cubes are staged
// through LDS 64 at a time with coalesced 16-byte loads.
//   phase 1  raw scores s[r][j] = <qc[i0+r], kc[j]> in float32, a sequential
//            FMA chain over d per score; thread (key j, wave w) forms the
//            wave's rows of column j, the query values coming through the
//            scalar cache.  Rows are kept in LDS;
//   phase 2  one wavefront per row: Top-K by radix select over the 32-bit
//            order-preserving key of each score, held in registers, one bit
//            per pass, counting with wavefront ballots; the selected indices
//            are emitted in ascending order through a ballot prefix count.
//            Ties at the threshold go to the lower index.  Then the row
//            softmax p_j = exp(scale*(s_j - max)), summed in a fixed order;
//   phase 3  O_c[r] = sum_j p_j * vc[j] / sum_j p_j; thread (4 columns of d,
//            row group) reads four probabilities and four value rows per
//            16-byte LDS read; with few rows the key range is split across
//            row groups and the partial sums are added in a fixed order.
// The scale 1/sqrt(d) > 0 does not change the ranking, so ranking uses the
// raw scores.
#include <mutex>

#include "vsa_internal.h"

namespace vsa {
namespace {

constexpr int kChunk = 64;   // key / value cubes staged per LDS pass

// Order-preserving map float -> uint32 (larger float -> larger key).  -0 is
// folded onto +0 so that equal scores compare equal.
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t b = __float_as_uint(f);
  if (b == 0x80000000u) b = 0u;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// The score of a key (inverse of order_key; -0 comes back as +0).
__device__ __forceinline__ float key_score(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

__device__ __forceinline__ int popc64(uint64_t m) { return __popcll(m); }

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Row stride of the score rows in LDS: a multiple of 4 floats so that four
// consecutive probabilities are one aligned 16-byte read.
__host__ __device__ inline int padded_cols(int Nc) { return (Nc + 3) & ~3; }

// Cubes [c0, c0 + kChunk) of one (batch, head) pass through registers
// (loaded one chunk ahead, so the global latency overlaps the previous
// chunk's arithmetic) into LDS rows of D + 4 floats; the pad makes a 16-lane
// group's row reads hit distinct banks.  Cubes past Nc read as zero.
template <int D, int kThreads>
struct ChunkStage {
  static constexpr int C4 = D / 4;
  static constexpr int PER = kChunk * C4 / kThreads;   // 16-byte pieces per thread
  float4 v[PER];
  __device__ __forceinline__ void load(const float* src, int c0, int Nc, int tid) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = tid + i * kThreads;
      const int row = e / C4, c4 = e - row * C4;
      v[i] = c0 + row < Nc ? reinterpret_cast<const float4*>(src)[(int64_t)(c0 + row) * C4 + c4]
                           : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
  __device__ __forceinline__ void store(float* chunk, int tid) const {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = tid + i * kThreads;
      const int row = e / C4, c4 = e - row * C4;
      *reinterpret_cast<float4*>(chunk + row * (D + 4) + 4 * c4) = v[i];
    }
  }
};

// Top-K of one score row (one wavefront): the selected cube indices in
// ascending order to out_idx and K to *valid_row; with want_p the row is
// replaced by its softmax numerators p_j = exp(scale * (s_j - max)) (pad
// columns 0) and 1 / sum_j p_j goes to *inv_sum_r.
template <int NS>
__device__ __forceinline__ void select_row(float* sr, int Nc, int NcP, int top_k, int32_t* out_idx,
                                           int32_t* valid_row, bool want_p, float scale, float* inv_sum_r,
                                           int lane) {
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  // Keys of this row, slot s = cube s*64 + lane; 0 (below every candidate
  // threshold, which always has a bit set) past Nc.
  uint32_t key[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int j = s * 64 + lane;
    key[s] = j < Nc ? order_key(sr[j]) : 0u;
  }
  // K-th largest key: build the threshold from the top bit down.  Each pass
  // counts the keys >= the candidate: every lane counts its own slots on the
  // vector ALU, and the wave total comes from one ballot per bit of those
  // counts (the scalar unit, shared by the CU's four SIMDs, does a few
  // popcounts per pass instead of one per slot).  Once exactly top_k keys
  // are >= the threshold, they are the selection whatever the lower bits,
  // and no key equals a lower candidate it would still set: stop there.
  uint32_t thr = 0u;
  // exact: exactly top_k keys are >= thr, so they are the selection and no
  // key equal to thr is left out (always so when every cube is selected)
  bool exact = top_k >= Nc;
  if (top_k < Nc) {
    constexpr int NB = NS >= 64 ? 7 : NS >= 32 ? 6 : NS >= 16 ? 5 : 4;   // bits of a count 0..NS
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t cand = thr | (1u << bit);
      uint32_t mine = 0;
#pragma unroll
      for (int s = 0; s < NS; ++s) mine += key[s] >= cand ? 1u : 0u;
      int cnt = 0;
#pragma unroll
      for (int b = 0; b < NB; ++b) cnt += popc64(__ballot((mine >> b) & 1u)) << b;
      if (cnt >= top_k) {
        thr = cand;
        if (cnt == top_k) {
          exact = true;
          break;
        }
      }
    }
  }
  if (exact) {
    // the keys >= thr, in ascending cube order
    int sel_before = 0;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int j = s * 64 + lane;
      const bool take = j < Nc && key[s] >= thr;
      const uint64_t tm = __ballot(take);
      if (take) out_idx[sel_before + popc64(tm & lt_mask)] = j;
      sel_before += popc64(tm);
    }
  } else {
    // ties at thr: all keys above it, then the lowest-index keys equal to it
    int gt = 0;
#pragma unroll
    for (int s = 0; s < NS; ++s) gt += popc64(__ballot(s * 64 + lane < Nc && key[s] > thr));
    const int need = top_k - gt;   // >= 1 entries equal to thr are taken
    int eq_before = 0, sel_before = 0;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int j = s * 64 + lane;
      const bool in = j < Nc;
      const bool eq = in && key[s] == thr;
      const uint64_t eqm = __ballot(eq);
      const int eq_rank = eq_before + popc64(eqm & lt_mask);
      const bool take = in && (key[s] > thr || (eq && eq_rank < need));
      const uint64_t tm = __ballot(take);
      if (take) out_idx[sel_before + popc64(tm & lt_mask)] = j;
      sel_before += popc64(tm);
      eq_before += popc64(eqm);
    }
  }
  if (lane == 0) *valid_row = top_k;

  if (want_p) {
    // the scores come back from the keys held in registers (order_key is
    // one-to-one except that -0 reads back as +0, which gives the same
    // weights): the row max is the largest key, and the row is read from
    // LDS only once, above
    uint32_t kmax = 0u;
#pragma unroll
    for (int s = 0; s < NS; ++s) kmax = max(kmax, key[s]);   // slots past Nc hold 0
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, o, 64));
    const float m = key_score(kmax);
    float sum = 0.f;
    // exp(scale * (s - m)) as the hardware exp2 of the scaled difference:
    // about 4e-6 relative for the differences of these rows, far inside
    // the coarse output's tolerance, and several times cheaper than expf
    const float scale2 = scale * 1.4426950408889634f;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int j = s * 64 + lane;
      if (j < NcP) {
        const float p = j < Nc ? __builtin_amdgcn_exp2f((key_score(key[s]) - m) * scale2) : 0.f;
        sr[j] = p;   // the pad columns hold 0
        sum += p;
      }
    }
    sum = wave_sum(sum);
    if (lane == 0) *inv_sum_r = 1.f / sum;
  }
}

// DQ: query/key head size (scores); DV: value head size (O_c).
template <int DQ, int DV, int R, int NS, int kThreads>
__global__ __launch_bounds__(kThreads) void coarse_topk_kernel(
    const float* __restrict__ qc, const float* __restrict__ kc, const float* __restrict__ vc,
    int32_t* __restrict__ lut, int32_t* __restrict__ valid, float* __restrict__ oc, int Nc, int top_k,
    int tiles_per_head, float scale, int group) {
  constexpr int kWaves = kThreads / 64;
  static_assert(R % kWaves == 0, "rows per workgroup");
  extern __shared__ float smem[];
  const int NcP = padded_cols(Nc);
  constexpr int DM = DQ > DV ? DQ : DV;
  float* chunk = smem;                       // [kChunk][DQ + 4] keys, then [kChunk][DV + 4] values
  float* srow = chunk + kChunk * (DM + 4);   // [R][NcP]
  float* inv_sum = srow + (int64_t)R * NcP;  // [R]

  const int64_t bh = blockIdx.x / tiles_per_head;
  const int i0 = (int)(blockIdx.x - bh * tiles_per_head) * R;
  const int rows = min(R, Nc - i0);
  const int64_t kvh = bh / group;   // key/value head of this query head
  const float* kh = kc + kvh * (int64_t)Nc * DQ;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // phase 1: raw scores.  A wave's query rows are uniform across its lanes,
  // so they are read straight from global memory through the scalar cache
  // (rows past the last cube repeat it; their scores are never used).
  constexpr int RW = R / kWaves;   // rows per thread
  const float* qrow[RW];
#pragma unroll
  for (int u = 0; u < RW; ++u)
    qrow[u] = qc + (bh * Nc + min(i0 + wave + kWaves * u, Nc - 1)) * (int64_t)DQ;
  ChunkStage<DQ, kThreads> st;
  st.load(kh, 0, Nc, tid);
  for (int c0 = 0; c0 < Nc; c0 += kChunk) {
    __syncthreads();   // previous chunk fully read
    st.store(chunk, tid);
    __syncthreads();
    if (c0 + kChunk < Nc) st.load(kh, c0 + kChunk, Nc, tid);
    float acc[RW];
#pragma unroll
    for (int u = 0; u < RW; ++u) acc[u] = 0.f;
    const float* kr = chunk + lane * (DQ + 4);
#pragma unroll 8
    for (int d4 = 0; d4 < DQ / 4; ++d4) {
      const float4 kv = *reinterpret_cast<const float4*>(kr + 4 * d4);
#pragma unroll
      for (int u = 0; u < RW; ++u) {
        const float4 qv = *reinterpret_cast<const float4*>(qrow[u] + 4 * d4);
        acc[u] = fmaf(qv.x, kv.x, acc[u]);
        acc[u] = fmaf(qv.y, kv.y, acc[u]);
        acc[u] = fmaf(qv.z, kv.z, acc[u]);
        acc[u] = fmaf(qv.w, kv.w, acc[u]);
      }
    }
    if (c0 + lane < Nc) {
#pragma unroll
      for (int u = 0; u < RW; ++u) srow[(int64_t)(wave + kWaves * u) * NcP + c0 + lane] = acc[u];
    }
  }
  // The first value chunk is in flight during the selection.
  const float* vh = vc + kvh * (int64_t)Nc * DV;
  ChunkStage<DV, kThreads> sv;
  if (oc != nullptr) sv.load(vh, 0, Nc, tid);
  __syncthreads();

  // phase 2: per-row Top-K and softmax weights, one wavefront per row
  for (int r = wave; r < rows; r += kWaves)
    select_row<NS>(srow + (int64_t)r * NcP, Nc, NcP, top_k, lut + (bh * Nc + i0 + r) * top_k,
                   valid + bh * Nc + i0 + r, oc != nullptr, scale, inv_sum + r, lane);
  if (oc == nullptr) return;

  // phase 3: O_c rows
  constexpr int C4 = DV / 4;                    // 16-byte column groups
  constexpr int NRG = kThreads / C4;            // row groups
  constexpr int RPT = R >= NRG ? R / NRG : 1;   // rows per thread
  constexpr int KS = R >= NRG ? 1 : NRG / R;    // key splits
  static_assert(RPT * NRG == R || KS * R == NRG, "phase 3 mapping");
  const int c4 = tid % C4;
  const int rg = tid / C4;
  const int r_first = KS == 1 ? rg : rg % R;
  const int ks = KS == 1 ? 0 : rg / R;
  float4 acc[RPT];
#pragma unroll
  for (int u = 0; u < RPT; ++u) acc[u] = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int c0 = 0; c0 < Nc; c0 += kChunk) {
    __syncthreads();   // phase 2 done / previous chunk fully read
    sv.store(chunk, tid);
    __syncthreads();
    if (c0 + kChunk < Nc) sv.load(vh, c0 + kChunk, Nc, tid);
    const int jend = min(kChunk, NcP - c0);   // multiple of 4; pad columns carry p = 0
    for (int j = 4 * ks; j < jend; j += 4 * KS) {
      const float4 v0 = *reinterpret_cast<const float4*>(chunk + (j + 0) * (DV + 4) + 4 * c4);
      const float4 v1 = *reinterpret_cast<const float4*>(chunk + (j + 1) * (DV + 4) + 4 * c4);
      const float4 v2 = *reinterpret_cast<const float4*>(chunk + (j + 2) * (DV + 4) + 4 * c4);
      const float4 v3 = *reinterpret_cast<const float4*>(chunk + (j + 3) * (DV + 4) + 4 * c4);
#pragma unroll
      for (int u = 0; u < RPT; ++u) {
        const int r = r_first + NRG * u;
        const float4 p = *reinterpret_cast<const float4*>(srow + (int64_t)r * NcP + c0 + j);
        acc[u].x = fmaf(p.x, v0.x, acc[u].x); acc[u].y = fmaf(p.x, v0.y, acc[u].y);
        acc[u].z = fmaf(p.x, v0.z, acc[u].z); acc[u].w = fmaf(p.x, v0.w, acc[u].w);
        acc[u].x = fmaf(p.y, v1.x, acc[u].x); acc[u].y = fmaf(p.y, v1.y, acc[u].y);
        acc[u].z = fmaf(p.y, v1.z, acc[u].z); acc[u].w = fmaf(p.y, v1.w, acc[u].w);
        acc[u].x = fmaf(p.z, v2.x, acc[u].x); acc[u].y = fmaf(p.z, v2.y, acc[u].y);
        acc[u].z = fmaf(p.z, v2.z, acc[u].z); acc[u].w = fmaf(p.z, v2.w, acc[u].w);
        acc[u].x = fmaf(p.w, v3.x, acc[u].x); acc[u].y = fmaf(p.w, v3.y, acc[u].y);
        acc[u].z = fmaf(p.w, v3.z, acc[u].z); acc[u].w = fmaf(p.w, v3.w, acc[u].w);
      }
    }
  }
  if (KS > 1) {
    // Partial sums of the key splits, added in split order.
    __syncthreads();
    float4* part = reinterpret_cast<float4*>(chunk);   // [KS][R][C4]
    part[(ks * R + r_first) * C4 + c4] = acc[0];
    __syncthreads();
    if (ks == 0) {
      float4 t = part[r_first * C4 + c4];
      for (int k2 = 1; k2 < KS; ++k2) {
        const float4 o = part[(k2 * R + r_first) * C4 + c4];
        t.x += o.x; t.y += o.y; t.z += o.z; t.w += o.w;
      }
      acc[0] = t;
    }
  }
  if (ks != 0) return;
#pragma unroll
  for (int u = 0; u < RPT; ++u) {
    const int r = r_first + NRG * u;
    if (r < rows) {
      const float is = inv_sum[r];
      const float4 a = acc[u];
      reinterpret_cast<float4*>(oc + (bh * Nc + i0 + r) * DV)[c4] =
          make_float4(a.x * is, a.y * is, a.z * is, a.w * is);
    }
  }
}

// ---- sixteen query cubes per workgroup, products on the matrix cores ----
// Used whenever sixteen score rows fit in LDS.  Both products run as
// v_mfma_f32_16x16x4_f32 (float32 operands and accumulation, so the scores
// keep the precision the ranking needs).  Each wavefront loads its own B
// operands from global memory into registers, one block ahead, so neither
// product stages data through LDS or waits at a barrier:
//   phase 1  S[i][j] = sum_d Q[i][d] K[j][d] for the 16 query cubes i of the
//            workgroup; wave w owns keys 16w .. 16w + 15 of every block of
//            128.  Product (s, e) maps the k index l/16 of lane l to
//            d = 16s + 4(l/16) + e: A = Q[l % 16][d] from registers, B =
//            K[key l % 16][d]; one 16-byte load feeds four products, and the
//            four lane groups of a key read 64 contiguous bytes.
//   phase 3  O_c[i][:] = sum_j P[i][j] V[j][:]; wave w owns one 64-column
//            group g of O_c (d_v / 64 groups) and every (8 / groups)-th
//            64-key chunk.  Slice t of chunk c maps lane group l/16 to key
//            64c + 16(l/16) + t: A = P[l % 16][key], four slices per 16-byte
//            LDS read; one 16-byte load of V[key][64g + 4(l % 16) ...] holds
//            the B operands of four products, one per column tile u, whose
//            column l % 16 stands for column 64g + 4(l % 16) + u.  The key
//            splits' partial sums are added in split order at the end.
// Phase 2 (Top-K and softmax weights) is the same as in the kernel above,
// two rows per wavefront.
typedef float floatx4 __attribute__((ext_vector_type(4)));   // MFMA 16x16 accumulator
constexpr int kMR = 16;                 // query cubes per workgroup
constexpr int kMThreads = 512;          // 8 wavefronts
constexpr int kMKeys = 128;             // keys per phase-1 block (16 per wave)
constexpr int kMPart = 8 * kMR * 64;    // floats of the phase-3 partial sums (8 waves x 16 rows x 64 columns)
constexpr size_t kCoarseLdsMax = 160 * 1024;

// LDS floats of the sixteen-row kernel at score-row stride sp: the score
// rows (which hold the phase-3 partial sums afterwards), then 1/sum per row.
__host__ __device__ inline int mfma_lds_floats(int sp) { return (kMR * sp > kMPart ? kMR * sp : kMPart) + kMR; }

// Row stride of the sixteen score rows: the padded row rounded up to 4 more
// than a multiple of 64 floats, where that still fits in LDS.  Phase 3 reads
// four consecutive probabilities of sixteen different rows in one 16-byte
// access per lane; at a stride that is a multiple of 64 floats all sixteen
// fall in the same four banks.  The largest cube counts keep the plain
// padded stride (same results, slower reads).
__host__ __device__ inline int mfma_row_stride(int Nc) {
  const int p = padded_cols(Nc);
  const int q = p + ((68 - p % 64) % 64);
  return sizeof(float) * (size_t)mfma_lds_floats(q) <= kCoarseLdsMax ? q : p;
}

static size_t coarse_mfma_lds_bytes(int Nc) { return sizeof(float) * (size_t)mfma_lds_floats(mfma_row_stride(Nc)); }

template <int DQ, int DV, int NS>
__global__ __launch_bounds__(kMThreads) void coarse_topk_mfma_kernel(
    const float* __restrict__ qc, const float* __restrict__ kc, const float* __restrict__ vc,
    int32_t* __restrict__ lut, int32_t* __restrict__ valid, float* __restrict__ oc, int Nc, int top_k,
    int tiles_per_head, float scale, int group) {
  constexpr int kWaves = kMThreads / 64;
  constexpr int QS = DQ / 16;        // phase-1 steps of four products
  constexpr int NG = DV / 64;        // phase-3 column groups
  constexpr int KS = kWaves / NG;    // phase-3 key splits
  extern __shared__ float smem[];
  const int NcP = padded_cols(Nc);
  const int SP = mfma_row_stride(Nc);
  float* srow = smem;                                                // [16][SP]
  float* inv_sum = smem + (kMR * SP > kMPart ? kMR * SP : kMPart);   // [16]

  const int64_t bh = blockIdx.x / tiles_per_head;
  const int i0 = (int)(blockIdx.x - bh * tiles_per_head) * kMR;
  const int rows = min(kMR, Nc - i0);
  const int64_t kvh = bh / group;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, kq = lane >> 4;

  // ---- phase 1: scores ----
  float4 qv[QS];   // Q[i0 + l16][16s + 4kq ...]; rows past the last cube repeat it
  {
    const float* qr = qc + (bh * Nc + min(i0 + l16, Nc - 1)) * (int64_t)DQ + 4 * kq;
#pragma unroll
    for (int s = 0; s < QS; ++s) qv[s] = *reinterpret_cast<const float4*>(qr + 16 * s);
  }
  // this lane's key row in the block at c0 (keys past the last cube repeat
  // it; their scores are not stored)
  const float* kh = kc + kvh * (int64_t)Nc * DQ + 4 * kq;
  auto kload = [&](float4 (&dst)[QS], int c0) {
    const float* kr = kh + (int64_t)min(c0 + 16 * wave + l16, Nc - 1) * DQ;
#pragma unroll
    for (int s = 0; s < QS; ++s) dst[s] = *reinterpret_cast<const float4*>(kr + 16 * s);
  };
  auto score_block = [&](const float4 (&cur)[QS], float4 (&nxt)[QS], int c0) {
    if (c0 + kMKeys < Nc) kload(nxt, c0 + kMKeys);
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < QS; ++s) {
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(qv[s].x, cur[s].x, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(qv[s].y, cur[s].y, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(qv[s].z, cur[s].z, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(qv[s].w, cur[s].w, acc, 0, 0, 0);
    }
    // D[i][j]: rows 4*kq + r, key c0 + 16*wave + l16
    const int j = c0 + 16 * wave + l16;
    if (j < Nc) {
#pragma unroll
      for (int r = 0; r < 4; ++r) srow[(4 * kq + r) * SP + j] = acc[r];
    }
  };
  {
    float4 k0[QS], k1[QS];
    kload(k0, 0);
    for (int c0 = 0; c0 < Nc; c0 += 2 * kMKeys) {
      score_block(k0, k1, c0);
      if (c0 + kMKeys < Nc) score_block(k1, k0, c0 + kMKeys);
    }
  }

  // phase 3's value rows: slices t0 .. t0 + 7 of chunk c (key 64c + 16kq + t;
  // keys past the last cube repeat it, with P = 0 there)
  const int nchunks = (Nc + 63) / 64;
  const int g = wave % NG, ks = wave / NG;
  const float* vh = vc + kvh * (int64_t)Nc * DV + 64 * g + 4 * l16;
  auto vload = [&](float4 (&dst)[8], int c, int t0) {
#pragma unroll
    for (int t = 0; t < 8; ++t)
      dst[t] = *reinterpret_cast<const float4*>(vh + (int64_t)min(64 * c + 16 * kq + t0 + t, Nc - 1) * DV);
  };
  float4 v0[8], v1[8];
  if (oc != nullptr && ks < nchunks) vload(v0, ks, 0);   // in flight during phase 2
  __syncthreads();

  // ---- phase 2 ----
  for (int r = wave; r < rows; r += kWaves)
    select_row<NS>(srow + (int64_t)r * SP, Nc, NcP, top_k, lut + (bh * Nc + i0 + r) * top_k,
                   valid + bh * Nc + i0 + r, oc != nullptr, scale, inv_sum + r, lane);
  if (oc == nullptr) return;
  __syncthreads();   // every P row and 1/sum written

  // ---- phase 3: O_c ----
  floatx4 o[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) o[u] = floatx4{0.f, 0.f, 0.f, 0.f};
  auto oc_half = [&](const float4 (&cur)[8], float4 (&nxt)[8], int c, int t0) {
    const int nc = t0 == 0 ? c : c + KS, nt = t0 == 0 ? 8 : 0;
    if (nc < nchunks) vload(nxt, nc, nt);
    // P past the padded row is not read (zero A value); pad columns hold 0
    const int kb = 64 * c + 16 * kq + t0;
    const float* pr = srow + (int64_t)l16 * SP + kb;
    const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
    const float4 p0 = kb < NcP ? *reinterpret_cast<const float4*>(pr) : z;
    const float4 p1 = kb + 4 < NcP ? *reinterpret_cast<const float4*>(pr + 4) : z;
    const float pv[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      o[0] = __builtin_amdgcn_mfma_f32_16x16x4f32(pv[t], cur[t].x, o[0], 0, 0, 0);
      o[1] = __builtin_amdgcn_mfma_f32_16x16x4f32(pv[t], cur[t].y, o[1], 0, 0, 0);
      o[2] = __builtin_amdgcn_mfma_f32_16x16x4f32(pv[t], cur[t].z, o[2], 0, 0, 0);
      o[3] = __builtin_amdgcn_mfma_f32_16x16x4f32(pv[t], cur[t].w, o[3], 0, 0, 0);
    }
  };
  for (int c = ks; c < nchunks; c += KS) {
    oc_half(v0, v1, c, 0);
    oc_half(v1, v0, c, 8);
  }
  // partial sums [split][row][column] over the score rows, added in split order
  __syncthreads();   // every wave done reading P
  float* part = smem;
#pragma unroll
  for (int r = 0; r < 4; ++r)
    *reinterpret_cast<float4*>(part + (ks * kMR + 4 * kq + r) * DV + 64 * g + 4 * l16) =
        make_float4(o[0][r], o[1][r], o[2][r], o[3][r]);
  __syncthreads();
  for (int e = tid; e < kMR * DV / 4; e += kMThreads) {
    const int i = e / (DV / 4), c4 = e - i * (DV / 4);
    if (i < rows) {
      float4 t = *reinterpret_cast<const float4*>(part + i * DV + 4 * c4);
#pragma unroll
      for (int k2 = 1; k2 < KS; ++k2) {
        const float4 u = *reinterpret_cast<const float4*>(part + (k2 * kMR + i) * DV + 4 * c4);
        t.x += u.x; t.y += u.y; t.z += u.z; t.w += u.w;
      }
      const float is = inv_sum[i];
      reinterpret_cast<float4*>(oc + (bh * Nc + i0 + i) * (int64_t)DV)[c4] =
          make_float4(t.x * is, t.y * is, t.z * is, t.w * is);
    }
  }
}

}  // namespace

static size_t coarse_lds_bytes(int R, int Nc, int D) {   // D: the wider of the two head sizes
  return sizeof(float) * ((size_t)kChunk * (D + 4) + (size_t)R * padded_cols(Nc) + R);
}

template <int DQ, int DV, int R, int NS, int T>
static hipError_t launch_rns(const Geom& g, int top_k, const float* qc, const float* kc, const float* vc,
                             int32_t* lut, int32_t* valid, float* oc, hipStream_t s) {
  const int Nc = (int)g.Nc;
  const int tiles = (Nc + R - 1) / R;
  const int64_t blocks = g.BH * tiles;
  const size_t lds = coarse_lds_bytes(R, Nc, DQ > DV ? DQ : DV);
  const float scale = 1.0f / sqrtf((float)DQ);
  auto k = coarse_topk_kernel<DQ, DV, R, NS, T>;
  if (lds > 65536) {
    // the granted size only grows, under a lock: host threads may launch concurrently
    static std::mutex mu;
    static int granted[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (granted[dev] < (int)lds) {
      const hipError_t e = hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return e;
      granted[dev] = (int)lds;
    }
  }
  hipLaunchKernelGGL(k, dim3((unsigned)blocks), dim3(T), lds, s, qc, kc, vc, lut, valid, oc, Nc, top_k,
                     tiles, scale, g.group);
  return hipGetLastError();
}

template <int DQ, int DV, int R, int T>
static hipError_t launch_r(const Geom& g, int top_k, const float* qc, const float* kc, const float* vc,
                           int32_t* lut, int32_t* valid, float* oc, hipStream_t s) {
  const int slots = (int)((g.Nc + 63) / 64);
  if (slots <= 8) return launch_rns<DQ, DV, R, 8, T>(g, top_k, qc, kc, vc, lut, valid, oc, s);
  if (slots <= 16) return launch_rns<DQ, DV, R, 16, T>(g, top_k, qc, kc, vc, lut, valid, oc, s);
  if (slots <= 32) return launch_rns<DQ, DV, R, 32, T>(g, top_k, qc, kc, vc, lut, valid, oc, s);
  return launch_rns<DQ, DV, R, 64, T>(g, top_k, qc, kc, vc, lut, valid, oc, s);
}

template <int DQ, int DV, int NS>
static hipError_t launch_mfma_ns(const Geom& g, int top_k, const float* qc, const float* kc, const float* vc,
                                 int32_t* lut, int32_t* valid, float* oc, hipStream_t s) {
  const int Nc = (int)g.Nc;
  const int tiles = (Nc + kMR - 1) / kMR;
  const int64_t blocks = g.BH * tiles;
  const size_t lds = coarse_mfma_lds_bytes(Nc);
  const float scale = 1.0f / sqrtf((float)DQ);
  auto k = coarse_topk_mfma_kernel<DQ, DV, NS>;
  if (lds > 65536) {
    static std::mutex mu;
    static int granted[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (granted[dev] < (int)lds) {
      const hipError_t e = hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return e;
      granted[dev] = (int)lds;
    }
  }
  hipLaunchKernelGGL(k, dim3((unsigned)blocks), dim3(kMThreads), lds, s, qc, kc, vc, lut, valid, oc, Nc, top_k,
                     tiles, scale, g.group);
  return hipGetLastError();
}

template <int DQ, int DV>
static hipError_t launch_mfma(const Geom& g, int top_k, const float* qc, const float* kc, const float* vc,
                              int32_t* lut, int32_t* valid, float* oc, hipStream_t s) {
  const int slots = (int)((g.Nc + 63) / 64);
  if (slots <= 8) return launch_mfma_ns<DQ, DV, 8>(g, top_k, qc, kc, vc, lut, valid, oc, s);
  if (slots <= 16) return launch_mfma_ns<DQ, DV, 16>(g, top_k, qc, kc, vc, lut, valid, oc, s);
  if (slots <= 32) return launch_mfma_ns<DQ, DV, 32>(g, top_k, qc, kc, vc, lut, valid, oc, s);
  return launch_mfma_ns<DQ, DV, 64>(g, top_k, qc, kc, vc, lut, valid, oc, s);
}

// Sixteen query cubes per workgroup with the products on the matrix cores
// where their score rows fit in LDS; else eight per 512-thread workgroup
// where those fit, else four per 256 threads (measured on 12 heads x 512
// cubes: more, smaller workgroups hide the staging latency better).
template <int DQ, int DV>
static hipError_t launch_d(const Geom& g, int top_k, const float* qc, const float* kc, const float* vc,
                           int32_t* lut, int32_t* valid, float* oc, hipStream_t s) {
  if (coarse_mfma_lds_bytes((int)g.Nc) <= kCoarseLdsMax)
    return launch_mfma<DQ, DV>(g, top_k, qc, kc, vc, lut, valid, oc, s);
  if (coarse_lds_bytes(8, (int)g.Nc, DQ > DV ? DQ : DV) <= kCoarseLdsMax)
    return launch_r<DQ, DV, 8, 512>(g, top_k, qc, kc, vc, lut, valid, oc, s);
  return launch_r<DQ, DV, 4, 256>(g, top_k, qc, kc, vc, lut, valid, oc, s);
}

hipError_t launch_coarse_topk(const Geom& g, int top_k, const float* qc, const float* kc,
                              const float* vc, int32_t* lut, int32_t* valid, float* oc,
                              hipStream_t s) {
  if (g.Nc < 1 || g.Nc > kMaxCoarseCubes) return hipErrorInvalidValue;
  if (g.D == 64 && g.Dv == 64) return launch_d<64, 64>(g, top_k, qc, kc, vc, lut, valid, oc, s);
  if (g.D == 128 && g.Dv == 128) return launch_d<128, 128>(g, top_k, qc, kc, vc, lut, valid, oc, s);
  if (g.D == 128 && g.Dv == 64) return launch_d<128, 64>(g, top_k, qc, kc, vc, lut, valid, oc, s);
  if (g.D == 64 && g.Dv == 128) return launch_d<64, 128>(g, top_k, qc, kc, vc, lut, valid, oc, s);
  return hipErrorInvalidValue;
}

}  // namespace vsa
