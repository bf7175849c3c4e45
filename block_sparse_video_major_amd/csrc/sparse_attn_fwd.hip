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
// Work decomposition (one workgroup per (batch, head, query cube)):
//   * 256 threads = 4 wavefronts.  Wave w owns query half qh = w & 1 (32 of
//     the cube's 64 query tokens) and key half kh = w >> 1 (32 of the 64
//     tokens of every selected key cube).  The two key halves keep separate
//     online-softmax states that are merged once at the end.
//   * Scores are formed transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x16_bf16: K rows come from LDS as the A operand, Q is
//     held in registers as the B operand for the whole kernel.  In the
//     accumulator layout each lane then owns one query (lane % 32) and 16 of
//     its keys, so the row max is a 16-way local max plus one
//     v_permlane32_swap, and all softmax state is lane-local.
//   * O^T += V^T P^T: P (bf16) is already in B-operand layout; V^T comes from
//     the V tile kept in its natural [key][d] layout in LDS through
//     ds_read_b64_tr_b16 transposing reads.
//   * Key/value cube tiles are double-buffered in LDS: the tiles of list entry
//     i+1 are fetched from global memory into registers while entry i is
//     computed, then written to the other LDS stage; one barrier per entry.
//   * Rescaling of O is lazy: the running max used for exponentiation only
//     moves when a block's max exceeds it by more than 8 (log2 units), which
//     keeps every exp2 <= 256 and is exact because numerator and denominator
//     share the same offset.
//   * Epilogue: the two key halves are merged through LDS, O is normalised,
//     staged in LDS, combined with the gates and the broadcast coarse output
//     and written with coalesced 16-byte stores.
#include "vsa_internal.h"

namespace vsa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));   // register-promotable 16-byte chunk
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kBlk = 64;        // tokens per cube: query tile and key tile
constexpr int kThreads = 256;
constexpr float kTau = 8.0f;    // lazy-rescale threshold (log2 units)

template <int D>
struct Cfg {
  static constexpr int KSTR = D + 8;                 // K tile row stride (bf16): conflict-free b128 reads
  static constexpr int VSTR = D + 32;                // V tile row stride (bf16): conflict-free transposing reads
  static constexpr int K_BYTES = kBlk * KSTR * 2;
  static constexpr int V_BYTES = kBlk * VSTR * 2;
  static constexpr int STAGE_BYTES = K_BYTES + V_BYTES;
  static constexpr int CPR = D / 8;                  // 16-byte chunks per token row
  static constexpr int LOADS = kBlk * CPR / kThreads;  // chunks per thread per tile
  static constexpr int OT = D / 32;                  // 32-row output tiles of O^T
  static constexpr int NOV = OT * 16;                // O^T accumulators per lane
  static constexpr int MERGE_BYTES = 2 * (NOV + 2) * 64 * 4;
  static constexpr int OSTR = D + 4;                 // fp32 staging row stride
  static constexpr int OST_BYTES = kBlk * OSTR * 4;
  static constexpr int LDS_BYTES =
      (2 * STAGE_BYTES > MERGE_BYTES + OST_BYTES) ? 2 * STAGE_BYTES : MERGE_BYTES + OST_BYTES;
};

__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const __bf16 ha = (__bf16)a, hb = (__bf16)b;
  return (uint32_t)__builtin_bit_cast(uint16_t, ha) | ((uint32_t)__builtin_bit_cast(uint16_t, hb) << 16);
}

__device__ __forceinline__ void unpack_bf16x8(const uint4& raw, float* f) {
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

template <int D>
__global__ __launch_bounds__(kThreads, 2) void sparse_attn_fwd_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    const int32_t* __restrict__ lut, const int32_t* __restrict__ valid, int max_kv,
    const float* __restrict__ oc, const __bf16* __restrict__ gate_c, const __bf16* __restrict__ gate_f,
    __bf16* __restrict__ out, float* __restrict__ lse, int Nc, int64_t total, float c_log2) {
  using C = Cfg<D>;
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int64_t wg = xcd_remap((int64_t)blockIdx.x, total);   // = bh * Nc + cube
  const int64_t bh = wg / Nc;
  const int cube = (int)(wg - bh * Nc);
  const int64_t head_off = bh * (int64_t)Nc * kBlk * D;      // element offset of this (b, h)
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int qh = wave & 1, kh = wave >> 1;
  const int n32 = lane & 31, g = lane >> 5;
  const int l16 = lane & 15, h16 = (lane >> 4) & 1;

  int nblk = valid[wg];
  nblk = nblk < 0 ? 0 : (nblk > max_kv ? max_kv : nblk);
  const int32_t* lrow = lut + wg * (int64_t)max_kv;

  // Q as the B operand of S^T = K Q^T: query 32*qh + n32, d = 16*s + 8*g + 0..7.
  bf16x8 qf[D / 16];
  {
    const __bf16* qrow = q + head_off + (int64_t)(cube * kBlk + 32 * qh + n32) * D + 8 * g;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) qf[s] = *reinterpret_cast<const bf16x8*>(qrow + 16 * s);
  }

  f32x16 o[C::OT];
#pragma unroll
  for (int t = 0; t < C::OT; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[t][r] = 0.f;
  float m_used = -INFINITY;  // log2-domain offset used for exponentiation
  float l_part = 0.f;        // this lane's partial row sum (its 16 keys per block)

  // Per-thread staging of one K tile and one V tile: chunk c = tid + u*256 of
  // the contiguous 64 x D tile is row c / CPR, 16-byte column c % CPR.
  u32x4 kreg[C::LOADS], vreg[C::LOADS];
  int st_k[C::LOADS], st_v[C::LOADS];   // LDS byte offsets of the chunks (stage 0)
#pragma unroll
  for (int u = 0; u < C::LOADS; ++u) {
    const int c = tid + u * kThreads;
    const int row = c / C::CPR, col = c % C::CPR;
    st_k[u] = (row * C::KSTR + col * 8) * 2;
    st_v[u] = C::K_BYTES + (row * C::VSTR + col * 8) * 2;
  }
#define VSA_FETCH(IT)                                                                    \
  do {                                                                                   \
    int blk_ = lrow[(IT)];                                                               \
    blk_ = blk_ < 0 ? 0 : (blk_ >= Nc ? Nc - 1 : blk_); /* memory-safety clamp */        \
    const u32x4* kt_ = reinterpret_cast<const u32x4*>(k + head_off + (int64_t)blk_ * kBlk * D); \
    const u32x4* vt_ = reinterpret_cast<const u32x4*>(v + head_off + (int64_t)blk_ * kBlk * D); \
    _Pragma("unroll") for (int u = 0; u < C::LOADS; ++u) {                               \
      kreg[u] = kt_[tid + u * kThreads];                                                 \
      vreg[u] = vt_[tid + u * kThreads];                                                 \
    }                                                                                    \
  } while (0)
#define VSA_STASH(STAGE)                                                                 \
  do {                                                                                   \
    char* base_ = smem + (STAGE) * C::STAGE_BYTES;                                       \
    _Pragma("unroll") for (int u = 0; u < C::LOADS; ++u) {                               \
      *reinterpret_cast<u32x4*>(base_ + st_k[u]) = kreg[u];                              \
      *reinterpret_cast<u32x4*>(base_ + st_v[u]) = vreg[u];                              \
    }                                                                                    \
  } while (0)

  if (nblk > 0) {
    VSA_FETCH(0);
    VSA_STASH(0);
  }
  __syncthreads();

  for (int it = 0; it < nblk; ++it) {
    const int cur = it & 1;
    const bool more = it + 1 < nblk;
    if (more) VSA_FETCH(it + 1);
    const char* kbase = smem + cur * C::STAGE_BYTES;
    const char* vbase = kbase + C::K_BYTES;

    // S^T tile: keys 32*kh + (8*(r/4) + 4*g + r%4), query n32.
    f32x16 s;
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = 0.f;
    const char* krow = kbase + ((32 * kh + n32) * C::KSTR + 8 * g) * 2;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(krow + 32 * ks);
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], s, 0, 0, 0);
    }

    // online softmax (log2 domain)
    float mx = s[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
    mx = pair_max(mx) * c_log2;
    if (__ballot(mx > m_used + kTau) != 0ull) {
      const float m_new = fmaxf(m_used, mx);
      const float alpha = __builtin_amdgcn_exp2f(m_used - m_new);
      l_part *= alpha;
#pragma unroll
      for (int t = 0; t < C::OT; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[t][r] *= alpha;
      m_used = m_new;
    }
    // P^T as the B operand: k-step j covers registers 8j..8j+7, i.e. keys
    // 16j + 8*(e/4) + 4*g + e%4 for slot e.
    bf16x8 pb[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float p = __builtin_amdgcn_exp2f(fmaf(s[8 * j + e], c_log2, -m_used));
        l_part += p;
        pb[j][e] = (__bf16)p;
      }
    }

    // O^T (d x query) += V^T (d x key) P^T (key x query).  For k-step j the
    // A operand of lane (g, d-row) holds keys base + 0..3 and base + 8..11
    // with base = 32*kh + 16*j + 4*g: exactly the keys of pb[j]'s slots.
#pragma unroll
    for (int t = 0; t < C::OT; ++t) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int key0 = 32 * kh + 16 * j + 4 * g + (l16 >> 2);
        const int col = 32 * t + 16 * h16 + 4 * (l16 & 3);
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4*)(vbase + (key0 * C::VSTR + col) * 2));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4*)(vbase + ((key0 + 8) * C::VSTR + col) * 2));
        // concatenate as whole vectors (element-wise bf16 inserts are avoided)
        const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[j], o[t], 0, 0, 0);
      }
    }

    if (more) VSA_STASH(cur ^ 1);
    __syncthreads();
  }

#undef VSA_FETCH
#undef VSA_STASH

  // ---- merge the two key halves, normalise, combine, store ----
  const float l_row = pair_sum(l_part);
  float* mbuf = reinterpret_cast<float*>(smem);                      // [qh][2 + NOV][64]
  float* ost = reinterpret_cast<float*>(smem + C::MERGE_BYTES);      // [64][OSTR]
  if (kh == 1) {
    float* b = mbuf + qh * (C::NOV + 2) * 64;
    b[lane] = m_used;
    b[64 + lane] = l_row;
#pragma unroll
    for (int t = 0; t < C::OT; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) b[(2 + t * 16 + r) * 64 + lane] = o[t][r];
  }
  __syncthreads();
  if (kh == 0) {
    const float* b = mbuf + qh * (C::NOV + 2) * 64;
    const float m1 = b[lane], l1 = b[64 + lane];
    const float m = fmaxf(m_used, m1);
    const float a0 = (m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_used - m);
    const float a1 = (m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m1 - m);
    const float l = l_row * a0 + l1 * a1;
    const float inv = l > 0.f ? 1.f / l : 0.f;
    float* orow = ost + (32 * qh + n32) * C::OSTR;
#pragma unroll
    for (int t = 0; t < C::OT; ++t)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        float4 w;
        w.x = (o[t][4 * rq + 0] * a0 + b[(2 + t * 16 + 4 * rq + 0) * 64 + lane] * a1) * inv;
        w.y = (o[t][4 * rq + 1] * a0 + b[(2 + t * 16 + 4 * rq + 1) * 64 + lane] * a1) * inv;
        w.z = (o[t][4 * rq + 2] * a0 + b[(2 + t * 16 + 4 * rq + 2) * 64 + lane] * a1) * inv;
        w.w = (o[t][4 * rq + 3] * a0 + b[(2 + t * 16 + 4 * rq + 3) * 64 + lane] * a1) * inv;
        // d = 32*t + 8*rq + 4*g + 0..3
        *reinterpret_cast<float4*>(orow + 32 * t + 8 * rq + 4 * g) = w;
      }
    if (lse != nullptr && g == 0) {
      const float val = (l > 0.f) ? (m + __log2f(l)) * 0.69314718055994531f : -INFINITY;
      lse[wg * kBlk + 32 * qh + n32] = val;
    }
  }
  __syncthreads();

  const float* ocrow = oc ? oc + wg * (int64_t)D : nullptr;
#pragma unroll
  for (int u = 0; u < C::LOADS; ++u) {
    const int c = tid + u * kThreads;
    const int row = c / C::CPR, col = c % C::CPR;
    const int64_t gidx = head_off + (int64_t)(cube * kBlk + row) * D + col * 8;
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

template <int D>
hipError_t launch_d(const Geom& g, const void* q, const void* k, const void* v, const int32_t* lut,
                    const int32_t* valid, int max_kv, const float* oc, const void* gate_c,
                    const void* gate_f, void* out, float* lse, hipStream_t s) {
  using C = Cfg<D>;
  auto kern = sparse_attn_fwd_kernel<D>;
  // The dynamic-LDS limit is raised once per device.
  static bool attr_set[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  if (!attr_set[dev]) {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       C::LDS_BYTES);
    if (e != hipSuccess) return e;
    attr_set[dev] = true;
  }
  const int64_t total = g.BH * g.Nc;
  const float c_log2 = 1.4426950408889634f / sqrtf((float)D);
  hipLaunchKernelGGL(kern, dim3((unsigned)total), dim3(kThreads), C::LDS_BYTES, s, (const __bf16*)q,
                     (const __bf16*)k, (const __bf16*)v, lut, valid, max_kv, oc, (const __bf16*)gate_c,
                     (const __bf16*)gate_f, (__bf16*)out, lse, (int)g.Nc, total, c_log2);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_sparse_attn_fwd(const Geom& g, const void* q, const void* k, const void* v,
                                  const int32_t* lut, const int32_t* valid, int max_kv,
                                  const float* oc, const void* gate_c, const void* gate_f,
                                  void* out, float* lse, hipStream_t s) {
  if (g.D == 128) return launch_d<128>(g, q, k, v, lut, valid, max_kv, oc, gate_c, gate_f, out, lse, s);
  if (g.D == 64) return launch_d<64>(g, q, k, v, lut, valid, max_kv, oc, gate_c, gate_f, out, lse, s);
  return hipErrorInvalidValue;
}

}  // namespace vsa
