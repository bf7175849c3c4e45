// Device helpers shared by the gfx950 attention kernels: bf16 vector types,
// bf16 packing, direct global->LDS tile loads and vector-memory waits.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vsa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef const __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  // built as a two-element vector so that both roundings are one packed
  // conversion instruction
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t h = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, h);
}

__device__ __forceinline__ void unpack_bf16x8(const uint4& raw, float* f) {
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

// Direct global->LDS loads of one wave's share of a tile: for piece
// n = 0..N-1 every lane moves the 16 bytes at base + voff[n] + 1024 n (base:
// wave-uniform pointer, voff: per-lane byte offsets) to LDS byte address
// lds_base + 1024 n + 16 * lane.  Issued through inline assembly so that the
// compiler does not track these LDS writes; completion is enforced
// explicitly (wait_vmem + barrier) before any wave reads the slot.
template <int N>
__device__ __forceinline__ void dma_tile(const void* base, const uint32_t (&voff)[N], uint32_t lds_base) {
  // M0 must come from a scalar register: force the (wave-uniform) address
  // there even where the compiler kept it in a vector register.  The
  // instruction offset n * 1024 moves both the global source and the LDS
  // destination of load n, so M0 is set once per tile; voff[n] holds the
  // lane's source offset minus n * 1024.
  lds_base = __builtin_amdgcn_readfirstlane(lds_base);
  static_assert(N == 2 || N == 4, "loads per tile");
  if constexpr (N == 4) {
    asm volatile(
        "s_mov_b32 m0, %4\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %0, %5\n\t"
        "global_load_lds_dwordx4 %1, %5 offset:1024\n\t"
        "global_load_lds_dwordx4 %2, %5 offset:2048\n\t"
        "global_load_lds_dwordx4 %3, %5 offset:3072"
        :
        : "v"(voff[0]), "v"(voff[1]), "v"(voff[2]), "v"(voff[3]), "s"(lds_base), "s"(base)
        : "memory", "m0");
  } else {
    asm volatile(
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %0, %3\n\t"
        "global_load_lds_dwordx4 %1, %3 offset:1024"
        :
        : "v"(voff[0]), "v"(voff[1]), "s"(lds_base), "s"(base)
        : "memory", "m0");
  }
}

// Direct global->LDS loads of one wave's N pieces of a tile whose pieces lie
// at their own offsets from the tile base: piece n moves the 16 bytes at
// base + pd[n] + voff + 1024 n of every lane to LDS byte address lds_base +
// 1024 n + 16 * lane (pd[n]: wave-uniform byte offsets, voff: the lane's
// offset within a piece).  The tile's rows are then gathered from a layout
// in which they are not contiguous, one contiguous 1 KiB run per piece.
template <int N>
__device__ __forceinline__ void dma_pieces(const char* base, const int64_t (&pd)[N], uint32_t voff,
                                           uint32_t lds_base) {
  lds_base = __builtin_amdgcn_readfirstlane(lds_base);
  static_assert(N == 2 || N == 4, "loads per tile");
  if constexpr (N == 4) {
    asm volatile(
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %0, %2\n\t"
        "global_load_lds_dwordx4 %0, %3 offset:1024\n\t"
        "global_load_lds_dwordx4 %0, %4 offset:2048\n\t"
        "global_load_lds_dwordx4 %0, %5 offset:3072"
        :
        : "v"(voff), "s"(lds_base), "s"(base + pd[0]), "s"(base + pd[1]), "s"(base + pd[2]), "s"(base + pd[3])
        : "memory", "m0");
  } else {
    asm volatile(
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %0, %2\n\t"
        "global_load_lds_dwordx4 %0, %3 offset:1024"
        :
        : "v"(voff), "s"(lds_base), "s"(base + pd[0]), "s"(base + pd[1])
        : "memory", "m0");
  }
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const lds_void*)p;
}

__device__ __forceinline__ const char* uniform_ptr(const char* p) {
  const uint64_t u = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  return (const char*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

// Wait until at most N of this wave's vector-memory operations are pending
// (expcnt and lgkmcnt fields at their no-wait maxima).  The builtin form is
// visible to the compiler's own wait-count tracking.
template <int N>
__device__ __forceinline__ void wait_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt field");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

}  // namespace vsa
