// Device helpers shared by the gfx950 kernels (wave64, LDS by absolute
// address, bf16 bit handling) and the host-side launch helpers.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>
#include <set>
#include <string>

#include "uw_internal.h"

namespace uw {

constexpr int kWave = 64;
constexpr int kLdsLimit = 160 * 1024;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ inline float bits_f32(uint32_t u) { return __builtin_bit_cast(float, u); }
__device__ inline uint32_t f32_bits(float f) { return __builtin_bit_cast(uint32_t, f); }

// fp32 -> bf16, round to nearest even; NaN stays a (quiet) NaN of the same sign.
__device__ inline uint16_t f32_to_bf16(float f) {
  uint32_t u = f32_bits(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return uint16_t((u >> 16) | 0x40);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

__device__ inline float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c, false);
}

// Sum over the 64 lanes; every lane gets the result.  DPP inside rows of 16,
// then the four row sums are read out of lanes 0, 16, 32, 48.
__device__ inline float wave_sum(float v) {
  v += bits_f32(__builtin_amdgcn_update_dpp(0, int(f32_bits(v)), 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
  v += bits_f32(__builtin_amdgcn_update_dpp(0, int(f32_bits(v)), 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
  v += bits_f32(__builtin_amdgcn_update_dpp(0, int(f32_bits(v)), 0x141, 0xF, 0xF, false));  // row_half_mirror
  v += bits_f32(__builtin_amdgcn_update_dpp(0, int(f32_bits(v)), 0x140, 0xF, 0xF, false));  // row_mirror
  float a = bits_f32(__builtin_amdgcn_readlane(int(f32_bits(v)), 0));
  float b = bits_f32(__builtin_amdgcn_readlane(int(f32_bits(v)), 16));
  float c = bits_f32(__builtin_amdgcn_readlane(int(f32_bits(v)), 32));
  float d = bits_f32(__builtin_amdgcn_readlane(int(f32_bits(v)), 48));
  return (a + b) + (c + d);
}

// Wave-level ballot helpers.
__device__ inline uint32_t lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi(uint32_t(mask >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(mask), 0u));
}

// s_waitcnt vmcnt(N) in the builtin form (gfx9 encoding: vmcnt in bits 3:0
// and 15:14, expcnt and lgkmcnt left at their maxima), so the compiler's own
// wait insertion knows which loads have completed.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt field");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier for LDS data only: waits for this wave's LDS accesses,
// not for its vector-memory loads still in flight.
__device__ inline void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__device__ inline void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// LDS is addressed with absolute byte addresses (kernels that use these
// helpers use only dynamic LDS, which starts at address 0).
typedef __attribute__((address_space(3))) uint32_t lds_word;
typedef __attribute__((address_space(3))) uint8_t lds_byte;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) u32x4 lds_quad;
typedef __attribute__((address_space(3))) uint16_t lds_half;

__device__ inline uint32_t ld32(uint32_t addr) { return *reinterpret_cast<const lds_word*>(size_t(addr)); }
__device__ inline void st32(uint32_t addr, uint32_t v) { *reinterpret_cast<lds_word*>(size_t(addr)) = v; }
__device__ inline uint32_t ld8(uint32_t addr) { return *reinterpret_cast<const lds_byte*>(size_t(addr)); }
__device__ inline uint32_t ld16(uint32_t addr) { return *reinterpret_cast<const lds_half*>(size_t(addr)); }
__device__ inline uint4 ld128(uint32_t addr) {
  const u32x4 v = *reinterpret_cast<const lds_quad*>(size_t(addr));
  return uint4{v.x, v.y, v.z, v.w};
}
__device__ inline void st128(uint32_t addr, uint4 v) {
  *reinterpret_cast<lds_quad*>(size_t(addr)) = u32x4{v.x, v.y, v.z, v.w};
}
__device__ inline void st16(uint32_t addr, uint32_t v) { *reinterpret_cast<lds_half*>(size_t(addr)) = uint16_t(v); }

typedef __attribute__((address_space(1))) void global_void;
typedef __attribute__((address_space(3))) void lds_void;

// 16 bytes per lane from global memory straight into LDS at dst + 16 * lane
// (no registers); completion is tracked by vmcnt.
__device__ inline void load_lds16(const void* src, uint32_t dst) {
  __builtin_amdgcn_global_load_lds((global_void*)(const_cast<void*>(src)), (lds_void*)(size_t(dst)), 16, 0, 0);
}
// The same, non-temporal (cache policy bit 2, nt), for bytes read once that
// share no cache line with later loads.
__device__ inline void load_lds16_stream(const void* src, uint32_t dst) {
  __builtin_amdgcn_global_load_lds((global_void*)(const_cast<void*>(src)), (lds_void*)(size_t(dst)), 16, 0, 2);
}

// Words read by the whole wave go through the constant address space so they
// become scalar loads.
typedef __attribute__((address_space(4))) const uint32_t const_word;
__device__ inline uint32_t scalar_word(const uint32_t* p, int64_t i) { return ((const const_word*)(p))[i]; }
// 16-bit entry i of a 4-byte aligned table, read as part of its 32-bit word
// (scalar loads move whole words)
__device__ inline uint32_t scalar_half(const uint16_t* p, int64_t i) {
  return (scalar_word(reinterpret_cast<const uint32_t*>(p), i >> 1) >> (16 * (i & 1))) & 0xFFFFu;
}

// ---------------------------------------------------------------------------
// Host side.
inline int hip_check(hipError_t e, const char* what) {
  if (e == hipSuccess) return UW_OK;
  return fail(UW_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

// Allow the full LDS of a CU for a kernel (once per kernel).
template <class K>
void allow_full_lds(K kernel) {
  static std::mutex mu;
  static std::set<const void*> done;
  const void* f = reinterpret_cast<const void*>(kernel);
  std::lock_guard<std::mutex> lk(mu);
  if (done.insert(f).second) (void)hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, kLdsLimit);
}

inline size_t elem_size(int t) { return t == UW_F32 ? 4 : 2; }

}  // namespace uw
