// Helpers of the kernels that stage operands through an LDS ring (gfx950
// only): direct global -> LDS loads, vector-memory waits, LDS swizzles.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sp24 {

// global_load_lds_dwordx4 / _dword: lane l of the instruction writes the bytes
// it loads to LDS at lds_dst + l * size (lds_dst is wave-uniform).  The loads
// count in vmcnt like ordinary vector-memory loads and complete in issue order.
__device__ __forceinline__ void dma16(const void* g, uint8_t* lds_dst) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)g,
                                   (__attribute__((address_space(3))) void*)lds_dst, 16, 0, 0);
}
// The same with the non-temporal hint (data read once, streamed past the caches).
__device__ __forceinline__ void dma16_nt(const void* g, uint8_t* lds_dst) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)g,
                                   (__attribute__((address_space(3))) void*)lds_dst, 16, 0, 2);
}
__device__ __forceinline__ void dma4_nt(const void* g, uint8_t* lds_dst) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)g,
                                   (__attribute__((address_space(3))) void*)lds_dst, 4, 0, 2);
}
__device__ __forceinline__ void dma4(const void* g, uint8_t* lds_dst) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)g,
                                   (__attribute__((address_space(3))) void*)lds_dst, 4, 0, 0);
}

// s_waitcnt vmcnt(n) with the other counters left alone (gfx9 encoding:
// vmcnt[3:0] in bits 3:0, vmcnt[5:4] in bits 15:14).
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 0xF) | (0x7 << 4) | (0xF << 8) | ((n >> 4) << 14));
}

// Wait until at most later * PER of this wave's loads are outstanding
// (`later` is wave-uniform and at most MAXL).
template <int PER, int MAXL>
__device__ __forceinline__ void wait_later(int later) {
  if constexpr (MAXL > 0) {
    if (later >= MAXL) {
      wait_vmcnt<MAXL * PER>();
      return;
    }
    wait_later<PER, MAXL - 1>(later);
  } else {
    wait_vmcnt<0>();
  }
}

// Slot of 16-byte piece c of LDS row r in rows of P pieces: the 16 rows read
// by one quarter-wave of a ds_read_b128 land on the 16 distinct 16-byte bank
// groups (64 banks of 4 bytes).  XOR swizzles are their own inverse: slot s
// of row r holds piece swz16<P>(r, s).
template <int P>
__device__ __forceinline__ int swz16(int r, int c) {
  static_assert(P > 0 && (P & (P - 1)) == 0, "power of two");
  if constexpr (P >= 16) return c ^ (r & 15);
  else return c ^ ((r / (16 / P)) & (P - 1));
}

}  // namespace sp24
