// Device helpers shared by the bf16 MFMA attention kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssa {

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Two floats -> two bfloat16 (round to nearest even) in one instruction.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const bf16x2_t r = __builtin_convertvector(f32x2_t{a, b}, bf16x2_t);
  return __builtin_bit_cast(uint32_t, r);
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Wait for every outstanding vector memory operation of this wave.
__device__ __forceinline__ void wait_vm() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }


typedef int i32x4_t __attribute__((ext_vector_type(4)));
// Buffer descriptor words for [base, base + bytes) (stride 0, raw buffer).
__device__ __forceinline__ i32x4_t make_rsrc_words(const void* base, uint32_t bytes) {
  const uint64_t p = (uint64_t)(uintptr_t)base;
  return i32x4_t{(int)__builtin_amdgcn_readfirstlane((uint32_t)p),
                 (int)(__builtin_amdgcn_readfirstlane((uint32_t)(p >> 32)) & 0xffffu),
                 (int)__builtin_amdgcn_readfirstlane(bytes), 0x00020000};
}
// One 16-byte-per-lane global -> LDS copy (buffer_load_dwordx4 ... lds),
// issued from inline assembly so that the compiler inserts no wait of its
// own before later LDS reads: the caller orders every copy against the
// reads of its stage with explicit vmcnt waits and barriers. m0 (the LDS
// destination of lane 0) is saved and restored around the copy.
__device__ __forceinline__ void copy16_to_lds(i32x4_t rsrc, uint32_t soff, uint32_t voff,
                                              uint32_t lds_addr) {
  uint32_t keep;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %2, %3, %4 offen lds\n\t"
      "s_nop 0\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(keep)
      : "s"(lds_addr), "v"(voff), "s"(rsrc), "s"(soff)
      : "memory");
}

// 16-byte chunk swizzle of LDS tiles whose MFMA reads touch, in one
// ds_read_b128 phase, 16 rows that differ in row bits 0, 1, 3 and 4 (rows
// 8a + 4c + b for a, b in 0..3 and a fixed c): those rows land on 16
// distinct 16-byte bank groups. 256-byte rows (16 chunks) use
// chunk ^ f(row) with f taking row bits 0,1,3,4; 128-byte rows (8 chunks, two
// rows per 256 bytes) use row bits 1,3,4. The map is an involution.
template <int SPR>
__device__ __forceinline__ int kswz(int row, int chunk) {
  if constexpr (SPR == 16) return chunk ^ ((row & 3) | ((row >> 1) & 12));
  else return chunk ^ (((row >> 1) & 1) | ((row >> 2) & 6));
}

}  // namespace ssa
