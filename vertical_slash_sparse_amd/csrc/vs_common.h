// vs_common.h -- internal helpers shared by the gfx950 kernels of libvs.
//
// Matrix-core operand layouts used throughout (measured on gfx950):
//   v_mfma_f32_32x32x16_bf16:  A[i][k] lives in lane i + 32*(k/8), element k%8;
//                              B[k][j] in lane j + 32*(k/8), element k%8;
//                              D[i][j] in lane j + 32*((i/4)%2), element 4*(i/8) + i%4.
// Only the products matter, so any permutation of k applied to both A and B
// gives the same D; the attention kernel uses that freedom to feed the
// softmax output straight back in as an operand.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vs {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// two fp32 -> packed bf16 pair (round to nearest even; v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// value of lane (l ^ 32): exchange between the two halves of a wave
__device__ __forceinline__ float swap_halves(float x) {
  return __shfl_xor(x, 32, 64);
}

// x of this lane combined with x of lane (l ^ 32), via v_permlane32_swap:
// after the swap one output holds the lower half's values and the other the
// upper half's, in every lane
__device__ __forceinline__ float half_max(float x) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __builtin_elementwise_maximum(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
}
__device__ __forceinline__ float half_sum(float x) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
}

// word 3 of a raw buffer resource on gfx9-family parts (32-bit data format);
// accesses at or past num_records return zero
constexpr int kBufferFlags = 0x00020000;

// raw buffer resource words: base, stride 0, num_records bytes
__device__ __forceinline__ u32x4 buffer_words(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)base;
  return u32x4{(uint32_t)a, (uint32_t)(a >> 32) & 0xffffu, bytes, (uint32_t)kBufferFlags};
}

// LDS-DMA: every lane moves 16 bytes from the buffer at byte offset voff into
// LDS at lds_addr + 16 * lane.  The instruction has no register results, so
// nothing the compiler allocates depends on it; completion is tracked by the
// caller with an explicit s_waitcnt vmcnt.  Offsets at or past num_records
// deliver zeros.
// The LDS address and the resource must be wave-uniform; readfirstlane
// states that to the compiler (it folds away when they already sit in SGPRs).
__device__ __forceinline__ void dma16(const u32x4& rsrc, uint32_t lds_addr, uint32_t voff) {
  const u32x4 r = {(uint32_t)__builtin_amdgcn_readfirstlane((int)rsrc[0]),
                   (uint32_t)__builtin_amdgcn_readfirstlane((int)rsrc[1]),
                   (uint32_t)__builtin_amdgcn_readfirstlane((int)rsrc[2]),
                   (uint32_t)__builtin_amdgcn_readfirstlane((int)rsrc[3])};
  const uint32_t a = (uint32_t)__builtin_amdgcn_readfirstlane((int)lds_addr);
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(a), "v"(voff), "s"(r)
               : "memory", "m0");
}

// per-lane select driven by a wave-uniform 64-bit lane mask
__device__ __forceinline__ float select_mask(uint64_t m, float a, float b) {
  return __builtin_amdgcn_inverse_ballot_w64(m) ? a : b;
}

__device__ __forceinline__ int wave_uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

}  // namespace vs
