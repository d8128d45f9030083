// kda_device.h -- gfx950 device helpers: vector types, MFMA wrappers, bf16/fp16
// conversions.  Lane layouts of the MFMA wrappers (wave64, l = lane, g = l / 16):
//   16x16x32 (A 16xK=32, B 32x16):  A lane l holds row l%16, k = 8g..8g+7;
//                                   B lane l holds col l%16, k = 8g..8g+7;
//   16x16x16 (A 16x16, B 16x16):    A lane l holds row l%16, k = 4g..4g+3;
//                                   B lane l holds col l%16, k = 4g..4g+3;
//   accumulator (16x16):            lane l holds col l%16, rows 4g..4g+3.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x4 mfma_f16_k32(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f16_k16(f16x4 a, f16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_bf16_k32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ f32x4 mfma_bf16_k16(bf16x4 a, bf16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4_t, a), __builtin_bit_cast(s16x4_t, b), c,
                                                   0, 0, 0);
}
// fp32 16x16x4: A lane l holds row l%16, k = l/16; B lane l holds col l%16, k = l/16.
__device__ __forceinline__ f32x4 mfma_f32_k4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// bf16 bit pattern -> fp32 (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// fp32 -> bf16 bits, round to nearest even (hardware conversion).
__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);   // (not a read through a uint16_t pointer: that aliasing is undefined)
}
// Two fp32 -> two bf16 in one word (lo in the low half), round to nearest even
// (one v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{lo, hi}), bf16x2));
}

// Four fp32 values rounded to bf16 (nearest even) and packed for one 8-byte
// store.
__device__ __forceinline__ u32x2 pack_out(f32x4 o) { return u32x2{pack_bf16(o[0], o[1]), pack_bf16(o[2], o[3])}; }

// Sets `bit` in the status word at `status` (global memory) when any lane of
// the wave holds a non-finite value among its M x NT x 4 state values: one
// vector atomic, by the wave's first lane, and only then.
template <int M, int NT>
__device__ __forceinline__ void flag_nonfinite(const f32x4 (&Z)[M][NT], int32_t* status, int bit) {
  bool bad = false;
#pragma unroll
  for (int m = 0; m < M; ++m)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) bad |= !__builtin_isfinite(Z[m][nt][i]);
  if (__builtin_amdgcn_ballot_w64(bad) != 0 && (threadIdx.x & 63) == 0) atomicOr(status, bit);
}

__device__ __forceinline__ uint32_t pack_f16(float lo, float hi) {
  typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
  const f16x2 v = {(_Float16)lo, (_Float16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// Transposing LDS read of a 16-bit matrix M stored row-major (stride in
// elements): within each group of 16 lanes (g = lane / 16), lane i receives
// M[4g + k][i] for k = 0..3, because lane j of the group fetches the 8 bytes at
// M[4g + j / 4][4 (j % 4)] and ds_read_b64_tr_b16 hands element i % 4 of lane
// 4k + i / 4's fetch to lane i as element k.  `m` points at M[0][0] (any column
// offset is part of the pointer).  For M token-major this yields the MFMA
// operand that holds four consecutive tokens of one column per lane.
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
__device__ __forceinline__ f16x4 lds_read_tr(const _Float16* m, int stride, int lane) {
  const int g = lane >> 4, j = lane & 15;
  const _Float16* p = m + (4 * g + (j >> 2)) * stride + 4 * (j & 3);
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
  return __builtin_bit_cast(f16x4, v);
}

// x from the lane n places lower in the same 16-lane row (row_shr:n); the
// first n lanes of a row read 0.
__device__ __forceinline__ float dpp_shr(float x, int n) {
  switch (n) {
    case 1: return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x111, 0xF, 0xF, true));
    case 2: return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x112, 0xF, 0xF, true));
    case 4: return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x114, 0xF, 0xF, true));
    default: return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x118, 0xF, 0xF, true));
  }
}
// Lane 15 of each 16-lane row, broadcast to the row (row_newbcast:15).
__device__ __forceinline__ float dpp_bcast15(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x15F, 0xF, 0xF, false));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

constexpr float kLog2e = 1.4426950408889634f;

// Stored position p (0..31) within a 32-channel block of the Qhat / -W record
// rows holds channel kPermCh(p); kPermPos is the inverse.  This order lets a
// lane of the recurrence feed its 16x16x32 operand straight from the two
// accumulator tiles of the state it owns (rows 4g..4g+3 of both 16-row tiles).
__host__ __device__ constexpr int kPermCh(int p) {
  return ((p & 7) < 4) ? 4 * (p >> 3) + (p & 7) : 16 + 4 * (p >> 3) + (p & 7) - 4;
}
__host__ __device__ constexpr int kPermPos(int c) {
  return (c < 16) ? 8 * (c >> 2) + (c & 3) : 8 * ((c - 16) >> 2) + 4 + ((c - 16) & 3);
}

}  // namespace kda
