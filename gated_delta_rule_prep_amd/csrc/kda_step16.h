// kda_step16.h -- one 16-token chunk step of the KDA recurrence on a wave's
// slice of the state (gfx950), shared by the split recurrence kernel and the
// fused kernel.
//
// The chunkwise form of the delta-rule recurrence (the second of the two
// stages in the FlashKDA blog post "FlashKDA：月之暗面开源的 Kimi Delta Attention
// 高性能内核", §二 2.2), with Z the chunk-start state slice (K x 16 NT), the
// chunk record (Qhat, -Khat, Kbar, T, Mqk, gamma) and the chunk's value rows V.
// The residual E = T V - (T Khat) Z is taken as T (V - Khat Z), so the record
// needs Khat itself rather than W = T Khat:
//   R = V + (-Khat) Z            fp16 MFMA 16x16x32 chain over the 128 channels,
//                                accumulating onto V (fp32)
//   E = T R                      fp16 MFMA 16x16x16
//   O^T = Z^T Qhat^T + E^T Mqk^T fp16 MFMA; the same register operands as
//                                O = Qhat Z + Mqk E with A and B swapped, so
//                                each lane ends up with four consecutive value
//                                columns of one token and stores them directly
//   Z = diag(gam) Z + Kbar^T E   fp16 MFMA 16x16x16, accumulating onto gam * Z
// Z is converted to fp16 per step for the two products that read it; the state
// itself stays fp32.  The channel order of Qhat / -Khat in the record matches the
// rows a lane holds in its two accumulator tiles (kPermCh), so the conversion
// needs no lane exchange.  The decay factors reach the lanes by DPP row
// broadcast from a permuted copy of gamma (kGamSlot).
//
// Record layout in LDS (byte offsets REC_* of kda_internal.h), swizzled so
// that the operand reads hit distinct banks: Qhat and -Khat token row r keeps
// its 16-byte piece p at piece position p ^ r; Kbar row r keeps piece p at
// p ^ 2 (r % 4); T^T, Mqk^T and gamma are stored as in the HBM record.  The
// value tile (raw bf16, `val_row_bytes` bytes per token row) keeps piece p of
// row r at p ^ 2 (r % 4).
#pragma once

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

__device__ __forceinline__ f16x4 f16x4_of(f32x4 x) {
  f16x4 r;
  r[0] = (_Float16)x[0]; r[1] = (_Float16)x[1]; r[2] = (_Float16)x[2]; r[3] = (_Float16)x[3];
  return r;
}

typedef __attribute__((address_space(3))) s16x4 lds_s16x4_t;

// Transposing read of the 16 x 16 block of a swizzled token-major 16-bit tile
// (row stride `rowb` bytes, piece p of row r at p ^ 2 (r % 4)) whose first
// column is `col` (a multiple of 16): lane (lc, lg) receives
// M[4lg..4lg+3][col + lc] (see lds_read_tr).
__device__ __forceinline__ s16x4 tr_swz(const char* tile, int rowb, int col, int lane) {
  const int g = lane >> 4, j = lane & 15;
  const int r = 4 * g + (j >> 2);
  const int c = col + 4 * (j & 3);                 // first of the 4 elements this lane fetches
  const int p = (c >> 3) ^ (2 * (r & 3));
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(tile + r * rowb + 16 * p + 2 * (c & 7)));
}

// The MFMA operands of one chunk step.
template <int NT>
struct Ops {
  f16x4 aT, am;          // T[lc][4lg..4lg+3], Mqk[lc][4lg..4lg+3]
  f32x4 v[NT];           // V[4lg..4lg+3][wc + 16nt + lc] (exact from bf16)
  f16x8 aw[4], aq[4];    // -Khat, Qhat row lc, channels of 32-block s at the lane's 8 positions
  f16x4 ak[8];           // Kbar[4lg..4lg+3][16m + lc]
  f32x2 g2;              // gamma of the rows that this lane hands to its 16-lane row
};

// Operands of one step from a record `rec` and a value tile `val` (raw bf16,
// `val_row_bytes` per token row) in LDS; `wc` is the wave's first column in
// the tile.
template <int NT>
__device__ __forceinline__ void read_ops(Ops<NT>& o, const char* rec, const char* val, int val_row_bytes, int wc,
                                         int lane) {
  const int lg = lane >> 4, lc = lane & 15;
  o.aT = lds_read_tr(reinterpret_cast<const _Float16*>(rec + REC_T), C, lane);
  o.am = lds_read_tr(reinterpret_cast<const _Float16*>(rec + REC_MQK), C, lane);
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const s16x4 raw = tr_swz(val, val_row_bytes, wc + 16 * nt, lane);
#pragma unroll
    for (int i = 0; i < 4; ++i) o.v[nt][i] = bf16_to_f32((uint16_t)raw[i]);
  }
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int p = (4 * s + lg) ^ lc;
    o.aw[s] = *reinterpret_cast<const f16x8*>(rec + REC_NK + 256 * lc + 16 * p);
    o.aq[s] = *reinterpret_cast<const f16x8*>(rec + REC_QH + 256 * lc + 16 * p);
  }
#pragma unroll
  for (int m = 0; m < 8; ++m) o.ak[m] = __builtin_bit_cast(f16x4, tr_swz(rec + REC_KB, 2 * K, 16 * m, lane));
  o.g2 = *reinterpret_cast<const f32x2*>(rec + REC_GAM + 8 * lane);
}

// x from lane L of this lane's 16-lane row.
template <int L>
__device__ __forceinline__ float row_bcast(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x150 + L, 0xF, 0xF, false));
}

// Row 16M + 4lg + i decays by gamma[16M + 4lg + i], held by lane 4 (M % 4) + i
// of the 16-lane row in register M / 4 (see kGamSlot).
template <int M>
__device__ __forceinline__ f32x4 decay(f32x4 z, f32x2 g2) {
  const float g = g2[M >> 2];
  return f32x4{z[0] * row_bcast<4 * (M & 3) + 0>(g), z[1] * row_bcast<4 * (M & 3) + 1>(g),
               z[2] * row_bcast<4 * (M & 3) + 2>(g), z[3] * row_bcast<4 * (M & 3) + 3>(g)};
}

// Precision variants of the step (compile-time bits), for the study of the
// choices in §二 2.3 of the FlashKDA blog post; the library's own arithmetic is
// kPrecDefault.
//   kPrecBf16State: the state is rounded to bf16 after every chunk update (the
//     pages store it in bf16 between updates; the update itself stays fp32).
//   kPrecBf16Inverse: E = T R with T and R in bf16 (the pages keep the inverse
//     in fp16); E is rounded to bf16 and, exactly representable in fp16, feeds
//     the later products unchanged.
//   kPrecBf16StateProducts: Khat Z and Qhat Z with the state copy and the
//     record's -Khat and Qhat in bf16 instead of fp16.
constexpr int kPrecDefault = 0, kPrecBf16State = 1, kPrecBf16Inverse = 2, kPrecBf16StateProducts = 4;

// bf16 rounding for the variants, written out on the fp32 bits (round to
// nearest even; the values here are finite): the bf16 bits of x, and x rounded
// to bf16 as an fp32 value.
__device__ __forceinline__ uint32_t bf16_bits(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ float bf16_round(float x) { return __uint_as_float(bf16_bits(x) << 16); }
__device__ __forceinline__ bf16x4 bf4_of(f32x4 x) {
  const u32x2 w = {bf16_bits(x[0]) | (bf16_bits(x[1]) << 16), bf16_bits(x[2]) | (bf16_bits(x[3]) << 16)};
  return __builtin_bit_cast(bf16x4, w);
}
__device__ __forceinline__ bf16x4 bf4_of(f16x4 h) {
  return bf4_of(f32x4{(float)h[0], (float)h[1], (float)h[2], (float)h[3]});
}
__device__ __forceinline__ bf16x8 bf8_of(f32x4 lo, f32x4 hi) {
  const u32x4 w = {bf16_bits(lo[0]) | (bf16_bits(lo[1]) << 16), bf16_bits(lo[2]) | (bf16_bits(lo[3]) << 16),
                   bf16_bits(hi[0]) | (bf16_bits(hi[1]) << 16), bf16_bits(hi[2]) | (bf16_bits(hi[3]) << 16)};
  return __builtin_bit_cast(bf16x8, w);
}
__device__ __forceinline__ bf16x8 bf8_of(f16x8 h) {
  return bf8_of(f32x4{(float)h[0], (float)h[1], (float)h[2], (float)h[3]},
                f32x4{(float)h[4], (float)h[5], (float)h[6], (float)h[7]});
}

// One chunk step from operands in registers: updates Z and returns the output
// tile as O^T in fp32 (lane (lc, lg): token lc, value columns 16nt + 4lg .. +3
// of the wave).  Callers round and store it a step later (pack_out), well
// after the MFMA that produces it: a vector read of an MFMA result soon after
// it issues, with further MFMAs queued behind it, has been measured on gfx950
// to return the register's old contents, although the compiler's wait states
// were in place (see the recurrence kernel's notes).
template <int NT, int PV = kPrecDefault>
__device__ __forceinline__ void compute(f32x4 (&Z)[8][NT], const Ops<NT>& o, f32x4 (&out)[NT]) {
  // ---- R = V + (-Khat) Z ; O^T = Z^T Qhat^T
  f32x4 R[NT], O[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    R[nt] = o.v[nt];
    O[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int s = 0; s < 4; ++s) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      if constexpr ((PV & kPrecBf16StateProducts) != 0) {
        const bf16x8 zb = bf8_of(Z[2 * s][nt], Z[2 * s + 1][nt]);
        R[nt] = mfma_bf16_k32(bf8_of(o.aw[s]), zb, R[nt]);
        O[nt] = mfma_bf16_k32(zb, bf8_of(o.aq[s]), O[nt]);
      } else {
        f16x8 zb;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          zb[i] = (_Float16)Z[2 * s][nt][i];
          zb[4 + i] = (_Float16)Z[2 * s + 1][nt][i];
        }
        R[nt] = mfma_f16_k32(o.aw[s], zb, R[nt]);
        O[nt] = mfma_f16_k32(zb, o.aq[s], O[nt]);
      }
    }
  }

  // ---- E = T R ; O^T += E^T Mqk^T (R's accumulator layout is the B operand
  // layout of the 16x16x16 product: rows 4lg..4lg+3 of column lc)
  f16x4 eb[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    if constexpr ((PV & kPrecBf16Inverse) != 0) {
      const f32x4 e = mfma_bf16_k16(bf4_of(o.aT), bf4_of(R[nt]), f32x4{0.f, 0.f, 0.f, 0.f});
      eb[nt] = f16x4_of(f32x4{bf16_round(e[0]), bf16_round(e[1]), bf16_round(e[2]), bf16_round(e[3])});
    } else {
      eb[nt] = f16x4_of(mfma_f16_k16(o.aT, f16x4_of(R[nt]), f32x4{0.f, 0.f, 0.f, 0.f}));
    }
    O[nt] = mfma_f16_k16(eb[nt], o.am, O[nt]);
  }

  // ---- Z = diag(gam) Z + Kbar^T E
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    Z[0][nt] = mfma_f16_k16(o.ak[0], eb[nt], decay<0>(Z[0][nt], o.g2));
    Z[1][nt] = mfma_f16_k16(o.ak[1], eb[nt], decay<1>(Z[1][nt], o.g2));
    Z[2][nt] = mfma_f16_k16(o.ak[2], eb[nt], decay<2>(Z[2][nt], o.g2));
    Z[3][nt] = mfma_f16_k16(o.ak[3], eb[nt], decay<3>(Z[3][nt], o.g2));
    Z[4][nt] = mfma_f16_k16(o.ak[4], eb[nt], decay<4>(Z[4][nt], o.g2));
    Z[5][nt] = mfma_f16_k16(o.ak[5], eb[nt], decay<5>(Z[5][nt], o.g2));
    Z[6][nt] = mfma_f16_k16(o.ak[6], eb[nt], decay<6>(Z[6][nt], o.g2));
    Z[7][nt] = mfma_f16_k16(o.ak[7], eb[nt], decay<7>(Z[7][nt], o.g2));
  }

  if constexpr ((PV & kPrecBf16State) != 0) {   // the state kept in bf16 between updates
#pragma unroll
    for (int m = 0; m < 8; ++m)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) Z[m][nt][i] = bf16_round(Z[m][nt][i]);
  }

#pragma unroll
  for (int nt = 0; nt < NT; ++nt) out[nt] = O[nt];
}

// State slice of a wave: Z[m][nt] holds rows 16m + 4lg + i, column
// col0 + 16nt + lc of the state of one (sequence, head), read from `s_in`
// ([V][K] of that pair, bf16 or fp32; nullptr = zero state).
template <int NT>
__device__ __forceinline__ void load_state(f32x4 (&Z)[8][NT], const void* s_in, int dtype, int64_t sbase, int col0,
                                           int lc, int lg) {
#pragma unroll
  for (int m = 0; m < 8; ++m)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int64_t idx = sbase + (int64_t)(col0 + 16 * nt + lc) * K + 16 * m + 4 * lg;
      if (s_in == nullptr) {
        Z[m][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
      } else if (dtype == 2 /* KDA_DTYPE_FP32 */) {
        Z[m][nt] = *reinterpret_cast<const f32x4*>(static_cast<const float*>(s_in) + idx);
      } else {
        const u32x2 w = *reinterpret_cast<const u32x2*>(static_cast<const uint16_t*>(s_in) + idx);
        Z[m][nt] = f32x4{bf16_lo(w[0]), bf16_hi(w[0]), bf16_lo(w[1]), bf16_hi(w[1])};
      }
    }
}

// The inverse of load_state: bf16 (round to nearest even) or fp32.
template <int NT>
__device__ __forceinline__ void store_state(const f32x4 (&Z)[8][NT], void* s_out, int dtype, int64_t sbase, int col0,
                                            int lc, int lg) {
#pragma unroll
  for (int m = 0; m < 8; ++m)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int64_t idx = sbase + (int64_t)(col0 + 16 * nt + lc) * K + 16 * m + 4 * lg;
      if (dtype == 2 /* KDA_DTYPE_FP32 */) {
        *reinterpret_cast<f32x4*>(static_cast<float*>(s_out) + idx) = Z[m][nt];
      } else {
        u32x2 w;
        w[0] = pack_bf16(Z[m][nt][0], Z[m][nt][1]);
        w[1] = pack_bf16(Z[m][nt][2], Z[m][nt][3]);
        *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(s_out) + idx) = w;
      }
    }
}

}  // namespace kda
