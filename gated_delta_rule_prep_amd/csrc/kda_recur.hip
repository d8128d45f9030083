// kda_recur.hip -- chunk-recurrence kernel for gfx950.
//
// The second stage of the split the pages describe (P1 §二 2.2: chunk-by-chunk
// delta-rule recurrence, output projection, rolling state).  One workgroup of
// 4 waves per (sequence, head); wave w owns the state's value columns
// [32w, 32w + 32), which never interact (every step acts on each value column of
// the state separately), so the waves need no exchange.  The 128 x 32 fp32
// state slice lives in registers as 8 x 2 MFMA accumulator tiles for the whole
// sequence.
//
// P1 = blog post "FlashKDA：月之暗面开源的 Kimi Delta Attention 高性能内核".
//
// Per chunk (records from the prep kernel, Z = chunk-start state, K x V):
//   U = T V                      fp16 MFMA 16x16x16
//   E = U + (-W) Z               fp16 MFMA 16x16x32 chain over the 128 channels
//   O = Qhat Z + Mqk E           fp16 MFMA (E feeds the B operand directly: the
//                                accumulator layout of E is the B-operand layout)
//   Z = diag(gam) Z + Kbar^T E   fp16 MFMA 16x16x16, accumulating onto gam * Z
// Z is converted to fp16 per step for the two products that read it; the state
// itself stays fp32.  The channel order of Qhat / -W in the record matches the
// rows a lane holds in its two accumulator tiles (kPermCh), so the conversion
// needs no lane exchange.
#include "kda_device.h"
#include "kda_internal.h"
#include "../../include/kda.h"

namespace kda {
namespace {

constexpr int kThreads = 256;
constexpr int SV = V + 8;   // bf16 [16][SV] staged values

struct __align__(16) RecurSmem {
  __align__(16) char rec[REC_BYTES];
  __align__(16) uint16_t v[C][SV];
};

__device__ __forceinline__ f16x4 f16x4_of(f32x4 x) {
  f16x4 r;
  r[0] = (_Float16)x[0]; r[1] = (_Float16)x[1]; r[2] = (_Float16)x[2]; r[3] = (_Float16)x[3];
  return r;
}

__global__ __launch_bounds__(kThreads) void recur_kernel(RecurArgs a) {
  __shared__ RecurSmem sm;
  const int64_t H = a.H;
  const int64_t slot = blockIdx.x / H;
  const int h = (int)(blockIdx.x - slot * H);
  const int32_t* order = reinterpret_cast<const int32_t*>(a.ws + a.lay.order);
  const int n = order[slot];
  const SeqEntry se = reinterpret_cast<const SeqEntry*>(a.ws + a.lay.seq_table)[n];
  const ChunkEntry* chunks = reinterpret_cast<const ChunkEntry*>(a.ws + a.lay.chunk_table);
  const char* recs = a.ws + a.lay.records + (int64_t)h * a.lay.max_chunks * REC_BYTES;

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, lg = lane >> 4, lc = lane & 15;
  const int64_t sbase = ((int64_t)n * H + h) * V * K;   // state [n][h][v][k]

  // ---- state slice: Z[m][nt] holds rows 16m + 4lg + i, column 32*wave + 16nt + lc
  f32x4 Z[8][2];
#pragma unroll
  for (int m = 0; m < 8; ++m)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const int64_t idx = sbase + (int64_t)(32 * wave + 16 * nt + lc) * K + 16 * m + 4 * lg;
      if (a.s_in == nullptr) {
        Z[m][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
      } else if (a.state_dtype == KDA_DTYPE_FP32) {
        Z[m][nt] = *reinterpret_cast<const f32x4*>(static_cast<const float*>(a.s_in) + idx);
      } else {
        const u32x2 w = *reinterpret_cast<const u32x2*>(static_cast<const uint16_t*>(a.s_in) + idx);
        Z[m][nt] = f32x4{bf16_lo(w[0]), bf16_hi(w[0]), bf16_lo(w[1]), bf16_hi(w[1])};
      }
    }

  for (int ci = 0; ci < se.nchunks; ++ci) {
    const int chunk = se.first_chunk + ci;
    const ChunkEntry ce = chunks[chunk];
    const char* rec = recs + (int64_t)chunk * REC_BYTES;

    // ---- stage the record and the chunk's values in LDS
    for (int o = tid * 16; o < REC_BYTES; o += kThreads * 16)
      *reinterpret_cast<u32x4*>(sm.rec + o) = *reinterpret_cast<const u32x4*>(rec + o);
    {
      const int r = tid >> 4, c8 = (tid & 15) * 8;
      u32x4 w = {0, 0, 0, 0};
      if (r < ce.len) w = *reinterpret_cast<const u32x4*>(a.v + (((int64_t)ce.row0 + r) * H + h) * V + c8);
      *reinterpret_cast<u32x4*>(&sm.v[r][c8]) = w;
    }
    __syncthreads();

    const _Float16* nW = reinterpret_cast<const _Float16*>(sm.rec + REC_NW);
    const _Float16* qH = reinterpret_cast<const _Float16*>(sm.rec + REC_QH);
    const _Float16* kBt = reinterpret_cast<const _Float16*>(sm.rec + REC_KBT);
    const _Float16* Tm = reinterpret_cast<const _Float16*>(sm.rec + REC_T);
    const _Float16* Mq = reinterpret_cast<const _Float16*>(sm.rec + REC_MQK);
    const float* gam = reinterpret_cast<const float*>(sm.rec + REC_GAM);

    // ---- U = T V
    f32x4 E[2], O[2];
    const f16x4 aT = *reinterpret_cast<const f16x4*>(Tm + lc * C + 4 * lg);
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const int col = 32 * wave + 16 * nt + lc;
      f16x4 bv;
#pragma unroll
      for (int i = 0; i < 4; ++i) bv[i] = (_Float16)bf16_to_f32(sm.v[4 * lg + i][col]);
      E[nt] = mfma_f16_k16(aT, bv, f32x4{0.f, 0.f, 0.f, 0.f});
      O[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    // ---- E += (-W) Z ; O = Qhat Z
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const f16x8 aw = *reinterpret_cast<const f16x8*>(nW + lc * K + 32 * s + 8 * lg);
      const f16x8 aq = *reinterpret_cast<const f16x8*>(qH + lc * K + 32 * s + 8 * lg);
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        f16x8 zb;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          zb[i] = (_Float16)Z[2 * s][nt][i];
          zb[4 + i] = (_Float16)Z[2 * s + 1][nt][i];
        }
        E[nt] = mfma_f16_k32(aw, zb, E[nt]);
        O[nt] = mfma_f16_k32(aq, zb, O[nt]);
      }
    }

    // ---- O += Mqk E
    f16x4 eb[2];
    const f16x4 am = *reinterpret_cast<const f16x4*>(Mq + lc * C + 4 * lg);
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      eb[nt] = f16x4_of(E[nt]);
      O[nt] = mfma_f16_k16(am, eb[nt], O[nt]);
    }

    // ---- Z = diag(gam) Z + Kbar^T E
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const f32x4 gm = *reinterpret_cast<const f32x4*>(gam + 16 * m + 4 * lg);
      const f16x4 ak = *reinterpret_cast<const f16x4*>(kBt + (16 * m + lc) * C + 4 * lg);
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        f32x4 zc = Z[m][nt] * gm;
        Z[m][nt] = mfma_f16_k16(ak, eb[nt], zc);
      }
    }

    // ---- output rows of this chunk
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const int col = 32 * wave + 16 * nt + lc;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * lg + i;
        if (r < ce.len) a.out[(((int64_t)ce.row0 + r) * H + h) * V + col] = f32_to_bf16(O[nt][i]);
      }
    }
    __syncthreads();
  }

  // ---- final state
  if (a.s_out != nullptr) {
#pragma unroll
    for (int m = 0; m < 8; ++m)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const int64_t idx = sbase + (int64_t)(32 * wave + 16 * nt + lc) * K + 16 * m + 4 * lg;
        if (a.state_dtype == KDA_DTYPE_FP32) {
          *reinterpret_cast<f32x4*>(static_cast<float*>(a.s_out) + idx) = Z[m][nt];
        } else {
          u32x2 w;
          w[0] = pack_bf16(Z[m][nt][0], Z[m][nt][1]);
          w[1] = pack_bf16(Z[m][nt][2], Z[m][nt][3]);
          *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(a.s_out) + idx) = w;
        }
      }
  }
}

}  // namespace

hipError_t launch_recur(const RecurArgs& a, hipStream_t s) {
  const int64_t grid = a.N * a.H;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL(recur_kernel, dim3((unsigned)grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace kda
