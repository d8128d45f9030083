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
// Per chunk (records from the prep kernel, Z = chunk-start state, K x V; T,
// Mqk, Kbar^T and V reach their MFMA operand layouts through transposing LDS
// reads of token-major tiles):
//   U = T V                      fp16 MFMA 16x16x16
//   E = U + (-W) Z               fp16 MFMA 16x16x32 chain over the 128 channels
//   O = Qhat Z + Mqk E           fp16 MFMA (E feeds the B operand directly: the
//                                accumulator layout of E is the B-operand layout)
//   Z = diag(gam) Z + Kbar^T E   fp16 MFMA 16x16x16, accumulating onto gam * Z
// Z is converted to fp16 per step for the two products that read it; the state
// itself stays fp32.  The channel order of Qhat / -W in the record matches the
// rows a lane holds in its two accumulator tiles (kPermCh), so the conversion
// needs no lane exchange.
//
// Memory pipeline: the record and the value rows of chunk c+2 are loaded into
// registers while chunk c is computed (two register sets, the loop unrolled by
// two), then written to one of two LDS buffers; one barrier per chunk.  Values
// are staged already in fp16; the output tile goes through LDS so that it
// leaves as 16-byte row stores, one chunk behind.
#include "kda_device.h"
#include "kda_internal.h"
#include "../../include/kda.h"

namespace kda {
namespace {

constexpr int kThreads = 256;
constexpr int kRecPieces = REC_BYTES / 16;   // 864 16-byte pieces per record
constexpr int SO = V + 8;                    // bf16 [16][SO] output tile

// LDS copy of one record plus the chunk's values (converted to fp16), all
// token-major and written as 16-byte rows.  Row strides are chosen per read
// pattern so the lanes of one read fall on distinct banks: 272 B for Qhat and
// -W (16-byte operand reads, one row per lane), 288 B for Kbar and V and 48 B
// for T^T and Mqk^T (transposing reads, four lanes per row).
constexpr int SQ = K + 8;                    // fp16 row stride of Qhat and -W
constexpr int SR = K + 16;                   // fp16 row stride of Kbar and V
constexpr int ST = C + 8;                    // fp16 row stride of T^T and Mqk^T

struct __align__(16) Stage {
  __align__(16) _Float16 qh[C][SQ];
  __align__(16) _Float16 nw[C][SQ];
  __align__(16) _Float16 kb[C][SR];
  __align__(16) _Float16 v[C][SR];
  __align__(16) _Float16 tt[C][ST];
  __align__(16) _Float16 mt[C][ST];
  __align__(16) float gam[K];
};

struct __align__(16) RecurSmem {
  Stage buf[2];
  __align__(16) uint16_t ot[2][C][SO];
};

// One chunk's worth of global data held in registers.
struct Prefetch {
  u32x4 rec[4];
  u32x4 v;
};

// Chunk j of a sequence: first flattened token row and length (1..16).
struct Rows {
  int64_t row0;
  int len;
};
__device__ __forceinline__ Rows chunk_rows(const SeqEntry& se, int j) {
  const int rem = se.len - C * j;
  return Rows{(int64_t)se.row0 + C * j, rem < C ? rem : C};
}

__device__ __forceinline__ f16x4 f16x4_of(f32x4 x) {
  f16x4 r;
  r[0] = (_Float16)x[0]; r[1] = (_Float16)x[1]; r[2] = (_Float16)x[2]; r[3] = (_Float16)x[3];
  return r;
}

// Every load is unconditional (indices clamped into range) so that the
// compiler can count outstanding loads exactly and wait only for the chunk it
// stages, not for the prefetch issued after it.
__device__ __forceinline__ void load_chunk(Prefetch& p, const char* recs, const SeqEntry& se,
                                           const uint16_t* v, int chunk, int64_t H, int h, int tid) {
  chunk = min(chunk, se.nchunks - 1);
  const Rows cr = chunk_rows(se, chunk);
  const char* rec = recs + (int64_t)chunk * REC_BYTES;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int piece = min(tid + kThreads * j, kRecPieces - 1);
    p.rec[j] = *reinterpret_cast<const u32x4*>(rec + 16 * piece);
  }
  const int r = min(tid >> 4, cr.len - 1), c8 = (tid & 15) * 8;
  p.v = *reinterpret_cast<const u32x4*>(v + ((cr.row0 + r) * H + h) * V + c8);
}

// Thread tid stages record pieces tid + 256 j (16 bytes each): j = 0 is a
// piece of Qhat, j = 1 of -W, j = 2 of Kbar, and j = 3 (tid < 96) of T^T,
// Mqk^T or gamma; plus 8 values of token row tid / 16 converted to fp16.
// Value rows past the end of a partial chunk are staged as zeros.
__device__ __forceinline__ void stage_chunk(const Prefetch& p, Stage& st, int len, int tid) {
  const int r16 = tid >> 4, c16 = (tid & 15) * 8;
  *reinterpret_cast<u32x4*>(&st.qh[r16][c16]) = p.rec[0];
  *reinterpret_cast<u32x4*>(&st.nw[r16][c16]) = p.rec[1];
  *reinterpret_cast<u32x4*>(&st.kb[r16][c16]) = p.rec[2];
  if (tid < 32) {
    *reinterpret_cast<u32x4*>(&st.tt[tid >> 1][(tid & 1) * 8]) = p.rec[3];
  } else if (tid < 64) {
    *reinterpret_cast<u32x4*>(&st.mt[(tid - 32) >> 1][(tid & 1) * 8]) = p.rec[3];
  } else if (tid < 96) {
    *reinterpret_cast<u32x4*>(&st.gam[4 * (tid - 64)]) = p.rec[3];
  }
  const bool live = r16 < len;
  u32x4 w;
#pragma unroll
  for (int j = 0; j < 4; ++j) w[j] = live ? pack_f16(bf16_lo(p.v[j]), bf16_hi(p.v[j])) : 0u;
  *reinterpret_cast<u32x4*>(&st.v[r16][c16]) = w;
}

// Output rows of a chunk from the LDS tile: 16 rows x 256 B, 16 B per thread.
__device__ __forceinline__ void store_out(const uint16_t (*ot)[SO], const Rows& cr, uint16_t* out, int64_t H,
                                          int h, int tid) {
  const int r = tid >> 4, c8 = (tid & 15) * 8;
  if (r < cr.len)
    *reinterpret_cast<u32x4*>(out + ((cr.row0 + r) * H + h) * V + c8) =
        *reinterpret_cast<const u32x4*>(&ot[r][c8]);
}

// One chunk step on the staged record: updates Z, writes the output tile.
__device__ __forceinline__ void step(f32x4 (&Z)[8][2], const Stage& st, uint16_t (*ot)[SO], int wave, int lg,
                                     int lc) {
  const int lane = 16 * lg + lc;
  // ---- U = T V
  f32x4 E[2], O[2];
  const f16x4 aT = lds_read_tr(&st.tt[0][0], ST, lane);   // T[lc][4lg..4lg+3]
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const f16x4 bv = lds_read_tr(&st.v[0][32 * wave + 16 * nt], SR, lane);
    E[nt] = mfma_f16_k16(aT, bv, f32x4{0.f, 0.f, 0.f, 0.f});
    O[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // ---- E += (-W) Z ; O = Qhat Z
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const f16x8 aw = *reinterpret_cast<const f16x8*>(&st.nw[lc][32 * s + 8 * lg]);
    const f16x8 aq = *reinterpret_cast<const f16x8*>(&st.qh[lc][32 * s + 8 * lg]);
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
  const f16x4 am = lds_read_tr(&st.mt[0][0], ST, lane);   // Mqk[lc][4lg..4lg+3]
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    eb[nt] = f16x4_of(E[nt]);
    O[nt] = mfma_f16_k16(am, eb[nt], O[nt]);
  }

  // ---- Z = diag(gam) Z + Kbar^T E
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    const f32x4 gm = *reinterpret_cast<const f32x4*>(&st.gam[16 * m + 4 * lg]);
    const f16x4 ak = lds_read_tr(&st.kb[0][16 * m], SR, lane);   // Kbar[4lg..4lg+3][16m + lc]
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) Z[m][nt] = mfma_f16_k16(ak, eb[nt], Z[m][nt] * gm);
  }

  // ---- output tile (rows 4lg + i, columns 32 wave + 16 nt + lc)
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
#pragma unroll
    for (int i = 0; i < 4; ++i) ot[4 * lg + i][32 * wave + 16 * nt + lc] = f32_to_bf16(O[nt][i]);
}

__global__ __launch_bounds__(kThreads) void recur_kernel(RecurArgs a) {
  __shared__ RecurSmem sm;
  const int64_t H = a.H;
  const int64_t slot = blockIdx.x / H;
  const int h = (int)(blockIdx.x - slot * H);
  const int32_t* order = reinterpret_cast<const int32_t*>(a.ws + a.lay.order);
  const int n = order[slot];
  const SeqEntry se = reinterpret_cast<const SeqEntry*>(a.ws + a.lay.seq_table)[n];
  const char* recs = a.ws + a.lay.records + ((int64_t)h * a.lay.max_chunks + se.first_chunk) * REC_BYTES;
  const int nch = se.nchunks;

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

  if (nch > 0) {
    Prefetch pa, pb;
    load_chunk(pa, recs, se, a.v, 0, H, h, tid);
    load_chunk(pb, recs, se, a.v, 1, H, h, tid);
    stage_chunk(pa, sm.buf[0], chunk_rows(se, 0).len, tid);
    __syncthreads();
    // Step ci computes chunk ci from buf[ci & 1].  First the output tile of
    // chunk ci - 1 is stored, then the register set that held chunk ci
    // (already staged) fetches chunk ci + 2 (clamped: past the end it reloads
    // the last chunk, which is never staged); after the compute the other set
    // (chunk ci + 1) is staged into the other buffer.  PCUR / PNEXT swap every
    // step, so the loop is unrolled by two to keep the register sets fixed.
#define KDA_RECUR_STEP(PCUR, PNEXT, B)                                                      \
  if (ci > 0) store_out(sm.ot[(B) ^ 1], chunk_rows(se, ci - 1), a.out, H, h, tid);         \
  load_chunk(PCUR, recs, se, a.v, ci + 2, H, h, tid);                                      \
  step(Z, sm.buf[B], sm.ot[B], wave, lg, lc);                                              \
  if (ci + 1 < nch) stage_chunk(PNEXT, sm.buf[(B) ^ 1], chunk_rows(se, ci + 1).len, tid); \
  __syncthreads();                                                                         \
  if (++ci >= nch) break;
    for (int ci = 0;;) {
      KDA_RECUR_STEP(pa, pb, 0)
      KDA_RECUR_STEP(pb, pa, 1)
    }
#undef KDA_RECUR_STEP
    store_out(sm.ot[(nch - 1) & 1], chunk_rows(se, nch - 1), a.out, H, h, tid);
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
