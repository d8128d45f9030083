// kda_recur.hip -- chunk-recurrence kernel for gfx950.
//
// The second stage of the split the pages describe (P1 §二 2.2: chunk-by-chunk
// delta-rule recurrence, output projection, rolling state).  The state's value
// columns never interact (every step acts on each value column of the state
// separately), so a (sequence, head) pair is cut into V-tiles of 32 * NW
// columns, one workgroup of NW waves per tile, and wave w of a tile owns 32 of
// its columns.  Nothing is exchanged between waves or workgroups.  The 128 x 32
// fp32 state slice of a wave lives in registers as 8 x 2 MFMA accumulator tiles
// for the whole sequence.  NW = 4 (one workgroup per pair) when there are
// enough pairs to fill the chip; with few pairs (one long sequence, 64-96
// heads) NW = 2 spreads the same columns over 2 workgroups.
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
// Memory pipeline: the record and the tile's value rows of chunk c+2 are loaded
// into registers while chunk c is computed (two register sets, the loop
// unrolled by two), then written to one of two LDS buffers; one barrier per
// chunk.  Values are staged already in fp16; the output tile goes through LDS
// so that it leaves as 16-byte row stores, one chunk behind.  Every operand of
// a step is read from LDS before its first product, so the LDS latency is paid
// once per step rather than once per product.
//
// Work placement: consecutive workgroup ids go round-robin to the 8 XCDs, and
// the V-tiles of one pair are given ids that land on the same XCD, so the
// pair's records come from HBM once per XCD L2 rather than once per tile.
#include "kda_device.h"
#include "kda_internal.h"
#include "../../include/kda.h"

namespace kda {
namespace {

constexpr int kRecPieces = REC_BYTES / 16;   // 864 16-byte pieces per record
#ifndef KDA_RECUR_DEPTH
#define KDA_RECUR_DEPTH 2
#endif
constexpr int kDepth = KDA_RECUR_DEPTH;      // chunks in flight from HBM

// LDS row strides (fp16 elements), chosen per read pattern so that the lanes
// of one read fall on distinct banks: 272 B for Qhat and -W (16-byte operand
// reads, one row per lane), 288 B for Kbar and 48 B for T^T and Mqk^T
// (transposing reads, four lanes per row, 32 B apart in bank space).
constexpr int SQ = K + 8;
constexpr int SR = K + 16;
constexpr int ST = C + 8;

template <int NW>
struct Tile {
  static constexpr int kThreads = 64 * NW;
  static constexpr int kCols = 32 * NW;                 // value columns per workgroup
  static constexpr int kTiles = V / kCols;              // workgroups per (sequence, head)
  static constexpr int kRecLoads = (kRecPieces + kThreads - 1) / kThreads;
  static constexpr int SV = kCols + 16;                 // value tile stride (transposing reads)
  static constexpr int SO = kCols + 8;                  // bf16 output tile stride
  static_assert(256 % kThreads == 0, "record fields are 256 pieces long");
};

// LDS copy of one record plus the tile's values (converted to fp16), all
// token-major and written as 16-byte rows.
template <int NW>
struct __align__(16) Stage {
  __align__(16) _Float16 qh[C][SQ];
  __align__(16) _Float16 nw[C][SQ];
  __align__(16) _Float16 kb[C][SR];
  __align__(16) _Float16 v[C][Tile<NW>::SV];
  __align__(16) _Float16 tt[C][ST];
  __align__(16) _Float16 mt[C][ST];
  __align__(16) float gam[K];
};

template <int NW>
struct __align__(16) RecurSmem {
  Stage<NW> buf[2];
  __align__(16) uint16_t ot[2][C][Tile<NW>::SO];
};

// One chunk's worth of global data held in registers.
template <int NW>
struct Prefetch {
  u32x4 rec[Tile<NW>::kRecLoads];
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
// stages, not for the prefetch issued after it.  Thread tid loads record
// pieces tid + kThreads * j and one 16-byte piece of the tile's values.
template <int NW>
__device__ __forceinline__ void load_chunk(Prefetch<NW>& p, const char* recs, const SeqEntry& se,
                                           const uint16_t* v, int chunk, int64_t H, int h, int v0, int tid) {
  using Tl = Tile<NW>;
  chunk = min(chunk, se.nchunks - 1);
  const Rows cr = chunk_rows(se, chunk);
  const char* rec = recs + (int64_t)chunk * REC_BYTES;
#pragma unroll
  for (int j = 0; j < Tl::kRecLoads; ++j) {
    const int piece = min(tid + Tl::kThreads * j, kRecPieces - 1);
    p.rec[j] = *reinterpret_cast<const u32x4*>(rec + 16 * piece);
  }
  constexpr int kRowPieces = Tl::kCols / 8;
  const int r = min(tid / kRowPieces, cr.len - 1), c8 = (tid % kRowPieces) * 8;
  p.v = *reinterpret_cast<const u32x4*>(v + ((cr.row0 + r) * H + h) * V + v0 + c8);
}

// Record piece p (16 bytes) to its LDS place: pieces 0-255 are Qhat, 256-511
// -W, 512-767 Kbar (16 pieces per token row), 768-799 T^T, 800-831 Mqk^T and
// 832-863 gamma.  For p < 768 the field is known at compile time after the
// loop below is unrolled (kThreads divides 256).
template <int NW>
__device__ __forceinline__ void stage_chunk(const Prefetch<NW>& p, Stage<NW>& st, int len, int tid) {
  using Tl = Tile<NW>;
#pragma unroll
  for (int j = 0; j < Tl::kRecLoads; ++j) {
    const int first = Tl::kThreads * j;                 // compile-time after unrolling
    if (first < 768) {
      const int field = first >> 8;
      const int loc = (first & 255) + tid, r = loc >> 4, c = (loc & 15) * 8;
      _Float16* dst = field == 0 ? &st.qh[r][c] : field == 1 ? &st.nw[r][c] : &st.kb[r][c];
      *reinterpret_cast<u32x4*>(dst) = p.rec[j];
    } else {
      const int sub = first - 768 + tid;
      if (sub < 32) {
        *reinterpret_cast<u32x4*>(&st.tt[sub >> 1][(sub & 1) * 8]) = p.rec[j];
      } else if (sub < 64) {
        *reinterpret_cast<u32x4*>(&st.mt[(sub - 32) >> 1][(sub & 1) * 8]) = p.rec[j];
      } else if (sub < 96) {
        *reinterpret_cast<u32x4*>(&st.gam[4 * (sub - 64)]) = p.rec[j];
      }
    }
  }
  constexpr int kRowPieces = Tl::kCols / 8;
  const int r = tid / kRowPieces, c8 = (tid % kRowPieces) * 8;
  const bool live = r < len;
  u32x4 w;
#pragma unroll
  for (int j = 0; j < 4; ++j) w[j] = live ? pack_f16(bf16_lo(p.v[j]), bf16_hi(p.v[j])) : 0u;
  *reinterpret_cast<u32x4*>(&st.v[r][c8]) = w;
}

// Output rows of a chunk from the LDS tile: 16 rows x kCols bf16, 16 B per
// thread.
template <int NW>
__device__ __forceinline__ void store_out(const uint16_t (*ot)[Tile<NW>::SO], const Rows& cr, uint16_t* out,
                                          int64_t H, int h, int v0, int tid) {
  constexpr int kRowPieces = Tile<NW>::kCols / 8;
  const int r = tid / kRowPieces, c8 = (tid % kRowPieces) * 8;
  if (r < cr.len)
    *reinterpret_cast<u32x4*>(out + ((cr.row0 + r) * H + h) * V + v0 + c8) =
        *reinterpret_cast<const u32x4*>(&ot[r][c8]);
}

// One chunk step on the staged record: updates Z, writes the output tile.
template <int NW>
__device__ __forceinline__ void step(f32x4 (&Z)[8][2], const Stage<NW>& st, uint16_t (*ot)[Tile<NW>::SO],
                                     int wave, int lg, int lc) {
  constexpr int SV = Tile<NW>::SV;
  const int lane = 16 * lg + lc;

  // ---- every operand of the step, read before the first product
  const f16x4 aT = lds_read_tr(&st.tt[0][0], ST, lane);   // T[lc][4lg..4lg+3]
  const f16x4 am = lds_read_tr(&st.mt[0][0], ST, lane);   // Mqk[lc][4lg..4lg+3]
  f16x4 bv[2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) bv[nt] = lds_read_tr(&st.v[0][32 * wave + 16 * nt], SV, lane);
  f16x8 aw[4], aq[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    aw[s] = *reinterpret_cast<const f16x8*>(&st.nw[lc][32 * s + 8 * lg]);
    aq[s] = *reinterpret_cast<const f16x8*>(&st.qh[lc][32 * s + 8 * lg]);
  }
  f16x4 ak[8];
  f32x4 gm[8];
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    ak[m] = lds_read_tr(&st.kb[0][16 * m], SR, lane);     // Kbar[4lg..4lg+3][16m + lc]
    gm[m] = *reinterpret_cast<const f32x4*>(&st.gam[16 * m + 4 * lg]);
  }

  // ---- U = T V ; E = U + (-W) Z ; O = Qhat Z
  f32x4 E[2], O[2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    E[nt] = mfma_f16_k16(aT, bv[nt], f32x4{0.f, 0.f, 0.f, 0.f});
    O[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int s = 0; s < 4; ++s) {
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      f16x8 zb;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        zb[i] = (_Float16)Z[2 * s][nt][i];
        zb[4 + i] = (_Float16)Z[2 * s + 1][nt][i];
      }
      E[nt] = mfma_f16_k32(aw[s], zb, E[nt]);
      O[nt] = mfma_f16_k32(aq[s], zb, O[nt]);
    }
  }

  // ---- O += Mqk E
  f16x4 eb[2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    eb[nt] = f16x4_of(E[nt]);
    O[nt] = mfma_f16_k16(am, eb[nt], O[nt]);
  }

  // ---- Z = diag(gam) Z + Kbar^T E
#pragma unroll
  for (int m = 0; m < 8; ++m)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) Z[m][nt] = mfma_f16_k16(ak[m], eb[nt], Z[m][nt] * gm[m]);

  // ---- output tile (rows 4lg + i, columns 32 wave + 16 nt + lc)
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
#pragma unroll
    for (int i = 0; i < 4; ++i) ot[4 * lg + i][32 * wave + 16 * nt + lc] = f32_to_bf16(O[nt][i]);
}

template <int NW>
__global__ __launch_bounds__(64 * NW) void recur_kernel(RecurArgs a) {
  using Tl = Tile<NW>;
  __shared__ RecurSmem<NW> sm;
  const int64_t H = a.H;
  // XCD-aware placement: id b runs on XCD b % 8; the kTiles tiles of pair
  // 8 * g + x get ids 8 * (kTiles * g + tile) + x.
  const int64_t b = blockIdx.x, x = b & 7, q = b >> 3;
  const int64_t pair = 8 * (q / Tl::kTiles) + x;
  const int tile = (int)(q % Tl::kTiles);
  if (pair >= a.N * H) return;
  const int64_t slot = pair / H;
  const int h = (int)(pair - slot * H);
  const int v0 = tile * Tl::kCols;
  const int32_t* order = reinterpret_cast<const int32_t*>(a.ws + a.lay.order);
  const int n = order[slot];
  const SeqEntry se = reinterpret_cast<const SeqEntry*>(a.ws + a.lay.seq_table)[n];
  const char* recs = a.ws + a.lay.records + ((int64_t)h * a.lay.max_chunks + se.first_chunk) * REC_BYTES;
  const int nch = se.nchunks;

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, lg = lane >> 4, lc = lane & 15;
  const int64_t sbase = ((int64_t)n * H + h) * V * K;   // state [n][h][v][k]
  const int col0 = v0 + 32 * wave;                      // first state column of this wave

  // ---- state slice: Z[m][nt] holds rows 16m + 4lg + i, column col0 + 16nt + lc
  f32x4 Z[8][2];
#pragma unroll
  for (int m = 0; m < 8; ++m)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const int64_t idx = sbase + (int64_t)(col0 + 16 * nt + lc) * K + 16 * m + 4 * lg;
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
    // kDepth register sets: step ci computes chunk ci from LDS buffer ci & 1
    // while set ci % kDepth, whose chunk is already staged, fetches chunk
    // ci + kDepth (clamped: past the end it reloads the last chunk, which is
    // never staged).  First the output tile of chunk ci - 1 is stored; after
    // the compute, set (ci + 1) % kDepth is staged into the other buffer.  The
    // loop is unrolled by 2 * kDepth so that every set and buffer index is a
    // compile-time constant.
    Prefetch<NW> pf[kDepth];
#pragma unroll
    for (int j = 0; j < kDepth; ++j) load_chunk<NW>(pf[j], recs, se, a.v, j, H, h, v0, tid);
    stage_chunk<NW>(pf[0], sm.buf[0], chunk_rows(se, 0).len, tid);
    __syncthreads();
    for (int ci = 0;;) {
#pragma unroll
      for (int u = 0; u < 2 * kDepth; ++u) {
        const int cur = u % kDepth, nxt = (u + 1) % kDepth, B = u & 1;
        if (ci > 0) store_out<NW>(sm.ot[B ^ 1], chunk_rows(se, ci - 1), a.out, H, h, v0, tid);
        load_chunk<NW>(pf[cur], recs, se, a.v, ci + kDepth, H, h, v0, tid);
        step<NW>(Z, sm.buf[B], sm.ot[B], wave, lg, lc);
        if (ci + 1 < nch) stage_chunk<NW>(pf[nxt], sm.buf[B ^ 1], chunk_rows(se, ci + 1).len, tid);
        __syncthreads();
        if (++ci >= nch) goto chunks_done;
      }
    }
  chunks_done:
    store_out<NW>(sm.ot[(nch - 1) & 1], chunk_rows(se, nch - 1), a.out, H, h, v0, tid);
  }

  // ---- final state
  if (a.s_out != nullptr) {
#pragma unroll
    for (int m = 0; m < 8; ++m)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const int64_t idx = sbase + (int64_t)(col0 + 16 * nt + lc) * K + 16 * m + 4 * lg;
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

template <int NW>
hipError_t launch_nw(const RecurArgs& a, hipStream_t s) {
  const int64_t pairs = a.N * a.H;
  const int64_t grid = 8 * Tile<NW>::kTiles * ((pairs + 7) / 8);
  hipLaunchKernelGGL(recur_kernel<NW>, dim3((unsigned)grid), dim3(Tile<NW>::kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

// Waves per workgroup from the number of (sequence, head) pairs: one
// workgroup per pair while that fills the 256 CUs, otherwise the value
// columns are split over 2 workgroups per pair.  (Four single-wave workgroups
// per pair measured slower at 96 pairs: each of them stages the whole record.)
int recur_waves_per_group(int64_t pairs) {
#ifdef KDA_RECUR_FORCE_NW
  (void)pairs;
  return KDA_RECUR_FORCE_NW;
#else
  return pairs >= 256 ? 4 : 2;
#endif
}

hipError_t launch_recur(const RecurArgs& a, hipStream_t s) {
  const int64_t pairs = a.N * a.H;
  if (pairs == 0) return hipSuccess;
  switch (recur_waves_per_group(pairs)) {
    case 2: return launch_nw<2>(a, s);
    default: return launch_nw<4>(a, s);
  }
}

}  // namespace kda
