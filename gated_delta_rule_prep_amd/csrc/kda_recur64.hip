// kda_recur64.hip -- chunk-recurrence kernel for 64-token chunks (gfx950).
//
// The chunk-by-chunk stage of the split the pages describe (P1 §二 2.2) with a
// state step every 64 tokens, the chunk size of Flash Linear Attention that
// P1 §二 2.1 compares its own 16 with.  It follows the 32-token kernel
// (kda_recur32.hip): value columns split over workgroups (64 per workgroup,
// two per (sequence, head)) and compute waves (16 each), the fp32 state slice
// in MFMA accumulators, chunk slots in LDS filled by buffer-to-LDS loads from
// loader waves, one barrier per chunk, XCD-aware placement.  A 64-token slot
// (the 66 KB record and the tile's value rows) leaves room for two slots
// only, so the loaders fetch chunk c + 1 while the compute waves work on c.
//
// P1 = blog post "FlashKDA：月之暗面开源的 Kimi Delta Attention 高性能内核".
//
// Per chunk (records from the 64-token prep kernel; Z = chunk-start state),
// with four 16-token tiles t and two 32-token halves u:
//   E_t = sum_u T_tu V_u + (-W_t) Z   fp16 MFMA 16x16x32 (T is block lower
//                                     triangular: tiles 0, 1 use half 0 only)
//   O_t^T = Z^T Qhat_t^T + sum_u E_u^T Mqk_tu^T
//   Z = diag(gam) Z + sum_u Kbar_u^T E_u
// The k-dimension of every token contraction is taken per half in the order
// kPermCh, where a lane's E accumulators sit, as in the 32-token kernel.
#include "kda_device.h"
#include "kda_internal.h"
#include "kda_lds_pipe.h"
#include "../../include/kda.h"

namespace kda {
namespace {

constexpr int CC = C64;
constexpr int kRecPieces = REC64_BYTES / 16;   // 4128 16-byte pieces per record
constexpr int kWaves = 4;                      // compute waves, 16 value columns each
constexpr int kLoaders = 4;                    // loader waves, each loads every fourth 64-piece block
constexpr int kSlots = 2;                      // ring slots: chunk c + 1 loads while c is computed
constexpr int kThreads = 64 * (kWaves + kLoaders);
constexpr int kFar = 0x7ffffff0;               // an offset past every descriptor's range: reads 0

constexpr int kCols = 16 * kWaves;                            // value columns per workgroup
constexpr int kTiles = V / kCols;                             // workgroups per (sequence, head)
constexpr int kRowPieces = kCols / 8;                         // 16-byte pieces per value row of the tile
constexpr int kValBlocks = CC * kRowPieces / 64;              // 64-piece blocks of values
constexpr int kRecBlocks = (kRecPieces + 63) / 64;            // 64-piece blocks of the record
constexpr int kBlocks = kValBlocks + kRecBlocks;
constexpr int kSlotBytes = kBlocks * 1024;                    // one ring slot
constexpr int kVal = 0;
constexpr int kRec = kValBlocks * 1024;
constexpr int kQh = kRec + REC64_QH, kNw = kRec + REC64_NW, kKb = kRec + REC64_KB;
constexpr int kTt = kRec + REC64_T, kMt = kRec + REC64_MQK, kGam = kRec + REC64_GAM;
static_assert(CC * kRowPieces % 64 == 0, "value rows fill whole blocks");
static_assert(kRowPieces >= 8, "the value swizzle needs at least 8 pieces (64 columns) per tile row");
static_assert(kSlots * kSlotBytes <= 159 * 1024, "the ring fits the LDS");
constexpr int kPerLoader = (kBlocks + kLoaders - 1) / kLoaders;   // 64-piece blocks per loader and chunk
static_assert(kPerLoader <= 60, "a loader's loads of one chunk fit the vmcnt counter");
// The T and Mqk blocks above the diagonal, (t, u) = (0, 1) and (1, 1), hold
// zeros that no step reads: slot blocks left unloaded.
__device__ __forceinline__ bool unread_block(int i) {
  const int tb = (kRec + REC64_T) / 1024, mb = (kRec + REC64_MQK) / 1024;
  return i == tb + 1 || i == tb + 3 || i == mb + 1 || i == mb + 3;
}

// Chunk j of a sequence: first flattened token row and length (1..64).
struct Rows {
  int64_t row0;
  int len;
};
__device__ __forceinline__ Rows chunk_rows(const SeqEntry& se, int j) {
  const int rem = se.len - CC * j;
  return Rows{(int64_t)se.row0 + CC * j, rem < CC ? rem : CC};
}

typedef __attribute__((address_space(3))) s16x4 lds_s16x4_t;

// ---- swizzled slot layout -------------------------------------------------
// Qhat and -W: token row r, 16-byte piece p at piece position p ^ (r % 16) of
// the row.  Kbar and the value tile: piece p of row r at p ^ 2 (r % 4).  T,
// Mqk and gamma are stored as in the record.
__device__ __forceinline__ int rec_source(int s) {
  if (s >= kRecPieces) return kFar;   // padding: reads zeros
  const int r = (s >> 4) & 63, p = s & 15;
  if (s < 2048) return 16 * ((s & ~15) | (p ^ (r & 15)));
  if (s < 3072) return 16 * ((s & ~15) | (p ^ (2 * (r & 3))));
  return 16 * s;
}

// Transposing read of the 16 x 16 block of a swizzled token-major 16-bit tile
// (row stride `rowb` bytes, `tile` at the block's first row, a multiple of 4)
// whose first column is `col`: lane (lc, lg) receives M[4lg..4lg+3][col + lc].
__device__ __forceinline__ s16x4 tr_swz(const char* tile, int rowb, int col, int lane) {
  const int g = lane >> 4, j = lane & 15;
  const int r = 4 * g + (j >> 2);
  const int c = col + 4 * (j & 3);
  const int p = (c >> 3) ^ (2 * (r & 3));
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(tile + r * rowb + 16 * p + 2 * (c & 7)));
}

// The 8 k-values of a token-major tile column for a 16x16x32 operand over one
// 32-token half: the transposing reads of its tokens 0..15 and 16..31 give the
// half's tokens kPermCh(8 lg + e).
__device__ __forceinline__ f16x8 join(s16x4 lo, s16x4 hi) {
  const f16x4 a = __builtin_bit_cast(f16x4, lo), b = __builtin_bit_cast(f16x4, hi);
  return f16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

__device__ __forceinline__ f16x8 bf16_to_f16x8(s16x4 lo, s16x4 hi) {
  f16x8 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r[i] = (_Float16)bf16_to_f32((uint16_t)lo[i]);
    r[4 + i] = (_Float16)bf16_to_f32((uint16_t)hi[i]);
  }
  return r;
}

__device__ __forceinline__ f16x8 lds16(const char* p) { return *reinterpret_cast<const f16x8*>(p); }

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

template <int M>
__device__ __forceinline__ void update(f32x4 (&Z)[8], const char* slot, const f16x8 (&eb)[2], f32x2 g2, int lane) {
  const f16x8 a0 = join(tr_swz(slot + kKb, 2 * K, 16 * M, lane), tr_swz(slot + kKb + 16 * 2 * K, 2 * K, 16 * M, lane));
  const f16x8 a1 = join(tr_swz(slot + kKb + 32 * 2 * K, 2 * K, 16 * M, lane),
                        tr_swz(slot + kKb + 48 * 2 * K, 2 * K, 16 * M, lane));
  Z[M] = mfma_f16_k32(a1, eb[1], mfma_f16_k32(a0, eb[0], decay<M>(Z[M], g2)));
}

// One chunk step on the slot in LDS: updates Z and returns the four output
// tiles as O^T (lane (lc, lg): token 16t + lc, value columns 4lg .. 4lg + 3
// of the wave) in fp32; the caller rounds them a step later.
__device__ __forceinline__ void compute(f32x4 (&Z)[8], const char* slot, int wc, int lane, f32x4 (&O)[4]) {
  const int lg = lane >> 4, lc = lane & 15;
  constexpr int vrow = 2 * kCols;
  f16x8 bv[2];
#pragma unroll
  for (int u = 0; u < 2; ++u)
    bv[u] = bf16_to_f16x8(tr_swz(slot + kVal + 32 * u * vrow, vrow, wc, lane),
                          tr_swz(slot + kVal + (32 * u + 16) * vrow, vrow, wc, lane));
  f32x4 E[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    E[t] = mfma_f16_k32(lds16(slot + kTt + 2 * t * 1024 + 64 * lc + 16 * lg), bv[0], f32x4{0.f, 0.f, 0.f, 0.f});
    if (t >= 2) E[t] = mfma_f16_k32(lds16(slot + kTt + (2 * t + 1) * 1024 + 64 * lc + 16 * lg), bv[1], E[t]);
    O[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    f16x8 zb;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      zb[i] = (_Float16)Z[2 * s][i];
      zb[4 + i] = (_Float16)Z[2 * s + 1][i];
    }
    const int p = 16 * ((4 * s + lg) ^ lc);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      E[t] = mfma_f16_k32(lds16(slot + kNw + 256 * (16 * t + lc) + p), zb, E[t]);
      O[t] = mfma_f16_k32(zb, lds16(slot + kQh + 256 * (16 * t + lc) + p), O[t]);
    }
  }

  // E in fp16, k = the tokens of half u in kPermCh order: E^T as an A
  // operand, E as a B operand
  f16x8 eb[2];
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      eb[u][i] = (_Float16)E[2 * u][i];
      eb[u][4 + i] = (_Float16)E[2 * u + 1][i];
    }
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    O[t] = mfma_f16_k32(eb[0], lds16(slot + kMt + 2 * t * 1024 + 64 * lc + 16 * lg), O[t]);
    if (t >= 2) O[t] = mfma_f16_k32(eb[1], lds16(slot + kMt + (2 * t + 1) * 1024 + 64 * lc + 16 * lg), O[t]);
  }

  // Z = diag(gam) Z + Kbar^T E
  const f32x2 g2 = *reinterpret_cast<const f32x2*>(slot + kGam + 8 * lane);
  update<0>(Z, slot, eb, g2, lane);
  update<1>(Z, slot, eb, g2, lane);
  update<2>(Z, slot, eb, g2, lane);
  update<3>(Z, slot, eb, g2, lane);
  update<4>(Z, slot, eb, g2, lane);
  update<5>(Z, slot, eb, g2, lane);
  update<6>(Z, slot, eb, g2, lane);
  update<7>(Z, slot, eb, g2, lane);
}

__device__ __forceinline__ void store_out(uint16_t* out, const Rows& pr, int64_t H, int h, int col0, int lc, int lg,
                                          const f32x4 (&o)[4]) {
#pragma unroll
  for (int t = 0; t < 4; ++t)
    if (16 * t + lc < pr.len)
      *reinterpret_cast<u32x2*>(out + ((pr.row0 + 16 * t + lc) * H + h) * V + col0 + 4 * lg) = pack_out(o[t]);
}

__global__ __launch_bounds__(kThreads) void recur64_kernel(RecurArgs a) {
  __shared__ __align__(1024) char ring[kSlots * kSlotBytes];
  const int64_t H = a.H;
  // Nothing is touched (no output, no state) unless the scheduler accepted
  // cu_seqlens.
  if (reinterpret_cast<const WsHeader*>(a.ws)->status & KDA_STATUS_BAD_CU_SEQLENS) return;
  // XCD-aware placement: id b runs on XCD b % 8; the kTiles tiles of pair
  // 8 * g + x get ids 8 * (kTiles * g + tile) + x.
  const int64_t bid = blockIdx.x, x = bid & 7, q = bid >> 3;
  const int64_t pair = 8 * (q / kTiles) + x;
  const int tile = (int)(q % kTiles);
  if (pair >= a.N * H) return;
  const int64_t slot_id = pair / H;
  const int h = (int)(pair - slot_id * H);
  const int v0 = tile * kCols;
  const int32_t* order = reinterpret_cast<const int32_t*>(a.ws + a.lay.order);
  const int n = order[slot_id];
  const SeqEntry se = reinterpret_cast<const SeqEntry*>(a.ws + a.lay.seq_table)[n];
  // Records are chunk-major: record (chunk c, head h) at (c H + h) REC64_BYTES.
  const char* recs = a.ws + a.lay.records + ((int64_t)se.first_chunk * H + h) * REC64_BYTES;
  const int nch = se.nchunks;
  // Chunks whose first token row lies in [row_lo, row_hi), with the state
  // handed over between parts as in the 16-token kernel.
  const auto first_at = [&](int64_t row) -> int {
    const int64_t d = row - se.row0;
    return d <= 0 ? 0 : (int)min((d + CC - 1) / CC, (int64_t)nch);
  };
  const int ci_lo = first_at(a.row_lo), ci_hi = first_at(a.row_hi);
  if (nch > 0 ? ci_lo >= ci_hi : a.part != 0) return;
  const int steps = ci_hi - ci_lo;
  const bool from_caller = ci_lo == 0, to_caller = ci_hi == nch;
  float* const ws_state = reinterpret_cast<float*>(a.ws + a.lay.state);

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, lg = lane >> 4, lc = lane & 15;
  const int row_bytes = (int)(H * V * 2);

  if (wave >= kWaves) {
    // ---------------- loader wave ----------------
    // Chunk c of the launch goes to slot c mod 2.  Both loaders issue their
    // blocks of chunk c + 1 right after barrier c (the compute waves are then
    // done with chunk c - 1, the slot's previous contents) and wait for them
    // (vmcnt(0)) just before barrier c + 1.  A loader never has more than one
    // chunk in flight, so each wait covers exactly that chunk's loads,
    // whatever order loads complete in.  Value rows past the end of a partial
    // chunk lie past the descriptor's range and read as zeros (the record
    // gives them zero weight), and so do the record's padding pieces.
    const int j = wave - kWaves;
    const char* vseq = reinterpret_cast<const char*>(a.v + ((int64_t)se.row0 * H + h) * V + v0);
    const uint32_t ring0 = lds_addr(ring);
    // Source offset of this lane's 16-byte position in each of the loader's
    // load instructions (slot blocks j, j + kLoaders, ...): value row r, piece
    // position p holds piece p ^ 2 (r % 4) of the row.
    int32_t off[kPerLoader];
#pragma unroll
    for (int k = 0; k < kPerLoader; ++k) {
      const int i = j + kLoaders * k;
      if (i < kValBlocks) {
        const int s = 64 * i + lane, r = s / kRowPieces, p = s % kRowPieces;
        off[k] = r * row_bytes + 16 * (p ^ (2 * (r & 3)));
      } else {
        off[k] = rec_source(64 * (i - kValBlocks) + lane);
      }
    }
    const auto issue = [&](int st) {
      const int c = ci_lo + st;
      const int len = min(se.len - CC * c, CC);
      const i32x4 rrec = buf_rsrc(recs + (int64_t)c * H * REC64_BYTES, REC64_BYTES);
      const i32x4 rval = buf_rsrc(vseq + (int64_t)c * CC * row_bytes, (len - 1) * row_bytes + 2 * kCols);
      const uint32_t slot = ring0 + (uint32_t)((st % kSlots) * kSlotBytes);
#pragma unroll
      for (int k = 0; k < kPerLoader; ++k) {
        const int i = j + kLoaders * k;
        if (i < kBlocks && !unread_block(i)) load_lds16(i < kValBlocks ? rval : rrec, slot + 1024 * i, off[k]);
      }
    };
    if (steps > 0) issue(0);
    for (int i = 0; i < steps; ++i) {
      wait_vmcnt<0>();   // chunk i has landed in its slot
      barrier();
      if (i + 1 < steps) issue(i + 1);
    }
    return;
  }

  // ---------------- compute wave ----------------
  const int64_t sbase = ((int64_t)n * H + h) * V * K;   // state [n][h][v][k]
  const int wc = 16 * wave;                              // first tile column of this wave
  const int col0 = v0 + wc;                              // first state column of this wave

  // ---- state slice: Z[m] holds rows 16m + 4lg + i, column col0 + lc
  f32x4 Z[8];
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    const int64_t idx = sbase + (int64_t)(col0 + lc) * K + 16 * m + 4 * lg;
    if (!from_caller) {
      Z[m] = *reinterpret_cast<const f32x4*>(ws_state + idx);
    } else if (a.s_in == nullptr) {
      Z[m] = f32x4{0.f, 0.f, 0.f, 0.f};
    } else if (a.state_dtype == KDA_DTYPE_FP32) {
      Z[m] = *reinterpret_cast<const f32x4*>(static_cast<const float*>(a.s_in) + idx);
    } else {
      const u32x2 w = *reinterpret_cast<const u32x2*>(static_cast<const uint16_t*>(a.s_in) + idx);
      Z[m] = f32x4{bf16_lo(w[0]), bf16_hi(w[0]), bf16_lo(w[1]), bf16_hi(w[1])};
    }
  }

  if (steps > 0) {
    // The output of a step is rounded and stored in the next step, well after
    // the MFMAs that produce it (as in the 16-token kernel), and a scheduling
    // barrier keeps each step's instructions on their side of the step barrier.
    f32x4 o_prev[4];
    for (int s = 0; s < steps; ++s) {
      __builtin_amdgcn_sched_barrier(0);
      barrier();
      if (s > 0) store_out(a.out, chunk_rows(se, ci_lo + s - 1), H, h, col0, lc, lg, o_prev);
      compute(Z, ring + (s % kSlots) * kSlotBytes, wc, lane, o_prev);
      wait_lgkm0();   // every read of this slot is done before the next barrier
    }
    __builtin_amdgcn_sched_barrier(0);
    store_out(a.out, chunk_rows(se, ci_hi - 1), H, h, col0, lc, lg, o_prev);
  }

  // ---- state out
  if (!to_caller || a.s_out != nullptr) {
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const int64_t idx = sbase + (int64_t)(col0 + lc) * K + 16 * m + 4 * lg;
      if (!to_caller) {
        *reinterpret_cast<f32x4*>(ws_state + idx) = Z[m];
      } else if (a.state_dtype == KDA_DTYPE_FP32) {
        *reinterpret_cast<f32x4*>(static_cast<float*>(a.s_out) + idx) = Z[m];
      } else {
        *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(a.s_out) + idx) = pack_out(Z[m]);
      }
    }
  }
  // an operand beyond the fp16 range (or a non-finite input) leaves the state
  // non-finite: reported in the status word
  f32x4 Zt[8][1];
#pragma unroll
  for (int m = 0; m < 8; ++m) Zt[m][0] = Z[m];
  flag_nonfinite<8, 1>(Zt, &reinterpret_cast<WsHeader*>(a.ws)->status, KDA_STATUS_OVERFLOW);
}

}  // namespace

// 64 value columns per workgroup (two workgroups per (sequence, head)); a
// 2-slot ring of 73 KB slots (146 KB).
hipError_t launch_recur64(const RecurArgs& a, hipStream_t s) {
  const int64_t pairs = a.N * a.H;
  if (pairs == 0) return hipSuccess;
  const int64_t grid = 8 * kTiles * ((pairs + 7) / 8);
  if (grid > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL(recur64_kernel, dim3((unsigned)grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace kda
