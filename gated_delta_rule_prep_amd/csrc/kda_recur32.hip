// kda_recur32.hip -- chunk-recurrence kernel for 32-token chunks (gfx950).
//
// The chunk-by-chunk stage of the split the pages describe (P1 §二 2.2) with a
// state step every 32 tokens instead of 16.  The per-step work that does not
// grow with the chunk (converting the state to fp16 for the MFMA operands,
// decaying it, the barrier and the loop and load bookkeeping) is paid half as
// often per token, while the MFMA work per token grows only in the small
// token-by-token products.  Everything else follows the 16-token kernel
// (kda_recur.hip): value columns split over workgroups and waves, the fp32
// state slice in MFMA accumulators, a ring of chunk slots in LDS filled by
// buffer-to-LDS loads, one barrier per chunk, XCD-aware placement.
//
// P1 = blog post "FlashKDA：月之暗面开源的 Kimi Delta Attention 高性能内核".
//
// Per chunk (records from the 32-token prep kernel; Z = chunk-start state):
//   U = T V                       2 token tiles x fp16 MFMA 16x16x32
//   E = U + (-W) Z                fp16 MFMA 16x16x32 chains over the 128 channels
//   O^T = Z^T Qhat^T + E^T Mqk^T  per token tile
//   Z = diag(gam) Z + Kbar^T E    one 16x16x32 per 16 channels (k = the 32 tokens)
// The k-dimension of every token contraction is taken in the order kPermCh
// (lane group g holds tokens 4g..4g+3 and 16+4g..16+4g+3): that is where a
// lane's E accumulators sit, so E converted to fp16 is at once the A operand
// of E^T Mqk^T and the B operand of Kbar^T E; the record stores T and Mqk with
// their columns in the same order.
#include "kda_device.h"
#include "kda_internal.h"
#include "kda_lds_pipe.h"
#include "../../include/kda.h"

namespace kda {
namespace {

constexpr int CC = C32;
constexpr int kRecPieces = REC32_BYTES / 16;   // 1824 16-byte pieces per record
constexpr int kWaves = 4;                      // compute waves
constexpr int kLoaders = 2;                    // loader waves
constexpr int kSlots = kLoaders + 2;           // ring slots: a chunk is issued kSlots - 2 steps ahead
constexpr int kThreads = 64 * (kWaves + kLoaders);
constexpr int kFar = 0x7ffffff0;               // an offset past every descriptor's range: reads 0

template <int NT>
struct Cfg {
  static constexpr int kWaveCols = 16 * NT;             // value columns per wave
  static constexpr int kCols = kWaveCols * kWaves;      // value columns per workgroup
  static constexpr int kTiles = V / kCols;              // workgroups per (sequence, head)
  static constexpr int kRowPieces = kCols / 8;          // 16-byte pieces per value row of the tile
  static constexpr int kValBlocks = CC * kRowPieces / 64;            // 64-piece blocks of values
  static constexpr int kRecBlocks = (kRecPieces + 63) / 64;          // 64-piece blocks of the record
  static constexpr int kSlotBytes = (kValBlocks + kRecBlocks) * 1024;   // one ring slot
  static constexpr int kVal = 0;
  static constexpr int kRec = kValBlocks * 1024;
  static constexpr int kQh = kRec + REC32_QH, kNw = kRec + REC32_NW, kKb = kRec + REC32_KB;
  static constexpr int kTt = kRec + REC32_T, kMt = kRec + REC32_MQK, kGam = kRec + REC32_GAM;
  static_assert(CC * kRowPieces % 64 == 0, "value rows fill whole blocks");
  // the value swizzle p ^ 2 (r % 4) stays inside a row of at least 8 pieces
  static_assert(kRowPieces >= 8, "the value swizzle needs at least 8 pieces (64 columns) per tile row");
  static_assert(kSlots * kSlotBytes <= 159 * 1024, "the ring fits the LDS");
  static_assert(V % kCols == 0, "tile shape");
};

// Chunk j of a sequence: first flattened token row and length (1..32).
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
  const int r = (s >> 4) & 31, p = s & 15;
  if (s < 1024) return 16 * ((s & ~15) | (p ^ (r & 15)));
  if (s < 1536) return 16 * ((s & ~15) | (p ^ (2 * (r & 3))));
  return 16 * s;
}

// Transposing read of the 16 x 16 block of a swizzled token-major 16-bit tile
// (row stride `rowb` bytes, `tile` at the block's first row) whose first column
// is `col`: lane (lc, lg) receives M[4lg..4lg+3][col + lc].  The swizzle
// depends on the row only through r % 4, the same for rows r and 16 + r.
__device__ __forceinline__ s16x4 tr_swz(const char* tile, int rowb, int col, int lane) {
  const int g = lane >> 4, j = lane & 15;
  const int r = 4 * g + (j >> 2);
  const int c = col + 4 * (j & 3);
  const int p = (c >> 3) ^ (2 * (r & 3));
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(tile + r * rowb + 16 * p + 2 * (c & 7)));
}

template <int NT>
struct Ops {
  f16x8 aT[2], am[2];    // T / Mqk row 16t + lc, k-values at the lane's 8 positions
  f16x8 bv[NT];          // V[tokens of the lane][wc + 16nt + lc] (converted from bf16)
  f16x8 aw[2][4], aq[2][4];   // -W, Qhat row 16t + lc, 32-block s at the lane's 8 positions
  f16x8 ak[8];           // Kbar[tokens of the lane][16m + lc]
  f32x2 g2;              // gamma of the rows that this lane hands to its 16-lane row
};

// The 8 k-values of a token-major tile column for a 16x16x32 operand: the
// transposing reads of tokens 0..15 and 16..31 give tokens kPermCh(8 lg + e).
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

template <int NT>
__device__ __forceinline__ void read_ops(Ops<NT>& o, const char* slot, int wc, int lane) {
  using Cf = Cfg<NT>;
  const int lg = lane >> 4, lc = lane & 15;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    o.aT[t] = *reinterpret_cast<const f16x8*>(slot + Cf::kTt + 64 * (16 * t + lc) + 16 * lg);
    o.am[t] = *reinterpret_cast<const f16x8*>(slot + Cf::kMt + 64 * (16 * t + lc) + 16 * lg);
  }
  const int vrow = 2 * Cf::kCols;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
    o.bv[nt] = bf16_to_f16x8(tr_swz(slot + Cf::kVal, vrow, wc + 16 * nt, lane),
                             tr_swz(slot + Cf::kVal + 16 * vrow, vrow, wc + 16 * nt, lane));
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int p = (4 * s + lg) ^ lc;
      o.aw[t][s] = *reinterpret_cast<const f16x8*>(slot + Cf::kNw + 256 * (16 * t + lc) + 16 * p);
      o.aq[t][s] = *reinterpret_cast<const f16x8*>(slot + Cf::kQh + 256 * (16 * t + lc) + 16 * p);
    }
#pragma unroll
  for (int m = 0; m < 8; ++m)
    o.ak[m] = join(tr_swz(slot + Cf::kKb, 2 * K, 16 * m, lane), tr_swz(slot + Cf::kKb + 16 * 2 * K, 2 * K, 16 * m, lane));
  o.g2 = *reinterpret_cast<const f32x2*>(slot + Cf::kGam + 8 * lane);
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

// One chunk step from operands in registers: updates Z and returns the two
// output tiles as O^T (lane (lc, lg): token 16t + lc, value columns 16nt +
// 4lg .. +3 of the wave) in fp32; the caller rounds them a step later.
template <int NT>
__device__ __forceinline__ void compute(f32x4 (&Z)[8][NT], const Ops<NT>& o, f32x4 (&O)[2][NT]) {
  f32x4 E[2][NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      E[t][nt] = mfma_f16_k32(o.aT[t], o.bv[nt], f32x4{0.f, 0.f, 0.f, 0.f});
      O[t][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
  for (int s = 0; s < 4; ++s) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      f16x8 zb;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        zb[i] = (_Float16)Z[2 * s][nt][i];
        zb[4 + i] = (_Float16)Z[2 * s + 1][nt][i];
      }
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        E[t][nt] = mfma_f16_k32(o.aw[t][s], zb, E[t][nt]);
        O[t][nt] = mfma_f16_k32(zb, o.aq[t][s], O[t][nt]);
      }
    }
  }

  // E in fp16, k = tokens in kPermCh order: E^T as an A operand, E as a B operand
  f16x8 eb[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      eb[nt][i] = (_Float16)E[0][nt][i];
      eb[nt][4 + i] = (_Float16)E[1][nt][i];
    }
#pragma unroll
    for (int t = 0; t < 2; ++t) O[t][nt] = mfma_f16_k32(eb[nt], o.am[t], O[t][nt]);
  }

  // Z = diag(gam) Z + Kbar^T E
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    Z[0][nt] = mfma_f16_k32(o.ak[0], eb[nt], decay<0>(Z[0][nt], o.g2));
    Z[1][nt] = mfma_f16_k32(o.ak[1], eb[nt], decay<1>(Z[1][nt], o.g2));
    Z[2][nt] = mfma_f16_k32(o.ak[2], eb[nt], decay<2>(Z[2][nt], o.g2));
    Z[3][nt] = mfma_f16_k32(o.ak[3], eb[nt], decay<3>(Z[3][nt], o.g2));
    Z[4][nt] = mfma_f16_k32(o.ak[4], eb[nt], decay<4>(Z[4][nt], o.g2));
    Z[5][nt] = mfma_f16_k32(o.ak[5], eb[nt], decay<5>(Z[5][nt], o.g2));
    Z[6][nt] = mfma_f16_k32(o.ak[6], eb[nt], decay<6>(Z[6][nt], o.g2));
    Z[7][nt] = mfma_f16_k32(o.ak[7], eb[nt], decay<7>(Z[7][nt], o.g2));
  }
}

template <int NT>
__device__ __forceinline__ void store_out(uint16_t* out, const Rows& pr, int64_t H, int h, int col0, int lc, int lg,
                                          const f32x4 (&o)[2][NT]) {
#pragma unroll
  for (int t = 0; t < 2; ++t)
    if (16 * t + lc < pr.len) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        *reinterpret_cast<u32x2*>(out + ((pr.row0 + 16 * t + lc) * H + h) * V + col0 + 16 * nt + 4 * lg) =
            pack_out(o[t][nt]);
    }
}

template <int NT>
__global__ __launch_bounds__(kThreads) void recur32_kernel(RecurArgs a) {
  using Cf = Cfg<NT>;
  __shared__ __align__(1024) char ring[kSlots * Cf::kSlotBytes];
  const int64_t H = a.H;
  // Nothing is touched (no output, no state) unless the scheduler accepted
  // cu_seqlens.
  if (reinterpret_cast<const WsHeader*>(a.ws)->status & KDA_STATUS_BAD_CU_SEQLENS) return;
  // XCD-aware placement: id b runs on XCD b % 8; the kTiles tiles of pair
  // 8 * g + x get ids 8 * (kTiles * g + tile) + x.
  const int64_t bid = blockIdx.x, x = bid & 7, q = bid >> 3;
  const int64_t pair = 8 * (q / Cf::kTiles) + x;
  const int tile = (int)(q % Cf::kTiles);
  if (pair >= a.N * H) return;
  const int64_t slot_id = pair / H;
  const int h = (int)(pair - slot_id * H);
  const int v0 = tile * Cf::kCols;
  const int32_t* order = reinterpret_cast<const int32_t*>(a.ws + a.lay.order);
  const int n = order[slot_id];
  const SeqEntry se = reinterpret_cast<const SeqEntry*>(a.ws + a.lay.seq_table)[n];
  // Records are chunk-major: record (chunk c, head h) at (c H + h) REC32_BYTES.
  const char* recs = a.ws + a.lay.records + ((int64_t)se.first_chunk * H + h) * REC32_BYTES;
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
    // Chunk c of the launch goes to slot c mod kSlots and belongs to loader
    // c mod kLoaders, which issues it right after barrier c - kSlots + 2 (the
    // compute waves are then done with chunk c - kSlots, the slot's previous
    // contents) and waits for it (vmcnt(0)) just before barrier c.  Its next
    // chunk, c + kLoaders = c + kSlots - 2, is issued only after that wait, so
    // a loader never has more than one chunk in flight and each wait covers
    // exactly that chunk's loads, whatever order loads complete in.
    static_assert(kLoaders == kSlots - 2, "one chunk in flight per loader");
    const int j = wave - kWaves;
    // Source offset of this lane's 16-byte position in each load instruction:
    // value row r, piece position p holds piece p ^ 2 (r % 4) of the row; rows
    // past the end of a partial chunk lie past the descriptor's range and read
    // as zeros (the record gives them zero weight), and so do the record's
    // padding pieces.
    int32_t vsrc[Cf::kValBlocks], rsrc[Cf::kRecBlocks];
#pragma unroll
    for (int i = 0; i < Cf::kValBlocks; ++i) {
      const int s = 64 * i + lane, r = s / Cf::kRowPieces, p = s % Cf::kRowPieces;
      vsrc[i] = r * row_bytes + 16 * (p ^ (2 * (r & 3)));
    }
#pragma unroll
    for (int i = 0; i < Cf::kRecBlocks; ++i) rsrc[i] = rec_source(64 * i + lane);
    const char* vseq = reinterpret_cast<const char*>(a.v + ((int64_t)se.row0 * H + h) * V + v0);
    const uint32_t ring0 = lds_addr(ring);
    const auto issue = [&](int st) {
      const int c = ci_lo + st;
      const int len = min(se.len - CC * c, CC);
      const i32x4 rrec = buf_rsrc(recs + (int64_t)c * H * REC32_BYTES, REC32_BYTES);
      const i32x4 rval = buf_rsrc(vseq + (int64_t)c * CC * row_bytes, (len - 1) * row_bytes + 2 * Cf::kCols);
      const uint32_t slot = ring0 + (uint32_t)((st % kSlots) * Cf::kSlotBytes);
#pragma unroll
      for (int i = 0; i < Cf::kValBlocks; ++i) load_lds16(rval, slot + Cf::kVal + 1024 * i, vsrc[i]);
#pragma unroll
      for (int i = 0; i < Cf::kRecBlocks; ++i) load_lds16(rrec, slot + Cf::kRec + 1024 * i, rsrc[i]);
    };
    for (int c = j; c < min(steps, kSlots - 2); c += kLoaders) issue(c);
    for (int i = 0; i < steps; ++i) {
      const bool mine = i % kLoaders == j;
      if (mine) wait_vmcnt<0>();   // chunk i has landed in its slot
      barrier();
      if (mine && i + kSlots - 2 < steps) issue(i + kSlots - 2);
    }
    return;
  }

  // ---------------- compute wave ----------------
  const int64_t sbase = ((int64_t)n * H + h) * V * K;   // state [n][h][v][k]
  const int wc = Cf::kWaveCols * wave;                   // first tile column of this wave
  const int col0 = v0 + wc;                              // first state column of this wave

  // ---- state slice: Z[m][nt] holds rows 16m + 4lg + i, column col0 + 16nt + lc
  f32x4 Z[8][NT];
#pragma unroll
  for (int m = 0; m < 8; ++m)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int64_t idx = sbase + (int64_t)(col0 + 16 * nt + lc) * K + 16 * m + 4 * lg;
      if (!from_caller) {
        Z[m][nt] = *reinterpret_cast<const f32x4*>(ws_state + idx);
      } else if (a.s_in == nullptr) {
        Z[m][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
      } else if (a.state_dtype == KDA_DTYPE_FP32) {
        Z[m][nt] = *reinterpret_cast<const f32x4*>(static_cast<const float*>(a.s_in) + idx);
      } else {
        const u32x2 w = *reinterpret_cast<const u32x2*>(static_cast<const uint16_t*>(a.s_in) + idx);
        Z[m][nt] = f32x4{bf16_lo(w[0]), bf16_hi(w[0]), bf16_lo(w[1]), bf16_hi(w[1])};
      }
    }

  if (steps > 0) {
    // The output of a step is rounded and stored in the next step, well after
    // the MFMAs that produce it (as in the 16-token kernel: a vector read of an
    // MFMA result shortly after it, with more MFMAs issued in between, is not
    // relied on), and a scheduling barrier keeps each step's instructions on
    // their side of the step barrier.
    f32x4 o_prev[2][NT];
    for (int s = 0; s < steps; ++s) {
      __builtin_amdgcn_sched_barrier(0);
      barrier();
      Ops<NT> ops;
      read_ops<NT>(ops, ring + (s % kSlots) * Cf::kSlotBytes, wc, lane);
      if (s > 0) store_out<NT>(a.out, chunk_rows(se, ci_lo + s - 1), H, h, col0, lc, lg, o_prev);
      compute<NT>(Z, ops, o_prev);
      wait_lgkm0();   // every read of this slot is done before the next barrier
    }
    __builtin_amdgcn_sched_barrier(0);
    store_out<NT>(a.out, chunk_rows(se, ci_hi - 1), H, h, col0, lc, lg, o_prev);
  }

  // ---- state out
  if (!to_caller || a.s_out != nullptr) {
#pragma unroll
    for (int m = 0; m < 8; ++m)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int64_t idx = sbase + (int64_t)(col0 + 16 * nt + lc) * K + 16 * m + 4 * lg;
        if (!to_caller) {
          *reinterpret_cast<f32x4*>(ws_state + idx) = Z[m][nt];
        } else if (a.state_dtype == KDA_DTYPE_FP32) {
          *reinterpret_cast<f32x4*>(static_cast<float*>(a.s_out) + idx) = Z[m][nt];
        } else {
          *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(a.s_out) + idx) = pack_out(Z[m][nt]);
        }
      }
  }
  // an operand beyond the fp16 range (or a non-finite input) leaves the state
  // non-finite: reported in the status word
  flag_nonfinite<8, NT>(Z, &reinterpret_cast<WsHeader*>(a.ws)->status, KDA_STATUS_OVERFLOW);
}

template <int NT>
hipError_t launch_tiles(const RecurArgs& a, hipStream_t s) {
  const int64_t pairs = a.N * a.H;
  const int64_t grid = 8 * Cfg<NT>::kTiles * ((pairs + 7) / 8);
  if (grid > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL((recur32_kernel<NT>), dim3((unsigned)grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

// 64 value columns per workgroup (two workgroups per (sequence, head)); a
// 4-slot ring of 33 KB slots (132 KB).
hipError_t launch_recur32(const RecurArgs& a, hipStream_t s) {
  if (a.N * a.H == 0) return hipSuccess;
  return launch_tiles<1>(a, s);
}

}  // namespace kda
