// kda_recur.hip -- chunk-recurrence kernel for gfx950.
//
// The second stage of the split the pages describe (P1 §二 2.2: chunk-by-chunk
// delta-rule recurrence, output projection, rolling state).  The state's value
// columns never interact (every step acts on each value column of the state
// separately), so a (sequence, head) pair is cut into V-tiles, one workgroup
// of four waves per tile, and each wave owns 16 (or, when built for it, 32) of
// the tile's columns.  Nothing is exchanged between workgroups.  The 128 x 16
// fp32 state slice of a wave lives in registers as 8 MFMA accumulator tiles
// for the whole sequence; two workgroups share a pair, so each wave's serial
// per-chunk work is half of what a whole pair would need (see launch_recur).
//
// P1 = blog post "FlashKDA：月之暗面开源的 Kimi Delta Attention 高性能内核".
//
// Per chunk (records from the prep kernel, Z = chunk-start state, K x V; T,
// Mqk, Kbar^T and V reach their MFMA operand layouts through transposing LDS
// reads of token-major tiles):
//   U = T V                      fp16 MFMA 16x16x16
//   E = U + (-W) Z               fp16 MFMA 16x16x32 chain over the 128 channels
//   O^T = Z^T Qhat^T + E^T Mqk^T fp16 MFMA; the same register operands as
//                                O = Qhat Z + Mqk E with A and B swapped, so
//                                each lane ends up with four consecutive value
//                                columns of one token and stores them directly
//   Z = diag(gam) Z + Kbar^T E   fp16 MFMA 16x16x16, accumulating onto gam * Z
// Z is converted to fp16 per step for the two products that read it; the state
// itself stays fp32.  The channel order of Qhat / -W in the record matches the
// rows a lane holds in its two accumulator tiles (kPermCh), so the conversion
// needs no lane exchange.  The decay factors reach the lanes by DPP row
// broadcast from a permuted copy of gamma (kGamSlot): two LDS words per lane
// instead of 32.
//
// Memory pipeline: a ring of kDepth chunk slots in LDS, filled by direct
// buffer-to-LDS loads (buffer_load_dwordx4 ... lds) issued kDepth - 1 chunks
// ahead, so no VGPRs or LDS write instructions are spent on staging and up to
// kDepth - 1 chunks are in flight from HBM.  Each slot holds the tile's value
// rows (raw bf16) and the chunk record.  Every 16-byte piece of a slot may come
// from any 16-byte piece of HBM, so the pieces are stored XOR-swizzled by row
// (rather than padded), which keeps the operand reads free of bank conflicts.
// One barrier per chunk: a wave waits for its own loads of the chunk (vmcnt),
// then the barrier makes every wave's loads visible, and only then is the slot
// of the previous chunk (read by every wave before the barrier) refilled.
//
// Work placement: consecutive workgroup ids go round-robin to the 8 XCDs, and
// the V-tiles of one pair are given ids that land on the same XCD, so the
// pair's records come from HBM once per XCD L2 rather than once per tile.
#include "kda_device.h"
#include "kda_internal.h"
#include "kda_lds_pipe.h"
#include "kda_step16.h"
#include "../../include/kda.h"

namespace kda {
namespace {

constexpr int kRecPieces = REC_BYTES / 16;   // 864 16-byte pieces per record

// NT: 16-column MFMA tiles per wave; D: ring depth; W: waves per workgroup.
template <int NT, int D, int W>
struct Cfg {
  static constexpr int kWaves = W;
  static constexpr int kThreads = 64 * W;
  static constexpr int kWaveCols = 16 * NT;             // value columns per wave
  static constexpr int kCols = kWaveCols * W;           // value columns per workgroup
  static constexpr int kTiles = V / kCols;              // workgroups per (sequence, head)
  static constexpr int kRowPieces = kCols / 8;          // 16-byte pieces per value row of the tile
  static constexpr int kValBlocks = C * kRowPieces / 64;             // 64-piece blocks of values
  static constexpr int kBlocks = kValBlocks + (kRecPieces + 63) / 64;   // 1 KB blocks of a slot
  static constexpr int kMaxLoads = (kBlocks + W - 1) / W;   // load instructions per wave per chunk (at most)
  static constexpr bool kEven = kBlocks % W == 0;           // every wave issues kMaxLoads
  static constexpr int kSlotBytes = kBlocks * 1024;     // one ring slot
  // byte offsets of the fields inside a slot
  static constexpr int kVal = 0;
  static constexpr int kRec = kValBlocks * 1024;
  static_assert(C * kRowPieces % 64 == 0, "value rows fill whole blocks");
  // The value rows are swizzled as piece p ^ 2 (r % 4) (see make_plan): with
  // fewer than 8 pieces per row that index leaves the tile, and for the last
  // tile of the last head it reads past the end of v (a 32-column build did,
  // and faulted).  So tiles are at least 64 columns wide.
  static_assert(kRowPieces >= 8, "the value swizzle needs at least 8 pieces (64 columns) per tile row");
  static_assert(D >= 3 && (D - 2) * kMaxLoads <= 63, "ring depth within the vmcnt range");
  static_assert(V % kCols == 0, "tile shape");
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

// ---- swizzled slot layout -------------------------------------------------
// Qhat and -W: token row r, 16-byte piece p (8 channels in record order) at
// piece position p ^ r of the row.  Kbar and the value tile: piece p of row r
// at position p ^ 2 (r % 4).  T^T, Mqk^T and gamma are stored as in the record.

// Byte offset (within the record) of the piece that record piece position `s`
// of a slot holds.
__device__ __forceinline__ int rec_source(int s) {
  if (s >= kRecPieces) return 0;   // padding: any valid piece
  const int r = (s >> 4) & 15, p = s & 15;
  if (s < 512) return 16 * ((s & ~15) | (p ^ r));
  if (s < 768) return 16 * ((s & ~15) | (p ^ (2 * (r & 3))));
  return 16 * s;
}

// Where this lane's load instruction j of a chunk reads from.  Slot block
// b = W j + wave (64 pieces, one per lane); blocks below kValBlocks hold the
// value tile, the rest the record.
template <int NT, int D, int W>
struct LoadPlan {
  int32_t off[Cfg<NT, D, W>::kMaxLoads];   // record byte offset, or value byte offset within the token row
  int32_t row[Cfg<NT, D, W>::kMaxLoads];   // value blocks: byte offset of the piece within the chunk's rows
};

template <int NT, int D, int W>
__device__ __forceinline__ void make_plan(LoadPlan<NT, D, W>& pl, int wave, int lane, int row_bytes) {
  using Cf = Cfg<NT, D, W>;
#pragma unroll
  for (int j = 0; j < Cf::kMaxLoads; ++j) {
    const int b = W * j + wave;
    if (b < Cf::kValBlocks) {
      const int s = 64 * b + lane, r = s / Cf::kRowPieces, p = s % Cf::kRowPieces;
      pl.off[j] = 16 * (p ^ (2 * (r & 3)));
      pl.row[j] = r * row_bytes + pl.off[j];
    } else {
      pl.row[j] = 0;
      pl.off[j] = rec_source(64 * (b - Cf::kValBlocks) + lane);
    }
  }
}

// Issue the loads of chunk min(c, clast) into the ring slot at LDS address
// `slot_lds` (all lanes, no waits); clast is the last chunk of the part, so
// loads never run ahead into records that the next part's prep may still be
// writing.  `vseq` is the sequence's first value row at this tile's first
// column; everything but the per-lane offsets of the load plan is
// wave-uniform, so the per-chunk bookkeeping stays in scalar registers.
// Value rows past the end of a partial chunk repeat the last row: the
// record gives them zero weight (their T rows and columns and their -W, Qhat
// and Kbar rows are exactly zero), so any finite values are harmless.
template <int NT, int D, int W>
__device__ __forceinline__ void issue_chunk(uint32_t slot_lds, const LoadPlan<NT, D, W>& pl, const char* recs,
                                            const char* vseq, const SeqEntry& se, int c, int clast, int row_bytes,
                                            int wave) {
  using Cf = Cfg<NT, D, W>;
  c = min(c, clast);
  const int len = min(se.len - C * c, C);
  const i32x4 rrec = buf_rsrc(recs + (int64_t)c * REC_BYTES, REC_BYTES);
  const i32x4 rval = buf_rsrc(vseq + (int64_t)c * C * row_bytes, C * row_bytes);
  const int last = (len - 1) * row_bytes;   // byte offset of the chunk's last value row
#pragma unroll
  for (int j = 0; j < Cf::kMaxLoads; ++j) {
    const int b = W * j + wave;   // wave-uniform
    if (b >= Cf::kBlocks) break;
    if (b < Cf::kValBlocks) {
      load_lds16(rval, slot_lds + 1024 * b, min(pl.row[j], last + pl.off[j]));
    } else {
      load_lds16(rrec, slot_lds + 1024 * b, pl.off[j]);
    }
  }
}

// Wait until this wave's loads of chunk ci have landed: at most the loads of
// the D - 2 later chunks may still be in flight (loads complete in issue
// order; the output stores, also counted, only make the wait stricter).
template <int NT, int D, int W>
__device__ __forceinline__ void wait_chunk(int wave) {
  using Cf = Cfg<NT, D, W>;
  if constexpr (Cf::kEven) {
    wait_vmcnt<(D - 2) * Cf::kMaxLoads>();
  } else {
    if (wave < Cf::kBlocks % W) wait_vmcnt<(D - 2) * Cf::kMaxLoads>();
    else wait_vmcnt<(D - 2) * (Cf::kMaxLoads - 1)>();
  }
}

template <int NT, int D, int W, int PV>
__global__ __launch_bounds__(64 * W) void recur_kernel(RecurArgs a) {
  using Cf = Cfg<NT, D, W>;
  __shared__ __align__(1024) char ring[D][Cf::kSlotBytes];
  const int64_t H = a.H;
  // XCD-aware placement: id b runs on XCD b % 8; the kTiles tiles of pair
  // 8 * g + x get ids 8 * (kTiles * g + tile) + x.
  const int64_t bid = blockIdx.x, x = bid & 7, q = bid >> 3;
  const int64_t pairs = a.N * H, pair2 = 8 * (q / Cf::kTiles) + x;
  const int tile = (int)(q % Cf::kTiles);
  if (pair2 >= (a.sets == 2 ? 2 * pairs : pairs)) return;
  const bool alt = pair2 >= pairs;   // the second set: the transition (zero values, identity start)
  const int64_t pair = alt ? pair2 - pairs : pair2;
  uint16_t* const outp = alt ? nullptr : a.out;
  const void* const s_in = alt ? nullptr : a.s_in;
  void* const s_out = alt ? static_cast<void*>(a.s_out2) : a.s_out;   // (alt: written below as fp16)
  const int sdt = alt ? KDA_DTYPE_FP32 : a.state_dtype;
  if (reinterpret_cast<const WsHeader*>(a.ws)->path == KDA_PATH_FUSED) return;   // the fused kernel runs instead
  const int64_t slot_id = pair / H;
  const int h = (int)(pair - slot_id * H);
  const int v0 = tile * Cf::kCols;
  const int32_t* order = reinterpret_cast<const int32_t*>(a.ws + a.lay.order);
  const int n = order[slot_id];
  const SeqEntry se = reinterpret_cast<const SeqEntry*>(a.ws + a.lay.seq_table)[n];
  const char* recs = a.ws + a.lay.records + ((int64_t)h * a.lay.max_chunks + se.first_chunk) * REC_BYTES;
  const int nch = se.nchunks;
  // This launch covers the chunks whose first token row lies in [row_lo,
  // row_hi): chunks ci_lo .. ci_hi - 1 of the sequence.  The state comes from
  // the caller's initial state when the part starts the sequence, otherwise
  // from the previous part (fp32 in the workspace), and goes to the caller's
  // final state when the part ends the sequence, otherwise to the next part.
  // An empty sequence passes its state through in part 0.
  const auto first_at = [&](int64_t row) -> int {
    const int64_t d = row - se.row0;
    return d <= 0 ? 0 : (int)min((d + C - 1) / C, (int64_t)nch);
  };
  const int ci_lo = first_at(a.row_lo), ci_hi = first_at(a.row_hi);
  if (nch > 0 ? ci_lo >= ci_hi : a.part != 0) return;
  const bool from_caller = ci_lo == 0, to_caller = ci_hi == nch;
  float* const ws_state = reinterpret_cast<float*>(a.ws + a.lay.state);

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, lg = lane >> 4, lc = lane & 15;
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
      } else if (alt) {   // stored [v][k] = (v == k); this lane holds k = 16 m + 4 lg + i, v = col0 + 16 nt + lc
        const int kv = col0 + 16 * nt + lc - 16 * m - 4 * lg;
        Z[m][nt] = f32x4{kv == 0 ? 1.f : 0.f, kv == 1 ? 1.f : 0.f, kv == 2 ? 1.f : 0.f, kv == 3 ? 1.f : 0.f};
      } else if (s_in == nullptr) {
        Z[m][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
      } else if (sdt == KDA_DTYPE_FP32) {
        Z[m][nt] = *reinterpret_cast<const f32x4*>(static_cast<const float*>(s_in) + idx);
      } else {
        const u32x2 w = *reinterpret_cast<const u32x2*>(static_cast<const uint16_t*>(s_in) + idx);
        Z[m][nt] = f32x4{bf16_lo(w[0]), bf16_hi(w[0]), bf16_lo(w[1]), bf16_hi(w[1])};
      }
    }

  if (ci_lo < ci_hi) {
    const int row_bytes = (int)(H * V * 2);
    LoadPlan<NT, D, W> pl;
    make_plan<NT, D, W>(pl, wave, lane, row_bytes);
    const int clast = ci_hi - 1;
    const char* vseq = reinterpret_cast<const char*>(a.v + ((int64_t)se.row0 * H + h) * V + v0);
    const uint32_t ring0 = (uint32_t)reinterpret_cast<uintptr_t>((lds_void*)ring[0]);
    // Output rows of a full chunk: a wave-uniform base per chunk plus this
    // lane's fixed offset (token lc, columns 16 nt + 4 lg .. +3).
    uint16_t* const out_seq = outp + ((int64_t)se.row0 * H + h) * V + col0;
    const int64_t out_chunk = (int64_t)C * H * V;
    const int out_lane = (int)((lc * H) * V) + 4 * lg;
    // Chunks ci_lo .. ci_lo + D-2 in flight before the first step.  Loads past
    // the part's last chunk repeat it into slots that are never read.
#pragma unroll
    for (int c = 0; c < D - 1; ++c)
      issue_chunk<NT, D, W>(ring0 + c * Cf::kSlotBytes, pl, recs, vseq, se, ci_lo + c, clast, row_bytes, wave);
    u32x2 o_prev[NT];
    int slot = 0;   // ring slot of chunk ci
    for (int ci = ci_lo; ci < ci_hi; ++ci) {
      // At most the D - 2 chunks issued after chunk ci may still be in flight
      // (loads complete in issue order); the output stores of the step
      // before, also counted, have had a whole step to complete.
      wait_chunk<NT, D, W>(wave);
      wait_lgkm0();
      barrier();
      // Every wave is done with chunk ci - 1, whose slot is refilled now, and
      // every wave's loads of chunk ci have landed.
      const int refill = slot == 0 ? D - 1 : slot - 1;
      issue_chunk<NT, D, W>(ring0 + refill * Cf::kSlotBytes, pl, recs, vseq, se, ci + D - 1, clast, row_bytes, wave);
      if (ci > ci_lo && outp != nullptr) {   // output of chunk ci - 1, a full chunk (only a sequence's last chunk is partial)
        uint16_t* const ob = out_seq + (int64_t)(ci - 1) * out_chunk;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) *reinterpret_cast<u32x2*>(ob + out_lane + 16 * nt) = o_prev[nt];
      }
      Ops<NT> ops;
      read_ops<NT>(ops, ring[slot] + Cf::kRec, ring[slot] + Cf::kVal, 2 * Cf::kCols, wc, lane);
      if (alt) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) ops.v[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
      compute<NT, PV>(Z, ops, o_prev);
      slot = slot == D - 1 ? 0 : slot + 1;
    }
    wait_vmcnt<0>();   // no load into the ring outlives the workgroup
    const Rows pr = chunk_rows(se, clast);
    if (lc < pr.len && outp != nullptr) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        *reinterpret_cast<u32x2*>(outp + ((pr.row0 + lc) * H + h) * V + col0 + 16 * nt + 4 * lg) = o_prev[nt];
    }
  }

  // ---- state out
  if (!to_caller || s_out != nullptr) {
#pragma unroll
    for (int m = 0; m < 8; ++m)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int64_t idx = sbase + (int64_t)(col0 + 16 * nt + lc) * K + 16 * m + 4 * lg;
        if (!to_caller) {
          *reinterpret_cast<f32x4*>(ws_state + idx) = Z[m][nt];
        } else if (alt) {   // the transition, fp16 in math layout [k][v]
          uint16_t* const at = a.s_out2 + sbase + (int64_t)(16 * m + 4 * lg) * V + col0 + 16 * nt + lc;
#pragma unroll
          for (int i = 0; i < 4; ++i) at[i * V] = __builtin_bit_cast(uint16_t, (_Float16)Z[m][nt][i]);
        } else if (sdt == KDA_DTYPE_FP32) {
          *reinterpret_cast<f32x4*>(static_cast<float*>(s_out) + idx) = Z[m][nt];
        } else {
          u32x2 w;
          w[0] = pack_bf16(Z[m][nt][0], Z[m][nt][1]);
          w[1] = pack_bf16(Z[m][nt][2], Z[m][nt][3]);
          *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(s_out) + idx) = w;
        }
      }
  }
}

// Launches recur_kernel<..., PV> for PV = a.precision, PV running over 0 .. 7.
template <int NT, int D, int W, int PV>
void launch_variant(const RecurArgs& a, int64_t grid, hipStream_t s) {
  if constexpr (PV < 8) {
    if (a.precision == PV) {
      hipLaunchKernelGGL((recur_kernel<NT, D, W, PV>), dim3((unsigned)grid), dim3(64 * W), 0, s, a);
      return;
    }
    launch_variant<NT, D, W, PV + 1>(a, grid, s);
  }
}

template <int NT, int D, int W>
hipError_t launch_tiles(const RecurArgs& a, hipStream_t s) {
  const int64_t pairs = a.N * a.H * (a.sets == 2 ? 2 : 1);
  const int64_t grid = 8 * Cfg<NT, D, W>::kTiles * ((pairs + 7) / 8);
  if (grid > INT32_MAX) return hipErrorInvalidValue;
  // the study's variants (kda_fwd_precision): any combination of the three bits
  if (a.precision < 0 || a.precision > 7) return hipErrorInvalidValue;
  launch_variant<NT, D, W, 0>(a, grid, s);
  return hipGetLastError();
}

}  // namespace

// Value columns per recurrence workgroup: 64.  Each wave takes 16 columns and
// a pair is split over two workgroups, so the per-step VALU work (state
// conversion and decay) and MFMA work of a wave are half of a whole pair's
// and the longest chain of the batch (the critical path) runs twice as fast
// per chunk.  One workgroup of eight 16-column waves per pair (W = 8: each
// record streamed once per pair, two recurrence waves per SIMD) measured
// slower: 0.43 ms against 0.33 at T = 8192, H = 96 fixed, 0.44 against 0.34 on
// the ragged batch, 0.26 against 0.27 at 8 x 1024.  Whole pairs per workgroup (32 columns per wave, NT = 2) read
// each record once instead of twice but measured faster only with many short
// sequences of equal length (3 % at 8 x 1024 tokens, H = 96) and 25 % slower
// with one long sequence among short ones.  A 4-chunk ring (64 KB) covers the
// HBM latency (deeper rings measured no faster).
#ifndef KDA_RECUR_DEPTH
#define KDA_RECUR_DEPTH 4
#endif

hipError_t launch_recur(const RecurArgs& a, hipStream_t s) {
  if (a.lay.chunk == C32) return a.sets == 2 || a.precision != 0 ? hipErrorInvalidValue : launch_recur32(a, s);
  if (a.N * a.H == 0) return hipSuccess;
  return launch_tiles<1, KDA_RECUR_DEPTH, 4>(a, s);
}

}  // namespace kda
