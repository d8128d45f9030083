// kda_recur.hip -- chunk-recurrence kernel for gfx950.
//
// The second stage of the split the pages describe (P1 §二 2.2: chunk-by-chunk
// delta-rule recurrence, output projection, rolling state).  The state's value
// columns never interact (every step acts on each value column of the state
// separately), so a (sequence, head) pair is cut into value tiles of 32, 64 or
// 128 columns, one workgroup per tile, and nothing is exchanged between
// workgroups.
//
// P1 = blog post "FlashKDA：月之暗面开源的 Kimi Delta Attention 高性能内核".
//
// Per chunk (records from the prep kernel, Z = chunk-start state, K x V), on
// the 16-column state slice of each compute wave (kda_step16.h):
//   R = V + (-Khat) Z              fp16 MFMA 16x16x32 chain over the channels
//   E = T R                        fp16 MFMA 16x16x16
//   O^T = Z^T Qhat^T + E^T Mqk^T   fp16 MFMA (each lane ends up with four
//                                  consecutive value columns of one token)
//   Z = diag(gam) Z + Kbar^T E     fp16 MFMA 16x16x16 onto the decayed state
// with the state itself in fp32 registers for the whole sequence.
//
// Workgroup = compute waves (16 value columns each) + kLoaders loader waves.
//   * Loader waves own every load.  Chunk c of the launch belongs to loader
//     c mod kLoaders, which streams the chunk's record (13.8 KB) and the
//     tile's value rows into LDS slot c mod kSlots (kSlots = kLoaders + 2)
//     with buffer-to-LDS loads and waits for them (vmcnt(0)) before it
//     reports the chunk.  A loader issues its next chunk only after that
//     wait, so it never has more than one chunk in flight and each wait
//     covers exactly the loads of that chunk, whatever order loads complete in.
//   * Compute waves read the step's operands from the slot (with fixed
//     per-lane addresses plus immediates: the slot pads rows instead of
//     swizzling them -- Qhat and -Khat rows 272 bytes apart, Kbar rows 288,
//     value rows 2 x columns + 32 -- which also keeps the 16-byte and
//     transposing 8-byte reads on distinct banks) and run the step.  They
//     issue no loads and keep no load bookkeeping, so their instruction
//     stream is the step itself (18 MFMA, 32 decay multiplies, 20 fp16
//     conversions, 20 LDS reads and little else).
//   * How they meet.  Four or more compute waves with a CU to themselves:
//     through flags in LDS.  A loader sets the slot's ready word to c + 1
//     once chunk c has landed; a compute wave waits for it, and sets its own
//     done word to s + 1 once its reads of step s are over; a loader refills
//     a slot when every compute wave is done with the slot's previous chunk.
//     The compute waves then drift apart within the ring instead of issuing
//     their record reads at the same moment.  Otherwise (two compute waves,
//     or two workgroups sharing a CU, where the flags measured no faster):
//     one workgroup barrier per step, loads issued kSlots - 2 steps ahead.
//
// What a step costs on MI355X (measured with probes shaped like this kernel,
// 192 workgroups, 512 steps): the chain of one 16-column wave alone issues
// one instruction per 4 cycles and takes 0.24 us; reading the 13 KB of
// operands from LDS adds 0.17 us when four waves read them at once (every wave
// needs the whole record; about 128 B per clock of LDS reads), and the
// loaders' LDS writes a little more.  So a CU's step time grows with the
// number of waves that read each record: 0.41 us per step with two compute
// waves (32-column tiles) against 0.60 us with four (64-column tiles) meeting
// at a barrier every step, 0.57 through the flags.  Waves
// of 32 columns each (half the reads per column) double each wave's issue
// time and measured slower.
//
// Tiles (recur_tiles): 32 columns while four tiles per pair still give one
// workgroup per CU, else 64, else (equal lengths and many pairs: throughput,
// not the longest chain, decides) 128.  Work placement: consecutive workgroup
// ids go round-robin to the 8 XCDs, and the tiles of one pair get ids on the
// same XCD, so the pair's records come from HBM once per L2 rather than once
// per tile.
#include "kda_device.h"
#include "kda_internal.h"
#include "kda_lds_pipe.h"
#include "kda_step16.h"
#include "../../include/kda.h"

namespace kda {
namespace {

// ---- LDS slot layout --------------------------------------------------------
// 16-byte positions: the tile's value rows first (row stride kValStride), then
// the record fields at padded row strides; each region a whole number of
// 64-position load instructions.  Offsets in bytes within the record region:
constexpr int kQkStride = 2 * K + 16;                // Qhat / -Khat row stride
constexpr int kKbStride = 2 * K + 32;                // Kbar row stride
constexpr int kSlotQh = 0;                           // Qhat  [16][272]
constexpr int kSlotNk = C * kQkStride;               // -Khat [16][272]
constexpr int kSlotKb = 2 * C * kQkStride;           // Kbar  [16][288]
constexpr int kSlotTail = kSlotKb + C * kKbStride;   // T^T, Mqk^T, gamma as in the record
constexpr int kRecRegion = kSlotTail + (REC_BYTES - REC_T);
constexpr int kRecLoads = (kRecRegion / 16 + 63) / 64;   // load instructions of the record region
constexpr int kFar = 0x7ffffff0;                     // an offset past every descriptor's range: reads 0
static_assert(REC_NK == REC_QH + C * 2 * K && REC_KB == REC_NK + C * 2 * K && REC_T == REC_KB + C * 2 * K,
              "Qhat, -Khat and Kbar are three consecutive [16][128] fp16 arrays");
static_assert(REC_MQK == REC_T + 512 && REC_GAM == REC_MQK + 512 && REC_BYTES == REC_GAM + 512,
              "T^T, Mqk^T and gamma end the record");

// WC compute waves of 16 value columns each, LD loader waves.
template <int WC, int LD>
struct Tile {
  static constexpr int kLoaders = LD;
  static constexpr int kSlots = kLoaders + 2;            // the loads of a chunk are issued kSlots - 2 steps ahead
  static constexpr int kThreads = 64 * (WC + kLoaders);
  static constexpr int kCols = 16 * WC;                   // value columns per workgroup
  static constexpr int kTiles = V / kCols;                // workgroups per (sequence, head)
  static constexpr int kValStride = 2 * kCols + 32;
  static constexpr int kRowPieces = kCols / 8;            // 16-byte pieces per value row
  static constexpr int kValPos = (C * kValStride / 16 + 63) / 64 * 64;
  static constexpr int kValLoads = kValPos / 64;
  static constexpr int kRecBase = 16 * kValPos;           // record region within a slot
  static constexpr int kSlotBytes = kRecBase + 64 * 16 * kRecLoads;
  static_assert(kSlots * kSlotBytes <= 159 * 1024, "the ring fits the LDS");
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

typedef __attribute__((address_space(3))) s16x4 lds_s16x4_r;
__device__ __forceinline__ s16x4 tr16(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_r*)p);
}

// The operands of one chunk step of a 16-column wave (wc = its first tile
// column): the record region `rec` and the value rows `val` of a slot.  Lane
// (lc, lg) = (lane % 16, lane / 16).  The transposing reads: lane j of 16-lane
// group g fetches the 8 bytes at row 4g + j / 4, columns 4 (j % 4) .. +3 of a
// token-major tile, and receives column j of rows 4g .. 4g + 3 (see
// lds_read_tr).
template <int VS>
__device__ __forceinline__ void read_slot(Ops<1>& o, const char* rec, const char* val, int wc, int lane) {
  const int lg = lane >> 4, lc = lane & 15;
  const int tr_row = 4 * lg + (lc >> 2), tr_col = 4 * (lc & 3);
  const char* tm = rec + kSlotTail + tr_row * 2 * C + 2 * tr_col;
  o.aT = __builtin_bit_cast(f16x4, tr16(tm));
  o.am = __builtin_bit_cast(f16x4, tr16(tm + 2 * C * C));
  const s16x4 raw = tr16(val + tr_row * VS + 2 * (wc + tr_col));
#pragma unroll
  for (int i = 0; i < 4; ++i) o.v[0][i] = bf16_to_f32((uint16_t)raw[i]);
  const char* qk = rec + lc * kQkStride + 16 * lg;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    o.aw[s] = *reinterpret_cast<const f16x8*>(qk + kSlotNk + 64 * s);
    o.aq[s] = *reinterpret_cast<const f16x8*>(qk + kSlotQh + 64 * s);
  }
  const char* kb = rec + kSlotKb + tr_row * kKbStride + 2 * tr_col;
#pragma unroll
  for (int m = 0; m < 8; ++m) o.ak[m] = __builtin_bit_cast(f16x4, tr16(kb + 32 * m));
  o.g2 = *reinterpret_cast<const f32x2*>(rec + kSlotTail + 4 * C * C + 8 * lane);
}

template <int WC, int LD, int PV>
__global__ __launch_bounds__((Tile<WC, LD>::kThreads)) void recur_kernel(RecurArgs a) {
  using Tl = Tile<WC, LD>;
  // How the waves meet: LDS flags (four or more compute waves with a CU to
  // themselves) or a workgroup barrier per step (see the loader and compute
  // loops).  T = 8192, H = 96 (64-column tiles), recurrence kernel alone:
  // 0.305 ms with barriers, 0.290 with flags; with two compute waves (H = 64)
  // and with two workgroups sharing a CU the flags were not faster (0.230
  // against 0.228 ms; 8 x 1024 tokens on the split path 0.266 against 0.269).
  constexpr bool kFlags = WC >= 4 && LD >= 4;
  __shared__ __align__(1024) char ring[Tl::kSlots * Tl::kSlotBytes];
  __shared__ int ready[Tl::kSlots];   // chunk + 1 of the chunk that has landed in each slot (0: none yet)
  __shared__ int done[WC];            // steps each compute wave has finished (its reads of them are done)
  const int64_t H = a.H;
  const WsHeader* hdr = reinterpret_cast<const WsHeader*>(a.ws);
  // Nothing is touched (no output, no state) unless the scheduler accepted
  // cu_seqlens; the fused kernel runs instead when the scheduler chose it.
  // (Without the scheduler, fixed_T > 0, neither can happen.)
  if (a.fixed_T == 0 && ((hdr->status & KDA_STATUS_BAD_CU_SEQLENS) || hdr->path == KDA_PATH_FUSED)) return;
  // XCD-aware placement: id b runs on XCD b % 8; the kTiles tiles of pair
  // 8 * g + x get ids 8 * (kTiles * g + tile) + x.
  const int64_t bid = blockIdx.x, x = bid & 7, q = bid >> 3;
  const int64_t pairs = a.N * H, pair2 = 8 * (q / Tl::kTiles) + x;
  const int tile = (int)(q % Tl::kTiles);
  if (pair2 >= (a.sets == 2 ? 2 * pairs : pairs)) return;
  const bool alt = pair2 >= pairs;   // the second set: the transition (zero values, identity start)
  const int64_t pair = alt ? pair2 - pairs : pair2;
  uint16_t* const outp = alt ? nullptr : a.out;
  const void* const s_in = alt ? nullptr : a.s_in;
  void* const s_out = alt ? static_cast<void*>(a.s_out2) : a.s_out;   // (alt: written below as fp16)
  const int sdt = alt ? KDA_DTYPE_FP32 : a.state_dtype;
  const int64_t slot_id = pair / H;
  const int h = (int)(pair - slot_id * H);
  const int v0 = tile * Tl::kCols;
  const int n = a.fixed_T > 0 ? (int)slot_id : reinterpret_cast<const int32_t*>(a.ws + a.lay.order)[slot_id];
  const SeqEntry se = a.fixed_T > 0 ? fixed_seq(a.fixed_T, C, n)
                                    : reinterpret_cast<const SeqEntry*>(a.ws + a.lay.seq_table)[n];
  // Records are chunk-major: record (chunk c, head h) at (c H + h) REC_BYTES,
  // so the chunks of one head lie H records apart.
  const char* recs = a.ws + a.lay.records + ((int64_t)se.first_chunk * H + h) * REC_BYTES;
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
  const int steps = ci_hi - ci_lo;
  const bool from_caller = ci_lo == 0, to_caller = ci_hi == nch;
  float* const ws_state = reinterpret_cast<float*>(a.ws + a.lay.state);

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int row_bytes = (int)(H * V * 2);
  if (tid < Tl::kSlots) ready[tid] = 0;
  if (tid < WC) done[tid] = 0;
  barrier();   // the flags start cleared
  int32_t* const status = const_cast<int32_t*>(&hdr->status);

  if (wave >= WC) {
    // ---------------- loader wave ----------------
    // Chunk c (step c of the launch) goes to slot c mod kSlots and belongs to
    // loader c mod kLoaders, which, in the order of its chunks: waits until
    // every compute wave is done with the slot's previous chunk, c - kSlots
    // (done[w] >= c - kSlots + 1); issues the chunk's loads; waits for them
    // (vmcnt(0): this loader has no other load in flight, so the wait covers
    // exactly these, whatever order loads complete in); and marks the slot
    // (ready = c + 1).  No cycle: a compute wave reaching step c - kSlots + 1
    // needs only chunks up to c - kSlots + 1, all issued before chunk c.
    static_assert(Tl::kLoaders <= Tl::kSlots, "a loader's chunks use distinct slots while in flight");
    const int j = wave - WC;
    // Source offset of this lane's 16-byte position in each load instruction.
    // Pads, and the value rows of a partial chunk past its end, lie past the
    // descriptor's range and read as zeros (the record gives those rows zero
    // weight); the transition set reads no values at all.
    int32_t vsrc[Tl::kValLoads], rsrc[kRecLoads];
#pragma unroll
    for (int i = 0; i < Tl::kValLoads; ++i) {
      const int P = 64 * i + lane, r = P / (Tl::kValStride / 16), p = P % (Tl::kValStride / 16);
      vsrc[i] = (r < C && p < Tl::kRowPieces) ? r * row_bytes + 16 * p : kFar;
    }
#pragma unroll
    for (int i = 0; i < kRecLoads; ++i) {
      const int P = 64 * i + lane;
      int src = kFar;
      if (P < kSlotNk / 16) {
        const int r = P / (kQkStride / 16), p = P % (kQkStride / 16);
        if (p < 16) src = REC_QH + 16 * (16 * r + p);
      } else if (P < kSlotKb / 16) {
        const int r = (P - kSlotNk / 16) / (kQkStride / 16), p = (P - kSlotNk / 16) % (kQkStride / 16);
        if (p < 16) src = REC_NK + 16 * (16 * r + p);
      } else if (P < kSlotTail / 16) {
        const int r = (P - kSlotKb / 16) / (kKbStride / 16), p = (P - kSlotKb / 16) % (kKbStride / 16);
        if (p < 16) src = REC_KB + 16 * (16 * r + p);
      } else if (P < kRecRegion / 16) {
        src = REC_T + 16 * (P - kSlotTail / 16);
      }
      rsrc[i] = src;
    }
    const char* vseq = reinterpret_cast<const char*>(a.v + ((int64_t)se.row0 * H + h) * V + v0);
    const uint32_t ring0 = lds_addr(ring);
    const auto issue = [&](int st) {
      const int c = ci_lo + st;
      const int len = min(se.len - C * c, C);
      const i32x4 rrec = buf_rsrc(recs + (int64_t)c * H * REC_BYTES, REC_BYTES);
      const i32x4 rval = buf_rsrc(vseq + (int64_t)c * C * row_bytes, alt ? 0 : (len - 1) * row_bytes + 2 * Tl::kCols);
      const uint32_t slot = ring0 + (uint32_t)((st % Tl::kSlots) * Tl::kSlotBytes);
#pragma unroll
      for (int i = 0; i < Tl::kValLoads; ++i) load_lds16(rval, slot + 1024 * i, vsrc[i]);
#pragma unroll
      for (int i = 0; i < kRecLoads; ++i) load_lds16(rrec, slot + Tl::kRecBase + 1024 * i, rsrc[i]);
    };
    if constexpr (kFlags) {
      bool ok = true;
      for (int c = j; c < steps; c += Tl::kLoaders) {
        if (c >= Tl::kSlots && ok)   // (after one wait gave up, none of this wave's waits spins)
          ok = spin_until<16>(a.spin_limit, [&] {
            int m = lds_get(&done[0]);
#pragma unroll
            for (int w = 1; w < WC; ++w) m = min(m, lds_get(&done[w]));
            return m >= c - Tl::kSlots + 1;
          });
        asm volatile("" ::: "memory");
        issue(c);
        wait_vmcnt<0>();   // chunk c has landed in its slot
        lds_put(&ready[c % Tl::kSlots], c + 1);
      }
      if (!ok && lane == 0) atomicOr(status, KDA_STATUS_SYNC_TIMEOUT);
    } else {
      // With barriers: chunk c is issued right after barrier c - kSlots + 2
      // (chunks 0 .. kSlots - 3 before the loop), when the compute waves are
      // done with the slot's previous chunk, c - kSlots (they finished it by
      // barrier c - kSlots + 1) and this loader has waited for its previous
      // chunk; it is waited for (vmcnt(0)) before barrier c.
      static_assert(kFlags || Tl::kLoaders == Tl::kSlots - 2, "one chunk in flight per loader");
      for (int c = j; c < min(steps, Tl::kSlots - 2); c += Tl::kLoaders) issue(c);
      for (int i = 0; i < steps; ++i) {
        const bool mine = i % Tl::kLoaders == j;
        if (mine) wait_vmcnt<0>();   // chunk i has landed in its slot
        barrier();
        if (mine && i + Tl::kSlots - 2 < steps) issue(i + Tl::kSlots - 2);
      }
    }
    return;
  }

  // ---------------- compute wave ----------------
  const int lg = lane >> 4, lc = lane & 15;
  const int64_t sbase = ((int64_t)n * H + h) * V * K;   // state [n][h][v][k]
  const int wc = 16 * wave;                              // first tile column of this wave
  const int col0 = v0 + wc;                              // first state column of this wave

  // ---- state slice: Z[m][0] holds rows 16m + 4lg + i, column col0 + lc
  f32x4 Z[8][1];
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    const int64_t idx = sbase + (int64_t)(col0 + lc) * K + 16 * m + 4 * lg;
    if (!from_caller) {
      Z[m][0] = *reinterpret_cast<const f32x4*>(ws_state + idx);
    } else if (alt) {   // stored [v][k] = (v == k); this lane holds k = 16 m + 4 lg + i, v = col0 + lc
      const int kv = col0 + lc - 16 * m - 4 * lg;
      Z[m][0] = f32x4{kv == 0 ? 1.f : 0.f, kv == 1 ? 1.f : 0.f, kv == 2 ? 1.f : 0.f, kv == 3 ? 1.f : 0.f};
    } else if (s_in == nullptr) {
      Z[m][0] = f32x4{0.f, 0.f, 0.f, 0.f};
    } else if (sdt == KDA_DTYPE_FP32) {
      Z[m][0] = *reinterpret_cast<const f32x4*>(static_cast<const float*>(s_in) + idx);
    } else {
      const u32x2 w = *reinterpret_cast<const u32x2*>(static_cast<const uint16_t*>(s_in) + idx);
      Z[m][0] = f32x4{bf16_lo(w[0]), bf16_hi(w[0]), bf16_lo(w[1]), bf16_hi(w[1])};
    }
  }

  if (steps > 0) {
    // Output rows of a full chunk: a wave-uniform base per chunk plus this
    // lane's fixed offset (token lc, columns 4 lg .. +3 of the wave).
    uint16_t* const out_seq = outp != nullptr ? outp + ((int64_t)(se.row0 + C * ci_lo) * H + h) * V + col0 : nullptr;
    const int64_t out_chunk = (int64_t)C * H * V;
    const int out_lane = (int)((lc * H) * V) + 4 * lg;
    // The output of a step is rounded and stored in the next step, well after
    // the MFMAs that produce it: a vector read of an MFMA result issued
    // shortly after it, with more MFMAs issued in between, has returned the
    // register's old contents on gfx950 although the compiler's wait states
    // were in place (a form of this loop unrolled by two, whose second copy
    // rounded its output right after computing it, got half of every lane's
    // values stale).  A scheduling barrier before every step barrier keeps
    // each step's instructions on their side of it.
    //
    // A compute wave waits for its step's chunk (ready == s + 1) by itself
    // and reports each finished step (done = s + 1) when its reads of the slot
    // are over, so the waves drift apart within the ring instead of meeting
    // at a barrier every step: their LDS reads and their MFMA chains overlap.
    f32x4 o_prev[1];
    bool ok = true;
    for (int s = 0; s < steps; ++s) {
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (kFlags) {
        if (ok) ok = spin_until(a.spin_limit, [&] { return lds_get(&ready[s % Tl::kSlots]) == s + 1; });
        asm volatile("" ::: "memory");   // the slot's reads stay behind the wait
      } else {
        barrier();
      }
      const char* slot = ring + (s % Tl::kSlots) * Tl::kSlotBytes;
      Ops<1> ops;
      read_slot<Tl::kValStride>(ops, slot + Tl::kRecBase, slot, wc, lane);
      if (s > 0 && outp != nullptr)   // output of step s - 1, a full chunk (only a sequence's last chunk is partial)
        *reinterpret_cast<u32x2*>(out_seq + (int64_t)(s - 1) * out_chunk + out_lane) = pack_out(o_prev[0]);
      compute<1, PV>(Z, ops, o_prev);
      wait_lgkm0();   // every read of this slot is done
      if constexpr (kFlags) lds_put(&done[wave], s + 1);
    }
    if (!ok && lane == 0) atomicOr(status, KDA_STATUS_SYNC_TIMEOUT);
    __builtin_amdgcn_sched_barrier(0);
    const Rows pr = chunk_rows(se, ci_hi - 1);
    if (lc < pr.len && outp != nullptr)
      *reinterpret_cast<u32x2*>(outp + ((pr.row0 + lc) * H + h) * V + col0 + 4 * lg) = pack_out(o_prev[0]);
  }

  // ---- state out
  if (!to_caller || s_out != nullptr) {
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const int64_t idx = sbase + (int64_t)(col0 + lc) * K + 16 * m + 4 * lg;
      if (!to_caller) {
        *reinterpret_cast<f32x4*>(ws_state + idx) = Z[m][0];
      } else if (alt) {   // the transition, fp16 in math layout [k][v]
        uint16_t* const at = a.s_out2 + sbase + (int64_t)(16 * m + 4 * lg) * V + col0 + lc;
#pragma unroll
        for (int i = 0; i < 4; ++i) at[i * V] = __builtin_bit_cast(uint16_t, (_Float16)Z[m][0][i]);
      } else if (sdt == KDA_DTYPE_FP32) {
        *reinterpret_cast<f32x4*>(static_cast<float*>(s_out) + idx) = Z[m][0];
      } else {
        *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(s_out) + idx) = pack_out(Z[m][0]);
      }
    }
  }
  // an operand beyond the fp16 range (or a non-finite input) leaves the state
  // non-finite: reported in the status word
  flag_nonfinite<8, 1>(Z, const_cast<int32_t*>(&hdr->status), KDA_STATUS_OVERFLOW);
}

template <int WC, int LD, int PV>
hipError_t launch_tiles(const RecurArgs& a, int64_t pairs, hipStream_t s) {
  using Tl = Tile<WC, LD>;
  const int64_t grid = 8 * Tl::kTiles * ((pairs + 7) / 8);
  if (grid > INT32_MAX) return hipErrorInvalidValue;
  RecurArgs b = a;
  b.spin_limit = spin_limit();
  hipLaunchKernelGGL((recur_kernel<WC, LD, PV>), dim3((unsigned)grid), dim3(Tl::kThreads), 0, s, b);
  return hipGetLastError();
}

// The precision study's variants (kda_fwd_precision) run on 64-column tiles.
template <int PV>
hipError_t launch_variant(const RecurArgs& a, int64_t pairs, hipStream_t s) {
  if constexpr (PV < 8) {
    if (a.precision == PV) return launch_tiles<4, 4, PV>(a, pairs, s);
    return launch_variant<PV + 1>(a, pairs, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

// Tiles per pair (recur_tiles, kda_internal.h), measured on MI355X
// (recurrence kernel alone, ms): T = 8192 H = 64 fixed: 0.210 with 4 tiles,
// 0.266 with 2; T = 8192 H = 96 fixed: 0.302 with 2 tiles, 0.395 with 4 (384
// workgroups > 256 CUs), 0.402 with 1; 12 ragged sequences, H = 96 (one of
// ~6000 tokens): 0.297 with 2, 0.396 with 1; 8 x 1024, H = 96: 0.239 with 1,
// 0.278 with 2.
//
// Loader waves and ring depth: while the launch has no more workgroups than
// the chip has CUs, each workgroup gets a CU to itself and a deep ring (six
// loaders and 8 slots for 32-column tiles, whose shorter steps need the loads
// issued further ahead: T = 8192, H = 64, 0.210 against 0.227 ms with four;
// four loaders and 6 slots otherwise: H = 96, 64 columns, 0.302 against 0.308
// with six).  With more workgroups than CUs, two loaders and 4 slots (68 / 74
// KB of LDS) let two workgroups share a CU, so that one's start (tables,
// state, the first chunk's latency: about 6 us) and end overlap the other's
// steps: 64 sequences of 128 tokens, H = 96, 0.479 -> 0.411 ms; 128 x 64,
// 0.768 -> 0.595; 8 x 1024, 0.276 -> 0.269.  With few workgroups the shallow
// ring is slower (T = 8192, H = 64: 0.210 -> 0.241), as two workgroups then
// share a CU while others idle.
hipError_t launch_recur(const RecurArgs& a, hipStream_t s) {
  if (a.lay.chunk == C32) return a.sets == 2 || a.precision != 0 ? hipErrorInvalidValue : launch_recur32(a, s);
  if (a.lay.chunk == C64) return a.sets == 2 || a.precision != 0 ? hipErrorInvalidValue : launch_recur64(a, s);
  const int64_t pairs = a.N * a.H * (a.sets == 2 ? 2 : 1);
  if (pairs == 0) return hipSuccess;
  if (a.precision < 0 || a.precision > 7) return hipErrorInvalidValue;
  if (a.precision != 0) return launch_variant<1>(a, pairs, s);
  const int tiles = a.tiles > 0 ? a.tiles : recur_tiles(pairs, false, a.cus);
  const bool shared = tiles * pairs > a.cus;   // more workgroups than CUs
  switch (tiles) {
    case 4: return launch_tiles<2, 6, 0>(a, pairs, s);   // (4 tiles only while 4 * pairs <= 256)
    case 2: return shared ? launch_tiles<4, 2, 0>(a, pairs, s) : launch_tiles<4, 4, 0>(a, pairs, s);
    case 1: return launch_tiles<8, 4, 0>(a, pairs, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace kda
