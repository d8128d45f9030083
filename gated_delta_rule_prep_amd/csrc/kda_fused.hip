// kda_fused.hip -- chunk prep and chunk recurrence of the KDA forward in one
// kernel for gfx950, with the chunk records kept in LDS.
//
// The FlashKDA blog post ("FlashKDA：月之暗面开源的 Kimi Delta Attention 高性能内核",
// §二 2.2) splits the forward pass into a token-parallel prep stage and a
// chunk-recurrent stage, joined by per-chunk records in global memory.  The
// raw inputs a chunk's record is made from (q, k, g, beta: 12.3 KB per chunk
// and head) are smaller than the record (13.8 KB), so building the record next
// to the recurrence that consumes it removes the record's round trip through
// HBM (written by the prep, read back by the recurrence) and the separate prep
// launch.  The price is that every workgroup builds its records itself: with
// two workgroups per (sequence, head) each record is built twice.
//
// One workgroup per (sequence, head, V-tile), eight waves:
//   * waves 0-3 run the recurrence (kda_step16.h) on 16 NT value columns each,
//     with the fp32 state slice in registers for the whole sequence; they
//     issue no loads;
//   * waves 4-7 build the records: prep wave p owns the chunks c = p mod 4 and
//     builds the record of chunk c during the four steps before step c - 1,
//     one phase per step (0: inputs, norms, channels 0-31; 1: channels 32-63;
//     2: channels 64-95; 3: channels 96-127, L and Mqk); the recurrence waves
//     invert I + L of chunk c at step c - 1.  At every step each prep wave
//     runs one phase, of four different chunks, so the per-step work is close
//     to even, and each SIMD holds one wave of each kind: the prep wave's ALU
//     work fills the recurrence wave's stalls.
// Steps s = -5 .. nchunks - 1.  Group s -- the raw q, k, g, beta of chunk
// s + 5 (read by the phase-0 wave of step s) and the value rows of chunk s
// (read by the recurrence at step s) -- is streamed HBM -> LDS with
// buffer_load ... lds into a ring of D group slots by the prep wave that reads
// its raw inputs, issued D - 1 steps ahead; that wave has no other group in
// flight and waits for it (vmcnt(0)) at the top of step s.  Records live in a
// ring of six slots (chunks s .. s + 5).  The record layout in LDS is the
// swizzled one kda_step16.h reads.
// The waves meet through progress flags in LDS, not a barrier per step: a
// prep wave starts step s once every recurrence wave has finished step s - 1
// (and, before reloading a group slot, once the prep wave that read it is
// done); a recurrence wave starts step s once every recurrence wave has
// finished step s - 1 (T of chunk s) and group s has landed, which also
// implies that chunks s and s + 1 are built (see the loop).  A barrier per
// step made every step as long as its slowest phase (phase 0 is about a fifth
// longer than phases 1 and 2); with the flags each prep wave runs its four
// phases back to back.  Every wait is bounded and reports a time-out in the
// status word.
//
// Per chunk, as in the split prep kernel (kda_prep.hip), with a2 the gate in
// log2 units, G its in-chunk inclusive cumulative sum, P = 2^G, Pinv = 2^-G,
// gam = P at the last token:
//   L   = strict_lower(diag(beta) (kn P)(kn Pinv)^T)
//   Mqk = lower_incl((qn P)(kn Pinv)^T)
//   T   = (I + L)^-1 diag(beta)   (forward substitution, exact for a unit
//                                 lower-triangular matrix)
//   record: Qhat = qn P, -Khat = -kn P, Kbar = kn Pinv gam, T^T, Mqk^T, gam
// L and Mqk multiply factors spanning up to e^(+-80) (the range argument of
// §二 2.1 of the same post at lower_bound = -5), so they are fp32 16x16x4
// products; the matrix cores run them beside the prep wave's vector work,
// which is what bounds the prep (each 64-lane vector instruction holds a
// SIMD for four cycles, a transcendental for sixteen).
#include "kda_device.h"
#include "kda_internal.h"
#include "kda_lds_pipe.h"
#include "kda_step16.h"
#include "../../include/kda.h"

namespace kda {
namespace {

constexpr int kRecWaves = 4;                 // recurrence waves
constexpr int kPrepWaves = 4;                // record-building waves
constexpr int kAllWaves = kRecWaves + kPrepWaves;
constexpr int kThreads = 64 * kAllWaves;
constexpr int kLead = 5;                     // raw inputs of chunk s + 5 arrive with group s
constexpr int kRecSlots = kLead + 1;         // records of chunks s .. s + 5
constexpr int kSlotBytes = REC_BYTES + 64;   // record + the chunk's beta (fp32 [16]) in LDS
constexpr float kEps = 1e-6f;
// The recurrence waves spend about half of each step waiting for the record
// builders; they poll their flags every 512 cycles (s_sleep 8), which leaves
// the SIMD and the LDS to the builder that shares it (varlen 8 x 1024, H = 96:
// fused kernel 0.453 ms against 0.454 polling every 64 cycles and 0.460 with a
// barrier per step; one 8192-token sequence 0.836 / 0.849 / 0.843 ms).
constexpr int kRecSleep = 8;

template <int NT, int D>
struct FCfg {
  static constexpr int kWaveCols = 16 * NT;               // value columns per recurrence wave
  static constexpr int kCols = kWaveCols * kRecWaves;     // value columns per workgroup
  static constexpr int kTiles = V / kCols;                // workgroups per (sequence, head)
  static constexpr int kRowPieces = kCols / 8;            // 16-byte pieces per value row of the tile
  static constexpr int kVBlocks = C * kRowPieces / 64;    // 1 KB blocks of value rows
  // 1 KB blocks of a group slot: q, k, g (4 each: 16 rows x 256 B), beta, values
  static constexpr int kQ = 0, kK = 4, kG = 8, kB = 12, kV = 13;
  static constexpr int kBlocks = kV + kVBlocks;
  static constexpr int kGroupBytes = kBlocks * 1024;
  static_assert(C * kRowPieces % 64 == 0, "value rows fill whole blocks");
  // group s is issued after barrier s - D + 1 and waited for before barrier s
  // by prep wave (s + kLead) mod 4, whose next group, s + 4, is issued after
  // barrier s + 5 - D: at most one group in flight per wave needs D <= 5
  static_assert(D >= 3 && D <= 5, "ring depth");
  static_assert(V % kCols == 0, "tile shape");
};

// Values a prep wave carries from one phase of a chunk to the next.
struct Carry {
  u32x4 qw[3], kw[3], gw[3];   // raw bf16 q, k, g of channel blocks 1..3 (block j at j - 1)
  float rq, rk;                // scale / |q|, 1 / |k| (0 for padded tokens)
  int valid;                   // token row < chunk length
  f32x4 accL[2], accM[2];      // L and Mqk partial sums over the blocks done so far (even / odd
                               // channels, two independent MFMA chains)
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

struct Seq {
  const uint16_t* q;       // q, k, g at (sequence row 0, head h)
  const uint16_t* k;
  const uint16_t* g;
  const char* beta;        // &beta[sequence row 0][h] (bytes)
  const uint16_t* v;       // v at (sequence row 0, head h, tile column 0)
  int64_t H;
  SeqEntry se;
};

// Issue the loads of group s into the group slot at LDS address `slot_lds`:
// q, k, g, beta of chunk s + kLead and the value rows of chunk s, each chunk
// index clamped into the sequence (clamped loads land in parts of slots that
// are never read).  One wave issues the whole group, all lanes, no waits.
// q / k / g: slot piece s of the tensor's 16 x 16-piece tile is row s / 16,
// position s % 16, and holds source piece position ^ row (XOR swizzle: the
// phase-0 reads of 16 rows at one piece index hit distinct banks).  Values:
// the swizzle kda_step16.h reads.  Beta: lane l fetches the 16-byte piece
// holding beta of token row l % 16.  Rows past the end of a partial chunk
// repeat its last row; the prep gives them zero weight.
template <int NT, int D>
__device__ __forceinline__ void issue_group(uint32_t slot_lds, const Seq& x, int s, int lane) {
  using F = FCfg<NT, D>;
  const int nch = x.se.nchunks;
  const int cq = min(max(s + kLead, 0), nch - 1), cv = min(max(s, 0), nch - 1);
  const Rows rq = chunk_rows(x.se, cq), rv = chunk_rows(x.se, cv);
  const int64_t H = x.H;
  const int rs = (int)(H * K * 2);   // bytes between token rows (q, k, g, v alike: K = V)
  const int64_t eq = (rq.row0 - x.se.row0) * H * K, ev = (rv.row0 - x.se.row0) * H * V;
  const int qbytes = (rq.len - 1) * rs + K * 2;
  const int lr = lane >> 4, lp = lane & 15;
  int qoff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 4 * i + lr;
    qoff[i] = min(r, rq.len - 1) * rs + 16 * (lp ^ r);
  }
  const uint16_t* const src[3] = {x.q, x.k, x.g};
#pragma unroll
  for (int t = 0; t < 3; ++t) {
    const i32x4 rsrc = buf_rsrc(src[t] + eq, qbytes);
#pragma unroll
    for (int i = 0; i < 4; ++i) load_lds16(rsrc, slot_lds + 1024 * (4 * t + i), qoff[i]);
  }
  static_assert(F::kQ == 0 && F::kK == 4 && F::kG == 8, "q, k, g blocks");
  {
    // 16-byte piece holding beta[row][h]; the descriptor starts at the piece
    // holding the chunk's first beta, so every offset is a multiple of 16
    const uintptr_t first = reinterpret_cast<uintptr_t>(x.beta + 2 * (rq.row0 - x.se.row0) * H);
    const uintptr_t mine = first + (uintptr_t)(2 * (int64_t)min(lp, rq.len - 1) * H);
    const uintptr_t base16 = first & ~(uintptr_t)15;
    load_lds16(buf_rsrc(reinterpret_cast<const void*>(base16), (rq.len - 1) * 2 * (int)H + 32),
               slot_lds + 1024 * F::kB, (int)((mine & ~(uintptr_t)15) - base16));
  }
  const i32x4 rval = buf_rsrc(x.v + ev, (rv.len - 1) * rs + F::kCols * 2);
#pragma unroll
  for (int i = 0; i < F::kVBlocks; ++i) {
    const int sp = 64 * i + lane, r = sp / F::kRowPieces, pos = sp % F::kRowPieces;
    load_lds16(rval, slot_lds + 1024 * (F::kV + i), min(r, rv.len - 1) * rs + 16 * (pos ^ (2 * (r & 3))));
  }
}

// Record field writers (swizzled layout of kda_step16.h).
__device__ __forceinline__ void put_qh(char* rec, int field, int row, int pos, u32x2 w) {
  // 4 fp16 values at channel position pos (a multiple of 4) of a Qhat / -W row
  *reinterpret_cast<u32x2*>(rec + field + 256 * row + 16 * ((pos >> 3) ^ row) + 2 * (pos & 7)) = w;
}

// Channel block J (channels 32 J + 8 cq .. + 7, lane (r, cq)) of a chunk:
// gates, their in-chunk cumulative sum, the decay factors and the decayed
// operands; Qhat, -Khat, Kbar and gamma go to the record, and the block's
// part of L and Mqk is added to accL / accM.  s_adt holds A2 * dt_bias, so
// the gate argument A2 (g + dt_bias) is one fma.
template <int J>
__device__ __forceinline__ void chan_block(u32x4 qw, u32x4 kw, u32x4 gw, float rq, float rk, bool valid, float A2,
                                           float lb2, const float* s_adt, int r, int cq, char* rec, f32x4 (&accL)[2],
                                           f32x4 (&accM)[2]) {
  const int c0 = 32 * J + 8 * cq;
  const f32x4 dtA = *reinterpret_cast<const f32x4*>(s_adt + c0);
  const f32x4 dtB = *reinterpret_cast<const f32x4*>(s_adt + c0 + 4);
  float kh[8], kb[8], qh[8], gm[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint32_t wg = gw[e >> 1], wq = qw[e >> 1], wk = kw[e >> 1];
    const float gv = (e & 1) ? bf16_hi(wg) : bf16_lo(wg);
    const float qv = (e & 1) ? bf16_hi(wq) : bf16_lo(wq);
    const float kv = (e & 1) ? bf16_hi(wk) : bf16_lo(wk);
    const float adt = e < 4 ? dtA[e] : dtB[e - 4];
    const float sg = valid ? fast_rcp(1.f + fast_exp2(fmaf(A2, gv, adt))) : 0.f;
    float cs = sg + dpp_shr(sg, 1);   // inclusive prefix sum over the 16 token lanes
    cs += dpp_shr(cs, 2);
    cs += dpp_shr(cs, 4);
    cs += dpp_shr(cs, 8);
    const float G = lb2 * cs;
    const float P = fast_exp2(G), Pinv = fast_exp2(-G);
    const float gam = dpp_bcast15(P);
    const float kn = kv * rk, qn = qv * rq;
    const float kP = kn * P, kI = kn * Pinv, qP = qn * P;
    // fp32 16x16x4: lane (r, cq) holds A[r][k = cq] and B[k = cq][r] for
    // channel c0 + e, so L and Mqk take the factors straight from registers
    accL[e & 1] = mfma_f32_k4(kP, kI, accL[e & 1]);
    accM[e & 1] = mfma_f32_k4(qP, kI, accM[e & 1]);
    kh[e] = -kP;
    qh[e] = qP;
    kb[e] = kI * gam;
    gm[e] = P;
  }
  u32x4 wkb;
#pragma unroll
  for (int w = 0; w < 4; ++w) wkb[w] = pack_f16(kb[2 * w], kb[2 * w + 1]);
  *reinterpret_cast<u32x4*>(rec + REC_KB + 256 * r + 16 * ((c0 >> 3) ^ (2 * (r & 3)))) = wkb;
  // Qhat and -Khat: channels 8cq .. 8cq+7 of block J sit at two runs of 4 positions
  const int p0 = 32 * J + kPermPos(8 * cq), p1 = 32 * J + kPermPos(8 * cq + 4);
  put_qh(rec, REC_QH, r, p0, u32x2{pack_f16(qh[0], qh[1]), pack_f16(qh[2], qh[3])});
  put_qh(rec, REC_QH, r, p1, u32x2{pack_f16(qh[4], qh[5]), pack_f16(qh[6], qh[7])});
  put_qh(rec, REC_NK, r, p0, u32x2{pack_f16(kh[0], kh[1]), pack_f16(kh[2], kh[3])});
  put_qh(rec, REC_NK, r, p1, u32x2{pack_f16(kh[4], kh[5]), pack_f16(kh[6], kh[7])});
  if (r == 15) {   // gam = P of the last token (padded tokens keep G constant)
    float* gam_out = reinterpret_cast<float*>(rec + REC_GAM);
#pragma unroll
    for (int e = 0; e < 8; ++e) gam_out[kGamSlot(c0 + e)] = gm[e];
  }
}

struct PrepCtx {
  float A2, lb2, scale;
  const float* s_adt;  // A2 * dt_bias of the head, in LDS
  int r, cq, lane;
};

// Phase 0 of a chunk: raw inputs from the group slot, norms, beta, channel
// block 0.
__device__ __forceinline__ void phase0(const PrepCtx& p, const char* grp, const Rows& rw, const Seq& x, char* rec,
                                       Carry& cr, int kQ, int kK, int kG, int kB) {
  const int r = p.r, cq = p.cq;
  u32x4 qw[4], kw[4], gw[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int o = 256 * r + 16 * ((4 * j + cq) ^ r);
    qw[j] = *reinterpret_cast<const u32x4*>(grp + 1024 * kQ + o);
    kw[j] = *reinterpret_cast<const u32x4*>(grp + 1024 * kK + o);
    gw[j] = *reinterpret_cast<const u32x4*>(grp + 1024 * kG + o);
  }
  const int rr = min(r, rw.len - 1);
  const uintptr_t addr = reinterpret_cast<uintptr_t>(x.beta + 2 * (rw.row0 - x.se.row0 + rr) * x.H);
  const uint16_t braw16 = *reinterpret_cast<const uint16_t*>(grp + 1024 * kB + 16 * r + (int)(addr & 15));
  const bool valid = r < rw.len;
  const float beta = valid ? fast_rcp(1.f + fast_exp2(-kLog2e * bf16_to_f32(braw16))) : 0.f;

  // sums of squares straight from the packed bf16 words (v_dot2: exact
  // products, fp32 accumulation), four independent chains per tensor.  The
  // words go through scalars before the bit cast: hipcc reads element 0 of
  // the vector for a bit cast applied to a vector element directly.
  float sqv[4] = {0.f, 0.f, 0.f, 0.f}, skv[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t qword = qw[j][w], kword = kw[j][w];
      const bf16x2 qv = __builtin_bit_cast(bf16x2, qword), kv = __builtin_bit_cast(bf16x2, kword);
      sqv[w] = __builtin_amdgcn_fdot2_f32_bf16(qv, qv, sqv[w], false);
      skv[w] = __builtin_amdgcn_fdot2_f32_bf16(kv, kv, skv[w], false);
    }
  float sq = (sqv[0] + sqv[1]) + (sqv[2] + sqv[3]), sk = (skv[0] + skv[1]) + (skv[2] + skv[3]);
  sq += __shfl_xor(sq, 16);
  sq += __shfl_xor(sq, 32);
  sk += __shfl_xor(sk, 16);
  sk += __shfl_xor(sk, 32);
  cr.rq = valid ? p.scale * __builtin_amdgcn_rsqf(sq + kEps) : 0.f;
  cr.rk = valid ? __builtin_amdgcn_rsqf(sk + kEps) : 0.f;
  cr.valid = valid;
  if (cq == 0) reinterpret_cast<float*>(rec + REC_BYTES)[r] = beta;

#pragma unroll
  for (int i = 0; i < 2; ++i) {
    cr.accL[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    cr.accM[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  chan_block<0>(qw[0], kw[0], gw[0], cr.rq, cr.rk, valid, p.A2, p.lb2, p.s_adt, r, cq, rec, cr.accL, cr.accM);
#pragma unroll
  for (int j = 1; j < 4; ++j) {
    cr.qw[j - 1] = qw[j];
    cr.kw[j - 1] = kw[j];
    cr.gw[j - 1] = gw[j];
  }
}

// Phases 1 and 2: channel block J (1 or 2).
template <int J>
__device__ __forceinline__ void phase_mid(const PrepCtx& p, char* rec, Carry& cr) {
  chan_block<J>(cr.qw[J - 1], cr.kw[J - 1], cr.gw[J - 1], cr.rq, cr.rk, cr.valid != 0, p.A2, p.lb2, p.s_adt, p.r,
                p.cq, rec, cr.accL, cr.accM);
}

// Phase 3: channel block 3, then L^T (to `lt`, for the inverse that the
// recurrence waves take one step later) and Mqk^T (record).
__device__ __forceinline__ void phase3(const PrepCtx& p, char* rec, float (*lt)[C + 4], Carry& cr) {
  chan_block<3>(cr.qw[2], cr.kw[2], cr.gw[2], cr.rq, cr.rk, cr.valid != 0, p.A2, p.lb2, p.s_adt, p.r, p.cq, rec,
                cr.accL, cr.accM);
  // lane (c, g) holds rows 4g..4g+3 of column c of L and Mqk
  const int lane = p.lane, lc = lane & 15, lg = lane >> 4;
  const float* beta = reinterpret_cast<const float*>(rec + REC_BYTES);
  const f32x4 accL = cr.accL[0] + cr.accL[1], accM = cr.accM[0] + cr.accM[1];
  float mv[4];
  f32x4 lv;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int rr = 4 * lg + i;
    lv[i] = lc < rr ? beta[rr] * accL[i] : 0.f;
    mv[i] = lc <= rr ? accM[i] : 0.f;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) lt[4 * lg + i][lc] = -lv[i];   // lt[r][m] = -L[r][m] (row-major)
  *reinterpret_cast<u32x2*>(rec + REC_MQK + (lc * C + 4 * lg) * 2) = u32x2{pack_f16(mv[0], mv[1]),
                                                                          pack_f16(mv[2], mv[3])};
}

// T = (I + L)^-1 diag(beta) of one chunk, columns 4w .. 4w + 3 by recurrence
// wave w, into the record as T^T.  Forward substitution by pivots, exact for
// a unit lower-triangular matrix: lane (r, j') holds x_r of column j = 4w + j'
// (x = e_j to start); once x_m is final (after pivots 0 .. m - 1), every row
// takes x_r -= L[r][m] x_m, with x_m broadcast from lane m of the lane's
// 16-lane row by DPP, one multiply-add per pivot (rows r <= m have L[r][m] = 0
// and keep their value).  The lane's row of -L comes from lt[r][0..15]
// (row-major, padded rows: the 16 rows' reads hit distinct banks); beta from
// the record's beta area.
template <int M>
__device__ __forceinline__ float subst_from(float x, const f32x4 (&l4)[4]) {
  // x_M from lane M of the 16-lane row (every lane of the row valid, so no
  // old value is needed), then x_r -= L[r][M] x_M with l4 holding -L
  const float xm = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x150 + M, 0xF, 0xF, true));
  x = fmaf(xm, l4[M >> 2][M & 3], x);
  if constexpr (M + 1 < C - 1) return subst_from<M + 1>(x, l4);
  return x;
}

__device__ __forceinline__ void chunk_inverse(const float (*lt)[C + 4], char* rec, int w, int lane) {
  const int r = lane & 15, j = 4 * w + (lane >> 4);
  f32x4 l4[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) l4[q] = *reinterpret_cast<const f32x4*>(&lt[r][4 * q]);
  const float x = subst_from<0>(r == j ? 1.f : 0.f, l4);
  const float bj = reinterpret_cast<const float*>(rec + REC_BYTES)[j];
  *reinterpret_cast<_Float16*>(rec + REC_T + (j * C + r) * 2) = (_Float16)(x * bj);   // T^T[j][r] = T[r][j]
}

template <int NT, int D>
__global__ __launch_bounds__(kThreads) void fused_kernel(FusedArgs a) {
  using F = FCfg<NT, D>;
  __shared__ __align__(1024) char groups[D][F::kGroupBytes];
  __shared__ __align__(16) char recs[kRecSlots][kSlotBytes];
  __shared__ __align__(16) float lts[2][C][C + 4];   // -L of chunks c (even / odd), from prep to the inverse
  __shared__ __align__(16) float s_adt[K];
  // Progress flags (the waves meet through them instead of a barrier per
  // step): steps are numbered s = -5 .. nch - 1 and a flag holds s + 6 once
  // its wave has finished step s (0: none).  pdone: prep waves; rdone:
  // recurrence waves (their reads of step s's record and value rows done, and
  // their part of T of chunk s + 1 written); gready: group slot holds group g
  // (g + 6), set by the wave that loaded it once the loads have landed.
  __shared__ __align__(16) int rdone[kRecWaves];
  __shared__ int pdone[kPrepWaves], gready[D];
  static_assert(kRecWaves == 4, "rdone is read as one 16-byte word");

  const int64_t H = a.H;
  // XCD-aware placement: id b runs on XCD b % 8; the kTiles tiles of pair
  // 8 * g + x get ids 8 * (kTiles * g + tile) + x, so they share an L2.
  const int64_t bid = blockIdx.x, xcd = bid & 7, qb = bid >> 3;
  const int64_t pair = 8 * (qb / F::kTiles) + xcd;
  const int tile = (int)(qb % F::kTiles);
  if (pair >= a.N * H) return;
  const WsHeader* hdr = reinterpret_cast<const WsHeader*>(a.ws);
  // Nothing is touched (no output, no state) unless the scheduler accepted
  // cu_seqlens; the split kernels run instead when the scheduler chose them.
  if ((hdr->status & KDA_STATUS_BAD_CU_SEQLENS) || hdr->path == KDA_PATH_SPLIT) return;
  const int64_t slot_id = pair / H;
  const int h = (int)(pair - slot_id * H);
  const int v0 = tile * F::kCols;
  const int n = reinterpret_cast<const int32_t*>(a.ws + a.lay.order)[slot_id];
  const SeqEntry se = reinterpret_cast<const SeqEntry*>(a.ws + a.lay.seq_table)[n];
  const int nch = se.nchunks;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, lg = lane >> 4, lc = lane & 15;
  const bool rec_wave = wave < kRecWaves;
  // The gate rate and bias, read before any buffer-to-LDS load is issued: the
  // compiler does not count those loads and would otherwise wait for all of
  // them at the first use of these values.
  float A2 = -expf(a.A_log[h]) * kLog2e;   // sigmoid(x) = 1 / (1 + 2^(-x log2 e))
  asm volatile("" : "+v"(A2));
  if (tid < K) s_adt[tid] = A2 * a.dt_bias[(int64_t)h * K + tid];
  // rdone starts at "step -2 done": the prep waves run steps -5 .. -1 (the
  // first records) before the recurrence waves have anything to do
  if (tid < kPrepWaves) pdone[tid] = 0;
  if (tid < kRecWaves) rdone[tid] = 4;
  if (tid < D) gready[tid] = 0;
  int32_t* const status = const_cast<int32_t*>(&hdr->status);
  bool ok = true;   // no wait of this wave gave up (after one did, it waits no more)

  const int64_t sbase = ((int64_t)n * H + h) * V * K;   // state [n][h][v][k]
  const int wc = F::kWaveCols * (rec_wave ? wave : 0);  // first tile column of a recurrence wave
  const int col0 = v0 + wc;
  f32x4 Z[8][NT];
  if (rec_wave) {
    load_state<NT>(Z, a.s_in, a.state_dtype, sbase, col0, lc, lg);
    // the state must have arrived before the first buffer-to-LDS load is
    // issued (otherwise the compiler's wait for it also waits for those)
#pragma unroll
    for (int m = 0; m < 8; ++m)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) asm volatile("" : "+v"(Z[m][nt]));
  }

  barrier();   // s_adt and the flags are set; the only workgroup barrier

  if (nch > 0) {
    Seq x;
    x.q = a.q + ((int64_t)se.row0 * H + h) * K;
    x.k = a.k + ((int64_t)se.row0 * H + h) * K;
    x.g = a.g + ((int64_t)se.row0 * H + h) * K;
    x.beta = reinterpret_cast<const char*>(a.beta + (int64_t)se.row0 * H + h);
    x.v = a.v + ((int64_t)se.row0 * H + h) * V + v0;
    x.H = H;
    x.se = se;
    const uint32_t g0 = lds_addr(groups[0]);

    // The two kinds of wave run separate loops over the same steps, meeting
    // through the progress flags, so that neither carries the other's
    // registers.
    if (rec_wave) {
      // The recurrence waves issue no loads: they wait for their LDS traffic
      // (reads of the step's operands, T written by the inverse) before they
      // report a step.  The output of a step is rounded and stored in the next
      // step, well after the MFMAs that produce it, and a scheduling barrier
      // keeps each step's instructions on their side of the waits.
      uint16_t* const out_seq = a.out + ((int64_t)se.row0 * H + h) * V + col0;
      const int64_t out_chunk = (int64_t)C * H * V;
      const int out_lane = (int)((lc * H) * V) + 4 * lg;
      f32x4 o_prev[NT];
      int gslot = kLead % D;   // group slot of group s (group g sits in slot (g + kLead) mod D)
      // step -1: the inverse of chunk 0, once its L is complete (phase 3 at
      // step -2 by prep wave 0)
      ok = spin_until(a.spin_limit, [&] { return lds_get(&pdone[0]) >= 4; });
      asm volatile("" ::: "memory");
      chunk_inverse(lts[0], recs[0], wave, lane);
      wait_lgkm0();
      lds_put(&rdone[wave], 5);
      const auto rec_min = [&] { return lds_min4(rdone); };
      int rs = 0;   // record slot of chunk s
      for (int s = 0; s < nch; ++s) {
        __builtin_amdgcn_sched_barrier(0);
        // Step s needs T of chunk s (every recurrence wave's part, written at
        // step s - 1) and group s (the value rows) landed.  It also needs
        // chunk s's record (phase 3 at step s - 2) and L of chunk s + 1 (phase
        // 3 at step s - 1, for this step's inverse), which those two waits
        // imply: the prep wave that finishes chunk s + 1 is the one that loads
        // group s and reports it only at the top of step s, after its step
        // s - 1; likewise group s - 1, waited for at step s - 1, came from the
        // wave that finished chunk s at step s - 2 (for s = 0: the wait before
        // the inverse of chunk 0).
        if (ok) ok = spin_until<kRecSleep>(a.spin_limit, [&] { return rec_min() >= s + 5; });
        if (ok) ok = spin_until<kRecSleep>(a.spin_limit, [&] { return lds_get(&gready[gslot]) == s + 6; });
        asm volatile("" ::: "memory");   // the step's LDS traffic stays behind the waits
        if (s > 0) {   // output of chunk s - 1, a full chunk (only the last chunk is partial)
          uint16_t* const ob = out_seq + (int64_t)(s - 1) * out_chunk;
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) *reinterpret_cast<u32x2*>(ob + out_lane + 16 * nt) = pack_out(o_prev[nt]);
        }
        // T of chunk s + 1, independent of this step's chain; past the last
        // chunk it lands in a record slot that no chunk uses any more
        const int rs1 = rs == kRecSlots - 1 ? 0 : rs + 1;
        chunk_inverse(lts[(s + 1) & 1], recs[rs1], wave, lane);
        Ops<NT> ops;
        read_ops<NT>(ops, recs[rs], groups[gslot] + 1024 * F::kV, 2 * F::kCols, wc, lane);
        compute<NT>(Z, ops, o_prev);
        wait_lgkm0();   // this step's reads are done and its part of T is written
        lds_put(&rdone[wave], s + 6);
        gslot = gslot == D - 1 ? 0 : gslot + 1;
        rs = rs1;
      }
      __builtin_amdgcn_sched_barrier(0);
      const Rows pr = chunk_rows(se, nch - 1);
      if (lc < pr.len) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          *reinterpret_cast<u32x2*>(a.out + ((pr.row0 + lc) * H + h) * V + col0 + 16 * nt + 4 * lg) = pack_out(o_prev[nt]);
      }
    } else {
      PrepCtx pc;
      pc.A2 = A2;
      pc.lb2 = a.lower_bound * kLog2e;
      pc.scale = a.scale;
      pc.s_adt = s_adt;
      pc.r = lc;
      pc.cq = lg;
      pc.lane = lane;
      Carry cr;
      const int pw = wave - kRecWaves;   // this prep wave builds the chunks c = pw mod 4
      // Group g (steps g = -5 .. nch - 1) belongs to the prep wave that reads
      // its raw inputs (phase 0 of chunk g + 5), pw = (g + 5) mod 4.  That wave
      // issues it at step g - D + 1 into the slot of group g - D, once every
      // wave is done with that group (the recurrence waves with step g - D, the
      // prep wave that read it with step g - D), waits for it (vmcnt(0)) at the
      // top of step g and reports it in gready.  The wave's next group, g + 4,
      // is issued at step g + 5 - D >= g, so a prep wave never has more than
      // one group in flight and each wait covers exactly that group's loads,
      // whatever order loads complete in.  Prep waves issue no other global
      // loads or stores in the loop.
      const auto mine = [&](int g) { return ((g + kLead) & 3) == pw; };
      const auto rec_min = [&] { return lds_min4(rdone); };
      for (int g = -kLead; g < min(-kLead + D - 1, nch); ++g)
        if (mine(g)) issue_group<NT, D>(g0 + (g + kLead) * F::kGroupBytes, x, g, lane);
      int gslot = 0;   // group slot of group s
      for (int s = -kLead; s < nch; ++s) {
        if (mine(s)) {
          wait_vmcnt<0>();   // group s has landed in its slot
          lds_put(&gready[gslot], s + 6);
        }
        // Every recurrence wave is done with step s - 1: with the record slot
        // that chunk s + 5 takes (chunk s - 1), with L of chunk s (the inverse
        // at step s - 1), whose buffer phase 3 of chunk s + 2 takes, and with
        // the value rows of group s - 1, whose slot group s + D - 1 takes.
        if (ok) ok = spin_until(a.spin_limit, [&] { return rec_min() >= s + 5; });
        asm volatile("" ::: "memory");
        // The lane id passes through an empty asm each step, so that the
        // lane-dependent addresses and constants of the group loads and of the
        // four phases are computed where they are used instead of being
        // hoisted out of the loop and held (or spilled) across it.
        int ln = lane;
        asm volatile("" : "+v"(ln));
        if (s + D - 1 < nch && mine(s + D - 1)) {
          // the prep wave that read group s - 1 (phase 0 at step s - 1) is done with it
          if (ok) ok = spin_until(a.spin_limit, [&] { return lds_get(&pdone[(s + 4) & 3]) >= s + 5; });
          asm volatile("" ::: "memory");
          issue_group<NT, D>(g0 + (gslot == 0 ? D - 1 : gslot - 1) * F::kGroupBytes, x, s + D - 1, ln);
        }
        // chunk c (c = pw mod 4) is built in phases 0..3 at steps c - 5 .. c - 2
        const int ph = (s + kLead - pw) & 3;
        const int c = s + kLead - ph;
        if (c >= 0 && c < nch) {
          pc.r = ln & 15;
          pc.cq = ln >> 4;
          pc.lane = ln;
          char* rec = recs[c % kRecSlots];
          if (ph == 0) {
            phase0(pc, groups[gslot], chunk_rows(se, c), x, rec, cr, F::kQ, F::kK, F::kG, F::kB);
          } else if (ph == 1) {
            phase_mid<1>(pc, rec, cr);
          } else if (ph == 2) {
            phase_mid<2>(pc, rec, cr);
          } else {
            phase3(pc, rec, lts[c & 1], cr);
          }
        }
        wait_lgkm0();   // this step's LDS writes are done
        lds_put(&pdone[pw], s + 6);
        gslot = gslot == D - 1 ? 0 : gslot + 1;
      }
      wait_vmcnt<0>();   // (nothing is in flight here: every group issued was waited for)
    }
  }

  if (!ok && lane == 0) atomicOr(status, KDA_STATUS_SYNC_TIMEOUT);
  if (rec_wave) {
    if (a.s_out != nullptr) store_state<NT>(Z, a.s_out, a.state_dtype, sbase, col0, lc, lg);
    // an operand beyond the fp16 range (or a non-finite input) leaves the
    // state non-finite: reported in the status word
    flag_nonfinite<8, NT>(Z, status, KDA_STATUS_OVERFLOW);
  }
}

template <int NT, int D>
hipError_t launch_tiles(const FusedArgs& a, hipStream_t s) {
  const int64_t pairs = a.N * a.H;
  const int64_t grid = 8 * FCfg<NT, D>::kTiles * ((pairs + 7) / 8);
  FusedArgs b = a;
  b.spin_limit = spin_limit();
  hipLaunchKernelGGL((fused_kernel<NT, D>), dim3((unsigned)grid), dim3(kThreads), 0, s, b);
  return hipGetLastError();
}

}  // namespace

// Value columns per workgroup (fused_two_tiles): 64 (two workgroups per
// (sequence, head), each building the pair's records itself) while the pairs
// are few, so that the longest chain of the batch runs at half the per-step
// work; 128 (one workgroup per pair, each record built once) once two tiles
// per pair would not all fit on the 256 CUs at once.
hipError_t launch_fused(const FusedArgs& a, hipStream_t s) {
  if (a.N * a.H == 0) return hipSuccess;
  if (fused_two_tiles(a.N * a.H, a.cus)) return launch_tiles<1, 4>(a, s);
  return launch_tiles<2, 3>(a, s);
}

}  // namespace kda
