// kda_prep.hip -- token-parallel chunk-prep kernel for gfx950.
//
// The first of the two stages the pages split the forward pass into (P1 §二
// 2.2: gate activation, L2 norm, decay, L / Mqk, inverse), with the base-2
// exponentials of P1 §二 2.4 taken from the native v_exp_f32 (which computes 2^x).
//
// P1 = blog post "FlashKDA：月之暗面开源的 Kimi Delta Attention 高性能内核".
//
// One wave per (chunk, head); the four waves of a workgroup take four heads of
// the same chunk and never synchronise with each other.  Chunks come from the
// scheduler's table, so a chunk never straddles two sequences; a partial chunk
// is treated as padded with a = 0, beta = 0, q = k = 0, which leaves every real
// token's result unchanged.
//
// Lane l holds token r = l % 16 and channels 32 j + 8 (l / 16) + e (j, e in
// 0..3, 0..7).  Per chunk of 16 tokens, with a2 the gate in log2 units:
//   a2[r][i] = lower_bound * log2(e) * sigmoid(exp(A_log) * (g + dt_bias))
//   G[r][i]  = sum_{j<=r} a2[j][i]    (DPP prefix scan over the 16 token lanes)
//   P = 2^G, Pinv = 2^-G, gam = P at the last token (DPP row broadcast)
//   kn = k / |k|, qn = scale * q / |q|     (|x| = sqrt(sum x^2 + 1e-6))
//   L   = strict_lower(diag(beta) (kn P)(kn Pinv)^T)   fp32 MFMA 16x16x4
//   Mqk = lower_incl((qn P)(kn Pinv)^T)                 fp32 MFMA 16x16x4
//   T   = (I + L)^-1 diag(beta)   forward substitution in fp32 (L is strictly
//                                 lower, so the inverse is exact)
// The record holds Qhat = qn P, -Khat = -kn P, Kbar = kn Pinv gam, T^T, Mqk^T
// and gam (the recurrence forms T (V - Khat Z), so W = T Khat is never needed).
// The factor pair (kn P, kn Pinv) spans up to e^(+-80) at lower_bound = -5 (the
// range argument of P1 §二 2.1): it fits fp32, so L and Mqk are multiplied in
// fp32 (rounding these factors to a 16-bit type costs about 2^-9 of every
// entry, which alone used more than the output error budget).  Everything the
// recurrence reads is bounded by 1 (or by scale) and is stored in fp16.
#include "kda_device.h"
#include "kda_internal.h"
#include "kda_lds_pipe.h"
#include "../../include/kda.h"

namespace kda {
namespace {

constexpr int kWaves = 2;
constexpr int kThreads = 64 * kWaves;
constexpr float kEps = 1e-6f;

// A wave builds its record in LDS and writes it out as whole contiguous
// pieces (16 bytes per lane, 1 KB per store instruction) with streaming
// (nontemporal) stores: the record's scattered 4- to 16-byte parts never reach
// the caches as partial lines, and the recurrence reads the records only after
// the whole prep has run.  Qhat, -Khat and Kbar are staged one 64-channel half
// of their rows at a time (written out after channel blocks 1 and 3, each half
// row a whole 128-byte line), T, Mqk and gamma at the end, so a wave needs
// 9 KB of LDS and the registers, not the LDS, bound the waves per CU.
constexpr int kHalfBytes = 128;                 // one 64-channel half of a 256-byte row
constexpr int kTailBytes = REC_BYTES - REC_T;   // T, Mqk, gamma
static_assert(REC_NK == REC_QH + C * 2 * K && REC_KB == REC_NK + C * 2 * K && REC_T == REC_KB + C * 2 * K,
              "Qhat, -Khat and Kbar are three consecutive [16][128] fp16 arrays");
struct __align__(16) WaveSmem {
  __align__(16) float L[C][C + 4];       // L (fp32), 80-byte rows
  float beta[C];
  __align__(16) char half[3][C][kHalfBytes];   // Qhat, -Khat, Kbar: the current half of every row
  __align__(16) char tail[kTailBytes];         // T^T, Mqk^T, gamma as in the record
};
static_assert(sizeof(WaveSmem::half) >= 4 * sizeof(float) * C * (C + 4),
              "the staged halves hold the four scratch matrices of the precision study's inverse");

// Writes the staged half `hf` of the three row arrays: 3 x 16 rows x 8 pieces.
__device__ __forceinline__ void flush_half(const WaveSmem& sm, char* rec_out, int hf, int lane) {
  wait_lgkm0();
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int i = 0; i < 3 * C * (kHalfBytes / 16) / 64; ++i) {
    const int pi = 64 * i + lane, arr = pi >> 7, row = (pi >> 3) & 15, part = pi & 7;
    const u32x4 x = *reinterpret_cast<const u32x4*>(&sm.half[arr][row][16 * part]);
    __builtin_nontemporal_store(x, reinterpret_cast<u32x4*>(rec_out + REC_QH + arr * C * 2 * K + row * 2 * K +
                                                            hf * kHalfBytes + 16 * part));
  }
  asm volatile("" ::: "memory");   // the next half's LDS writes stay behind these reads
}

// The inverse in the form the pages give it (P1 §二 2.1, 2.3), for the
// precision study only: (I + L)^-1 = (I - L)(I + L^2)(I + L^4)(I + L^8),
// exact because L is strictly lower (L^16 = 0).  Every factor and product is
// an fp16 operand of a 16x16x16 MFMA with fp32 accumulation, each result
// rounded to fp16 before it is used again.  Lane (c, g) of an MFMA holds
// rows 4g..4g+3 of column c of the result; the 16 x 16 matrices pass between
// the products through LDS (fp32 rows of 20).
typedef float Mat16[C][C + 4];

// A operand of s M + d I: lane (c, g) holds row c, columns 4g..4g+3.
__device__ __forceinline__ f16x4 nm_a(const Mat16& m, float sc, float d, int lc, int lg) {
  f16x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = (_Float16)(sc * m[lc][4 * lg + i] + (lc == 4 * lg + i ? d : 0.f));
  return r;
}
// B operand of s M + d I: lane (c, g) holds rows 4g..4g+3 of column c.
__device__ __forceinline__ f16x4 nm_b(const Mat16& m, float sc, float d, int lc, int lg) {
  f16x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = (_Float16)(sc * m[4 * lg + i][lc] + (lc == 4 * lg + i ? d : 0.f));
  return r;
}
__device__ __forceinline__ void nm_store(Mat16& m, f32x4 acc, int lc, int lg) {
#pragma unroll
  for (int i = 0; i < 4; ++i) m[4 * lg + i][lc] = (float)(_Float16)acc[i];
  __builtin_amdgcn_wave_barrier();
}

// T^T of the chunk (row j = column j of (I + L)^-1 times beta_j) into the
// record tail, from L and beta in LDS; `scratch` holds four matrices.
__device__ __forceinline__ void neumann_inverse(const Mat16& L, const float* beta, Mat16* scratch, char* tail,
                                                int lane) {
  const int lc = lane & 15, lg = lane >> 4;
  const f32x4 z = {0.f, 0.f, 0.f, 0.f};
  nm_store(scratch[0], mfma_f16_k16(nm_a(L, 1.f, 0.f, lc, lg), nm_b(L, 1.f, 0.f, lc, lg), z), lc, lg);   // L^2
  nm_store(scratch[1], mfma_f16_k16(nm_a(scratch[0], 1.f, 0.f, lc, lg), nm_b(scratch[0], 1.f, 0.f, lc, lg), z),
           lc, lg);                                                                                        // L^4
  nm_store(scratch[2], mfma_f16_k16(nm_a(scratch[1], 1.f, 0.f, lc, lg), nm_b(scratch[1], 1.f, 0.f, lc, lg), z),
           lc, lg);                                                                                        // L^8
  nm_store(scratch[3], mfma_f16_k16(nm_a(L, -1.f, 1.f, lc, lg), nm_b(scratch[0], 1.f, 1.f, lc, lg), z),
           lc, lg);                                                          // (I - L)(I + L^2)
  nm_store(scratch[0], mfma_f16_k16(nm_a(scratch[3], 1.f, 0.f, lc, lg), nm_b(scratch[1], 1.f, 1.f, lc, lg), z),
           lc, lg);                                                          //   (I + L^4)
  const f32x4 n = mfma_f16_k16(nm_a(scratch[0], 1.f, 0.f, lc, lg), nm_b(scratch[2], 1.f, 1.f, lc, lg), z);   // (I + L^8)
  const float bj = beta[lc];
  u32x2 w;
  w[0] = pack_f16(n[0] * bj, n[1] * bj);
  w[1] = pack_f16(n[2] * bj, n[3] * bj);
  *reinterpret_cast<u32x2*>(tail + (lc * C + 4 * lg) * 2) = w;   // T^T[c][4g..4g+3] = T[4g..4g+3][c]
}

// INV = 0: the inverse by forward substitution in fp32 (the library's);
// INV = 1: the fp16 Neumann product above (kda_fwd_precision only).
template <int INV>
__global__ __launch_bounds__(kThreads) void prep_kernel(PrepArgs a) {
  __shared__ WaveSmem wsm[kWaves];
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int64_t H = a.H;
  // One linear grid, head groups fastest: the workgroups of one chunk launch
  // together, so they read the same token rows (and the same beta sectors) of
  // q, k, g and beta at about the same time.
  const int hx = (int)((H + kWaves - 1) / kWaves);
  const int hgrp = (int)(blockIdx.x % (unsigned)hx), cidx = (int)(blockIdx.x / (unsigned)hx);
  const int h = hgrp * kWaves + wave;
  const WsHeader* hdr = reinterpret_cast<const WsHeader*>(a.ws);
  int chunk = cidx;
  ChunkEntry ce;
  if (a.fixed_T > 0) {
    const int64_t total = a.fixed_B * ((a.fixed_T + C - 1) / C);
    if (blockIdx.x == 0 && tid == 0) {   // the header the scheduler kernel would have written
      WsHeader* w = reinterpret_cast<WsHeader*>(a.ws);
      w->status = KDA_STATUS_OK;
      w->chunk_count = (int32_t)total;
      w->path = KDA_PATH_SPLIT;
      w->part_first[0] = 0;
      w->part_first[1] = (int32_t)total;
    }
    if (chunk >= total || h >= H) return;   // whole waves only; no barriers below
    ce = fixed_chunk(a.fixed_T, C, chunk);
  } else {
    chunk = hdr->part_first[a.part] + cidx;   // this launch covers one part
    if (chunk >= hdr->part_first[a.part + 1] || h >= H) return;
    if (hdr->path == KDA_PATH_FUSED) return;   // the scheduler chose the fused kernel
    ce = reinterpret_cast<const ChunkEntry*>(a.ws + a.lay.chunk_table)[chunk];
  }
  WaveSmem& sm = wsm[wave];
  const int r = lane & 15, cq = lane >> 4;
  const bool valid = r < ce.len;
  const int64_t tok = (int64_t)ce.row0 + min(r, ce.len - 1);   // clamped: loads stay in the sequence
  const int64_t base = (tok * H + h) * K + 8 * cq;

  // ---- loads: q, k (4 x 16 B each) and beta; g per channel block below
  u32x4 qw[4], kw[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    qw[j] = *reinterpret_cast<const u32x4*>(a.q + base + 32 * j);
    kw[j] = *reinterpret_cast<const u32x4*>(a.k + base + 32 * j);
  }
  const float braw = bf16_to_f32(a.beta[tok * H + h]);
  const float beta = valid ? 1.f / (1.f + expf(-braw)) : 0.f;

  // ---- L2 norms: 32 channels per lane, then the 4 lanes of the token
  float sq = 0.f, sk = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float q0 = bf16_lo(qw[j][w]), q1 = bf16_hi(qw[j][w]);
      const float k0 = bf16_lo(kw[j][w]), k1 = bf16_hi(kw[j][w]);
      sq = fmaf(q0, q0, fmaf(q1, q1, sq));
      sk = fmaf(k0, k0, fmaf(k1, k1, sk));
    }
  sq += __shfl_xor(sq, 16);
  sq += __shfl_xor(sq, 32);
  sk += __shfl_xor(sk, 16);
  sk += __shfl_xor(sk, 32);
  const float rq = valid ? a.scale / sqrtf(sq + kEps) : 0.f;
  const float rk = valid ? 1.f / sqrtf(sk + kEps) : 0.f;

  const float A2 = -expf(a.A_log[h]) * kLog2e;   // sigmoid(x) = 1 / (1 + 2^(-x log2 e))
  const float lb2 = a.lower_bound * kLog2e;
  char* const rec_out = a.ws + a.lay.records + ((int64_t)chunk * H + h) * REC_BYTES;   // chunk-major
  // staged row r of the three arrays (element e of the current half) and the tail
  _Float16* const st_qh = reinterpret_cast<_Float16*>(sm.half[0][r]);
  _Float16* const st_nk = reinterpret_cast<_Float16*>(sm.half[1][r]);
  _Float16* const st_kb = reinterpret_cast<_Float16*>(sm.half[2][r]);
  char* const tail = sm.tail;
  float* const rec_gam = reinterpret_cast<float*>(tail + (REC_GAM - REC_T));

  // ---- per channel slot: gate, scan, decay factors, products, L / Mqk MFMAs
  f32x4 accL = {0.f, 0.f, 0.f, 0.f}, accM = {0.f, 0.f, 0.f, 0.f};
  // g is needed one channel block at a time: block j + 1 loads while block j
  // computes, so only two of its four 16-byte pieces are ever held
  u32x4 gnext = *reinterpret_cast<const u32x4*>(a.g + base);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const u32x4 gcur = gnext;
    if (j < 3) gnext = *reinterpret_cast<const u32x4*>(a.g + base + 32 * (j + 1));
    const int c0 = 32 * j + 8 * cq;
    const f32x4 dtA = *reinterpret_cast<const f32x4*>(a.dt_bias + (int64_t)h * K + c0);
    const f32x4 dtB = *reinterpret_cast<const f32x4*>(a.dt_bias + (int64_t)h * K + c0 + 4);
    float kh[8], qh[8], kb[8], gm[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t wg = gcur[e >> 1], wq = qw[j][e >> 1], wk = kw[j][e >> 1];
      const float gv = (e & 1) ? bf16_hi(wg) : bf16_lo(wg);
      const float qv = (e & 1) ? bf16_hi(wq) : bf16_lo(wq);
      const float kv = (e & 1) ? bf16_hi(wk) : bf16_lo(wk);
      const float dt = e < 4 ? dtA[e] : dtB[e - 4];
      const float sg = valid ? fast_rcp(1.f + fast_exp2(A2 * (gv + dt))) : 0.f;
      float cs = sg + dpp_shr(sg, 1);   // inclusive prefix sum over the 16 token lanes
      cs += dpp_shr(cs, 2);
      cs += dpp_shr(cs, 4);
      cs += dpp_shr(cs, 8);
      const float G = lb2 * cs;
      const float P = fast_exp2(G), Pinv = fast_exp2(-G);
      const float gam = dpp_bcast15(P);
      const float kn = kv * rk, qn = qv * rq;
      const float kP = kn * P, kI = kn * Pinv;
      const float qP = qn * P;
      accL = mfma_f32_k4(kP, kI, accL);   // k-slot lane/16 carries channel c0 + e
      accM = mfma_f32_k4(qP, kI, accM);
      kh[e] = kP;
      qh[e] = qP;
      kb[e] = kI * gam;
      gm[e] = P;
    }
    // Kbar -> record (token-major); Qhat and -Khat -> record (channels
    // 8cq .. 8cq+7 of 32-block j sit at two runs of 4 positions)
    u32x4 wkb;
#pragma unroll
    for (int w = 0; w < 4; ++w) wkb[w] = pack_f16(kb[2 * w], kb[2 * w + 1]);
    const int hb = 64 * (j >> 1);   // first channel (element) of the staged half
    *reinterpret_cast<u32x4*>(st_kb + c0 - hb) = wkb;
    const int p0 = 32 * j + kPermPos(8 * cq) - hb, p1 = 32 * j + kPermPos(8 * cq + 4) - hb;
    *reinterpret_cast<u32x2*>(st_qh + p0) = u32x2{pack_f16(qh[0], qh[1]), pack_f16(qh[2], qh[3])};
    *reinterpret_cast<u32x2*>(st_qh + p1) = u32x2{pack_f16(qh[4], qh[5]), pack_f16(qh[6], qh[7])};
    *reinterpret_cast<u32x2*>(st_nk + p0) = u32x2{pack_f16(-kh[0], -kh[1]), pack_f16(-kh[2], -kh[3])};
    *reinterpret_cast<u32x2*>(st_nk + p1) = u32x2{pack_f16(-kh[4], -kh[5]), pack_f16(-kh[6], -kh[7])};
    if (r == 15) {   // gam = P of the last token (padded tokens keep G constant)
#pragma unroll
      for (int e = 0; e < 8; ++e) rec_gam[kGamSlot(c0 + e)] = gm[e];
    }
    if (j & 1) flush_half(sm, rec_out, j >> 1, lane);
  }

  // ---- L (to LDS) and Mqk^T (to the record); lane (c, g) holds rows 4g..4g+3 of column c
  if (cq == 0) sm.beta[r] = beta;
  __builtin_amdgcn_wave_barrier();
  const int lc = lane & 15, lg = lane >> 4;
  {
    u32x2 wm;
    float mv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rr = 4 * lg + i;
      sm.L[rr][lc] = lc < rr ? sm.beta[rr] * accL[i] : 0.f;
      mv[i] = lc <= rr ? accM[i] : 0.f;
    }
    wm[0] = pack_f16(mv[0], mv[1]);
    wm[1] = pack_f16(mv[2], mv[3]);
    *reinterpret_cast<u32x2*>(tail + (REC_MQK - REC_T) + (lc * C + 4 * lg) * 2) = wm;   // Mqk^T[c][4g..4g+3]
  }
  __builtin_amdgcn_wave_barrier();

  // ---- T^T row j = column j of (I + L)^-1 times beta_j (lanes 0..15)
  if constexpr (INV == 1) {
    wait_lgkm0();   // the staged halves are read out: their LDS serves as scratch
    __builtin_amdgcn_wave_barrier();
    neumann_inverse(sm.L, sm.beta, reinterpret_cast<Mat16*>(&sm.half[0][0][0]), tail, lane);
  } else if (lane < C) {
    const int jc = lane;
    float x[C];
#pragma unroll
    for (int rr = 0; rr < C; ++rr) {
      float s = rr == jc ? 1.f : 0.f;
#pragma unroll
      for (int m = 0; m < rr; ++m) s = fmaf(-sm.L[rr][m], x[m], s);
      x[rr] = s;
    }
    const float bj = sm.beta[jc];
    u32x4 t0, t1;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      t0[w] = pack_f16(x[2 * w] * bj, x[2 * w + 1] * bj);
      t1[w] = pack_f16(x[8 + 2 * w] * bj, x[8 + 2 * w + 1] * bj);
    }
    *reinterpret_cast<u32x4*>(tail + jc * C * 2) = t0;
    *reinterpret_cast<u32x4*>(tail + jc * C * 2 + 16) = t1;
  }

  // ---- the tail of the record to HBM
  wait_lgkm0();   // this wave's LDS writes are done
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int i = 0; i < (kTailBytes / 16 + 63) / 64; ++i) {
    const int piece = 64 * i + lane;
    if (piece < kTailBytes / 16)
      __builtin_nontemporal_store(*reinterpret_cast<const u32x4*>(tail + 16 * piece),
                                  reinterpret_cast<u32x4*>(rec_out + REC_T + 16 * piece));
  }
}

}  // namespace

hipError_t launch_prep(const PrepArgs& a, hipStream_t s) {
  if (a.lay.chunk == C32) return launch_prep32(a, s);
  if (a.lay.chunk == C64) return launch_prep64(a, s);
  if (a.grid_chunks == 0) return hipSuccess;
  const unsigned hx = (unsigned)((a.H + kWaves - 1) / kWaves);
  const int64_t grid = (int64_t)hx * a.grid_chunks;
  if (grid > INT32_MAX) return hipErrorInvalidValue;
  if (a.precision & KDA_PREC_NEUMANN_FP16)
    hipLaunchKernelGGL(prep_kernel<1>, dim3((unsigned)grid), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL(prep_kernel<0>, dim3((unsigned)grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace kda
