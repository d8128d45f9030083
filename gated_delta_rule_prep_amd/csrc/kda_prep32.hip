// kda_prep32.hip -- chunk-prep kernel for 32-token chunks (gfx950).
//
// The token-parallel stage of the split the pages describe (P1 §二 2.2) for a
// chunk of 32 tokens, built from two 16-token halves.  The pages take 16-token
// chunks so that the in-chunk decay stays within the range of the arithmetic
// (P1 §二 2.1): 2^-G of a 32-token cumulative gate can reach e^160 and
// overflow fp32.  Here each half works exactly as the 16-token kernel does,
// relative to its own start, and the block that couples the halves comes out
// of products of bounded factors only.
//
// P1 = blog post "FlashKDA：月之暗面开源的 Kimi Delta Attention 高性能内核".
//
// Two waves per (chunk, head): wave A takes tokens 0..15, wave B tokens
// 16..31.  Each half h computes, relative to its own first token,
//   G_h (in-half cumulative gate), Khat'_h = kn 2^G_h, Kbar'_h = kn 2^(G_h,15 - G_h),
//   Qhat'_h = qn 2^G_h, gam_h = 2^G_h,15, and L_h, Mqk_h, T_h = (I + L_h)^-1 diag(beta_h)
// as the 16-token kernel does.  Relative to the chunk start, with gA = gam_A:
//   Khat_B = gA Khat'_B, Qhat_B = gA Qhat'_B, Kbar_A = gam_B Kbar'_A, gam = gA gam_B,
// and for token r of B and j of A the exponent G_r - G_j splits into
// G'_B,r (<= 0) plus G_A,15 - G_A,j (<= 0), so
//   X    = Khat'_B Kbar'_A^T           (fp32 MFMA; every factor lies in [-1, 1])
//   L_BA = diag(beta_B) X,   Mqk_BA = Qhat'_B Kbar'_A^T
// and the block inverse of [[I + L_A, 0], [L_BA, I + L_B]] gives
//   T_BA = -T_B X T_A.
// Then -W = -T Khat over all 32 tokens (fp16 MFMA 16x16x32).  A partial chunk
// is padded with a = 0, beta = 0, q = k = 0 as in the 16-token kernel.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

constexpr int kThreads = 128;   // wave 0: tokens 0..15, wave 1: tokens 16..31
constexpr int CH = 16;          // tokens per half
constexpr float kEps = 1e-6f;

struct __align__(16) Smem {
  __align__(16) _Float16 kh[C32][K + 8];   // Khat relative to the chunk start (fp16), 272-byte rows
  __align__(16) float kbA[32][64];         // Kbar'_A, [channel slot 8 j + e][lane]
  __align__(16) float L[2][CH][CH + 4];    // L of each half
  __align__(16) float T[2][CH][CH + 4];    // T of each half, T[r][j]
  __align__(16) float X[CH][CH + 4];       // X, then X T_A
  __align__(16) _Float16 tp[C32][C32 + 8]; // T, row-major, columns at kPermPos (fp16)
  __align__(16) _Float16 mp[C32][C32 + 8]; // Mqk, row-major, columns at kPermPos (fp16)
  float gam[2][K];                         // gam of each half
  float beta[C32];
};

__device__ __forceinline__ void sync_block() { __syncthreads(); }

__global__ __launch_bounds__(kThreads) void prep32_kernel(PrepArgs a) {
  __shared__ Smem sm;
  const int tid = threadIdx.x;
  const int hf = tid >> 6, lane = tid & 63;
  const int64_t H = a.H;
  const int h = blockIdx.y;
  const WsHeader* hdr = reinterpret_cast<const WsHeader*>(a.ws);
  const int chunk = hdr->part_first[a.part] + (int)blockIdx.x;
  if (chunk >= hdr->part_first[a.part + 1]) return;   // the same for both waves: barriers below are safe
  const ChunkEntry ce = reinterpret_cast<const ChunkEntry*>(a.ws + a.lay.chunk_table)[chunk];
  const int r = lane & 15, cq = lane >> 4;
  const int t = CH * hf + r;                                    // token within the chunk
  const bool valid = t < ce.len;
  const int64_t tok = (int64_t)ce.row0 + min(t, ce.len - 1);   // clamped: loads stay in the sequence
  const int64_t base = (tok * H + h) * K + 8 * cq;

  // ---- loads: q, k, g (4 x 16 B each) and beta
  u32x4 qw[4], kw[4], gw[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    qw[j] = *reinterpret_cast<const u32x4*>(a.q + base + 32 * j);
    kw[j] = *reinterpret_cast<const u32x4*>(a.k + base + 32 * j);
    gw[j] = *reinterpret_cast<const u32x4*>(a.g + base + 32 * j);
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
  char* rec = a.ws + a.lay.records + ((int64_t)chunk * a.H + h) * REC32_BYTES;   // chunk-major
  _Float16* rec_qh = reinterpret_cast<_Float16*>(rec + REC32_QH) + t * K;
  _Float16* rec_kb = reinterpret_cast<_Float16*>(rec + REC32_KB) + t * K;
  float* rec_gam = reinterpret_cast<float*>(rec + REC32_GAM);

  // ---- per channel slot of the own half: gate, scan, decay factors, L / Mqk
  f32x4 accL = {0.f, 0.f, 0.f, 0.f}, accM = {0.f, 0.f, 0.f, 0.f};
  float khB[32], qhB[32];   // wave B keeps Khat'_B, Qhat'_B for the coupling block
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int c0 = 32 * j + 8 * cq;
    const f32x4 dtA = *reinterpret_cast<const f32x4*>(a.dt_bias + (int64_t)h * K + c0);
    const f32x4 dtB = *reinterpret_cast<const f32x4*>(a.dt_bias + (int64_t)h * K + c0 + 4);
    float kh[8], qh[8], kb[8], gm[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t wg = gw[j][e >> 1], wq = qw[j][e >> 1], wk = kw[j][e >> 1];
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
      gm[e] = gam;
    }
    if (hf == 0) {
      // Khat_A and Qhat_A are already relative to the chunk start; Kbar'_A
      // waits for gam_B and also feeds the coupling products of wave B.
      u32x4 wkh;
#pragma unroll
      for (int w = 0; w < 4; ++w) wkh[w] = pack_f16(kh[2 * w], kh[2 * w + 1]);
      *reinterpret_cast<u32x4*>(&sm.kh[r][c0]) = wkh;
      const int p0 = 32 * j + kPermPos(8 * cq), p1 = 32 * j + kPermPos(8 * cq + 4);
      *reinterpret_cast<u32x2*>(rec_qh + p0) = u32x2{pack_f16(qh[0], qh[1]), pack_f16(qh[2], qh[3])};
      *reinterpret_cast<u32x2*>(rec_qh + p1) = u32x2{pack_f16(qh[4], qh[5]), pack_f16(qh[6], qh[7])};
#pragma unroll
      for (int e = 0; e < 8; ++e) sm.kbA[8 * j + e][lane] = kb[e];
    } else {
      // Kbar'_B is already relative to the chunk end
      u32x4 wkb;
#pragma unroll
      for (int w = 0; w < 4; ++w) wkb[w] = pack_f16(kb[2 * w], kb[2 * w + 1]);
      *reinterpret_cast<u32x4*>(rec_kb + c0) = wkb;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        khB[8 * j + e] = kh[e];
        qhB[8 * j + e] = qh[e];
      }
    }
    if (r == 0) {
#pragma unroll
      for (int e = 0; e < 8; ++e) sm.gam[hf][c0 + e] = gm[e];
    }
  }

  // ---- L_h (to LDS) and Mqk_h (into the permuted fp16 tile); lane (c, g)
  // holds rows 4g..4g+3 of column c of the 16 x 16 block
  if (cq == 0) sm.beta[t] = beta;
  __builtin_amdgcn_wave_barrier();
  const int lc = lane & 15, lg = lane >> 4;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int rr = 4 * lg + i;
    sm.L[hf][rr][lc] = lc < rr ? sm.beta[CH * hf + rr] * accL[i] : 0.f;
    sm.mp[CH * hf + rr][kPermPos(CH * hf + lc)] = (_Float16)(lc <= rr ? accM[i] : 0.f);
    if (hf == 0) sm.mp[rr][kPermPos(CH + lc)] = (_Float16)0.f;   // tokens of B never reach A
  }
  __builtin_amdgcn_wave_barrier();

  // ---- T_h column jc = column jc of (I + L_h)^-1 times beta_jc (lanes 0..15)
  if (lane < CH) {
    const int jc = lane;
    float x[CH];
#pragma unroll
    for (int rr = 0; rr < CH; ++rr) {
      float s = rr == jc ? 1.f : 0.f;
#pragma unroll
      for (int m = 0; m < rr; ++m) s = fmaf(-sm.L[hf][rr][m], x[m], s);
      x[rr] = s;
    }
    const float bj = sm.beta[CH * hf + jc];
#pragma unroll
    for (int rr = 0; rr < CH; ++rr) {
      const float tv = x[rr] * bj;
      sm.T[hf][rr][jc] = tv;
      sm.tp[CH * hf + rr][kPermPos(CH * hf + jc)] = (_Float16)tv;
      if (hf == 0) sm.tp[rr][kPermPos(CH + jc)] = (_Float16)0.f;
    }
  }
  sync_block();   // both halves' L, T, gam, Kbar'_A and Khat_A are visible

  if (hf == 1) {
    // ---- coupling block: X = Khat'_B Kbar'_A^T, Mqk_BA = Qhat'_B Kbar'_A^T
    f32x4 accX = {0.f, 0.f, 0.f, 0.f}, accQ = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 32; ++s) {
      const float kbv = sm.kbA[s][lane];   // the same (token, channel) slot as this lane's own values
      accX = mfma_f32_k4(khB[s], kbv, accX);
      accQ = mfma_f32_k4(qhB[s], kbv, accQ);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sm.X[4 * lg + i][lc] = accX[i];
      sm.mp[CH + 4 * lg + i][kPermPos(lc)] = (_Float16)accQ[i];
    }
    __builtin_amdgcn_wave_barrier();
    // Y = X T_A
    f32x4 accY = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) accY = mfma_f32_k4(sm.X[lc][4 * q4 + lg], sm.T[0][4 * q4 + lg][lc], accY);
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int i = 0; i < 4; ++i) sm.X[4 * lg + i][lc] = accY[i];
    __builtin_amdgcn_wave_barrier();
    // T_BA = -T_B Y
    f32x4 accT = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) accT = mfma_f32_k4(sm.T[1][lc][4 * q4 + lg], sm.X[4 * q4 + lg][lc], accT);
#pragma unroll
    for (int i = 0; i < 4; ++i) sm.tp[CH + 4 * lg + i][kPermPos(lc)] = (_Float16)(-accT[i]);
    // Khat_B and Qhat_B relative to the chunk start
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c0 = 32 * j + 8 * cq;
      float kv[8], qv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float gA = sm.gam[0][c0 + e];
        kv[e] = khB[8 * j + e] * gA;
        qv[e] = qhB[8 * j + e] * gA;
      }
      u32x4 wkh;
#pragma unroll
      for (int w = 0; w < 4; ++w) wkh[w] = pack_f16(kv[2 * w], kv[2 * w + 1]);
      *reinterpret_cast<u32x4*>(&sm.kh[CH + r][c0]) = wkh;
      const int p0 = 32 * j + kPermPos(8 * cq), p1 = 32 * j + kPermPos(8 * cq + 4);
      *reinterpret_cast<u32x2*>(rec_qh + p0) = u32x2{pack_f16(qv[0], qv[1]), pack_f16(qv[2], qv[3])};
      *reinterpret_cast<u32x2*>(rec_qh + p1) = u32x2{pack_f16(qv[4], qv[5]), pack_f16(qv[6], qv[7])};
    }
  } else {
    // ---- Kbar_A relative to the chunk end, and gam of the whole chunk
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c0 = 32 * j + 8 * cq;
      u32x4 wkb;
#pragma unroll
      for (int w = 0; w < 4; ++w)
        wkb[w] = pack_f16(sm.kbA[8 * j + 2 * w][lane] * sm.gam[1][c0 + 2 * w],
                          sm.kbA[8 * j + 2 * w + 1][lane] * sm.gam[1][c0 + 2 * w + 1]);
      *reinterpret_cast<u32x4*>(rec_kb + c0) = wkb;
    }
#pragma unroll
    for (int c = lane; c < K; c += 64) rec_gam[kGamSlot(c)] = sm.gam[0][c] * sm.gam[1][c];
  }
  sync_block();   // Khat rows 16..31 and the coupling blocks of T and Mqk are in place

  // ---- -W rows of the own half: W^T tile n (channels 16n..16n+15) =
  // Khat^T T^T over all 32 tokens; the k-order of both operands is kPermCh
  // (tokens 4g..4g+3 and 16+4g..16+4g+3 in lane group g)
  const f16x8 bT = *reinterpret_cast<const f16x8*>(&sm.tp[CH * hf + lc][8 * lg]);
  _Float16* rec_nw = reinterpret_cast<_Float16*>(rec + REC32_NW) + (CH * hf + lc) * K;
#pragma unroll
  for (int n = 0; n < 8; ++n) {
    const f16x4 k0 = lds_read_tr(&sm.kh[0][16 * n], K + 8, lane);
    const f16x4 k1 = lds_read_tr(&sm.kh[CH][16 * n], K + 8, lane);
    const f16x8 aK = {k0[0], k0[1], k0[2], k0[3], k1[0], k1[1], k1[2], k1[3]};
    const f32x4 w4 = mfma_f16_k32(aK, bT, f32x4{0.f, 0.f, 0.f, 0.f});
    const int c = 16 * n + 4 * lg;
    *reinterpret_cast<u32x2*>(rec_nw + (c & ~31) + kPermPos(c & 31)) =
        u32x2{pack_f16(-w4[0], -w4[1]), pack_f16(-w4[2], -w4[3])};
  }

  // ---- T and Mqk tiles to the record: 32 rows x 64 B each, one 16-byte piece per thread
  {
    const int row = tid >> 2, piece = tid & 3;
    *reinterpret_cast<u32x4*>(rec + REC32_T + row * 64 + piece * 16) =
        *reinterpret_cast<const u32x4*>(&sm.tp[row][8 * piece]);
    *reinterpret_cast<u32x4*>(rec + REC32_MQK + row * 64 + piece * 16) =
        *reinterpret_cast<const u32x4*>(&sm.mp[row][8 * piece]);
  }
}

}  // namespace

hipError_t launch_prep32(const PrepArgs& a, hipStream_t s) {
  if (a.grid_chunks == 0) return hipSuccess;
  hipLaunchKernelGGL(prep32_kernel, dim3((unsigned)a.grid_chunks, (unsigned)a.H), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace kda
