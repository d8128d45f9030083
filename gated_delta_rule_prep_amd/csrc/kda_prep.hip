// kda_prep.hip -- token-parallel chunk-prep kernel for gfx950.
//
// One workgroup (256 threads = 4 waves) per (chunk, head); chunks come from the
// scheduler's table, so a chunk never straddles two sequences and a partial
// chunk is padded with a = 0, beta = 0, q = k = 0, which leaves every real
// token's result unchanged.  This is the first of the two stages the pages
// split the forward pass into (P1 §二 2.2: gate activation, L2 norm, decay,
// L / Mqk, inverse), with the base-2 exponentials of P1 §二 2.4 taken from the
// native v_exp_f32 (which computes 2^x).
//
// P1 = blog post "FlashKDA：月之暗面开源的 Kimi Delta Attention 高性能内核".
//
// Per chunk of 16 tokens r with per-channel log2 decay a2 (so a = a2 / log2 e):
//   a2[r][i] = lower_bound * log2(e) * sigmoid(exp(A_log) * (g + dt_bias))
//   G[r][i]  = sum_{j<=r} a2[j][i]        P = 2^G,  Pinv = 2^-G,  gam = 2^G[15]
//   kn = k / |k|, qn = scale * q / |q|     (|x| = sqrt(sum x^2 + 1e-6))
//   L   = strict_lower(diag(beta) (kn P)(kn Pinv)^T)       fp32 MFMA
//   Mqk = lower_incl((qn P)(kn Pinv)^T)                     fp32 MFMA
//   T   = (I + L)^-1 diag(beta)     forward substitution in fp32 (L is strictly
//                                   lower, so the inverse is exact: no series
//                                   truncation and no pivoting)
//   W   = T (kn P)                  fp16 MFMA, fp32 sum
// and writes the record {Qhat = qn P, -W, Kbar^T = (kn Pinv gam)^T, T, Mqk, gam}.
// The pair of factors (kn P, kn Pinv) spans at most 2^(+-16 * 5 * log2 e) =
// e^(+-80) at lower_bound = -5, inside the fp32 exponent range (the range
// argument of P1 §二 2.1).  Their products are taken on the fp32 matrix cores:
// rounding these factors to a 16-bit type costs about 2^-9 of every L / Mqk
// entry, which alone used more than the whole output error budget.  Everything
// the recurrence reads is bounded by 1 (or by scale) and is stored in fp16.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

constexpr int kThreads = 256;
constexpr float kEps = 1e-6f;

// LDS strides (elements) padded against bank conflicts where cheap.
constexpr int SA = K + 4;      // fp32 [16][SA] gate / cumsum
constexpr int SB = K + 8;      // bf16/fp16 [16][SB] row-major operands
constexpr int SKT = C + 8;     // fp16 [128][SKT] transposed operands (48-byte rows)

constexpr int SF = K + 4;      // fp32 [16][SF] L / Mqk operands

struct __align__(16) PrepSmem {
  union {
    float a2[C][SA];             // gate (log2 units), then its in-chunk cumsum
    float part[2][4][C][C + 1];  // per-wave partial L / Mqk sums
  } u0;
  float gam2[K];                 // G[last] per channel (log2 units)
  float beta[C];
  float L[C][C + 1];
  union {
    struct {
      __align__(16) float kP[C][SF];   // kn * P      (A operand of L)
      __align__(16) float qP[C][SF];   // qn * P      (A operand of Mqk)
      __align__(16) float kI[C][SF];   // kn * Pinv   (B operand of L and Mqk)
    } f;
    __align__(16) _Float16 nW[C][SB];  // -W in the record's permuted channel order
  } u1;
  __align__(16) _Float16 kHt[K][SKT]; // (kn * P)^T  fp16 (B operand of W = T Khat)
  __align__(16) _Float16 kBt[K][SKT]; // Kbar^T      fp16 (record)
  __align__(16) _Float16 Tm[C][C + 8];
  __align__(16) _Float16 Mq[C][C + 8];
  __align__(16) _Float16 qH[C][SB];   // Qhat in the record's permuted channel order
};

__global__ __launch_bounds__(kThreads) void prep_kernel(PrepArgs a) {
  __shared__ PrepSmem sm;
  const WsHeader* hdr = reinterpret_cast<const WsHeader*>(a.ws);
  const int chunk = blockIdx.x;
  if (chunk >= hdr->chunk_count) return;  // capacity bound: unused slots exit
  const int h = blockIdx.y;
  const ChunkEntry ce = reinterpret_cast<const ChunkEntry*>(a.ws + a.lay.chunk_table)[chunk];
  const int64_t H = a.H;
  const int tid = threadIdx.x;
  const int r = tid >> 4;        // token within the chunk
  const int cg = tid & 15;       // channels 8*cg .. 8*cg+7
  const bool valid = r < ce.len;
  const int64_t row = (int64_t)ce.row0 + r;

  // ---- load q, k, g (16 B each) and beta
  u32x4 qw = {0, 0, 0, 0}, kw = {0, 0, 0, 0}, gw = {0, 0, 0, 0};
  float braw = 0.f;
  if (valid) {
    const int64_t off = (row * H + h) * K + 8 * cg;
    qw = *reinterpret_cast<const u32x4*>(a.q + off);
    kw = *reinterpret_cast<const u32x4*>(a.k + off);
    gw = *reinterpret_cast<const u32x4*>(a.g + off);
    braw = bf16_to_f32(a.beta[row * H + h]);
  }
  float qv[8], kv[8], gv[8];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    qv[2 * j] = bf16_lo(qw[j]); qv[2 * j + 1] = bf16_hi(qw[j]);
    kv[2 * j] = bf16_lo(kw[j]); kv[2 * j + 1] = bf16_hi(kw[j]);
    gv[2 * j] = bf16_lo(gw[j]); gv[2 * j + 1] = bf16_hi(gw[j]);
  }

  // ---- gate activation, in log2 units: lb*log2e * sigmoid(A * (g + dt))
  const float A = expf(a.A_log[h]);
  const float lb2 = a.lower_bound * kLog2e;
  const float Ax = -A * kLog2e;   // sigmoid(x) = 1 / (1 + 2^(-x log2 e))
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float dt = a.dt_bias[(int64_t)h * K + 8 * cg + j];
    const float e = fast_exp2(Ax * (gv[j] + dt));
    const float a2 = valid ? lb2 * fast_rcp(1.f + e) : 0.f;
    sm.u0.a2[r][8 * cg + j] = a2;
  }

  // ---- L2 norms (16 lanes share a token)
  float sq = 0.f, sk = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    sq = fmaf(qv[j], qv[j], sq);
    sk = fmaf(kv[j], kv[j], sk);
  }
#pragma unroll
  for (int m = 1; m < 16; m <<= 1) {
    sq += __shfl_xor(sq, m);
    sk += __shfl_xor(sk, m);
  }
  const float rq = a.scale / sqrtf(sq + kEps);
  const float rk = 1.f / sqrtf(sk + kEps);
  if (cg == 0) sm.beta[r] = valid ? 1.f / (1.f + expf(-braw)) : 0.f;
  __syncthreads();

  // ---- in-chunk cumulative sum along tokens (one channel per thread)
  if (tid < K) {
    float s = 0.f;
#pragma unroll
    for (int t = 0; t < C; ++t) {
      s += sm.u0.a2[t][tid];
      sm.u0.a2[t][tid] = s;
    }
    sm.gam2[tid] = s;
  }
  __syncthreads();

  // ---- decayed operands
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int c = 8 * cg + j;
    const float G = sm.u0.a2[r][c];
    const float P = fast_exp2(G);
    const float Pinv = fast_exp2(-G);
    const float gam = fast_exp2(sm.gam2[c]);
    const float kn = kv[j] * rk, qn = qv[j] * rq;
    const float kP = kn * P, kPi = kn * Pinv;
    sm.u1.f.kP[r][c] = kP;
    sm.u1.f.qP[r][c] = qn * P;
    sm.u1.f.kI[r][c] = kPi;
    sm.kHt[c][r] = (_Float16)kP;
    sm.kBt[c][r] = (_Float16)(kPi * gam);
    const int pc = (c & ~31) + kPermPos(c & 31);
    sm.qH[r][pc] = (_Float16)(qn * P);
  }
  __syncthreads();

  const int wave = tid >> 6, lane = tid & 63, lg = lane >> 4, lc = lane & 15;

  // ---- L and Mqk: 16x16, reduce over 128 channels on the fp32 matrix cores.
  // Wave w reduces channels [32w, 32w + 32): in step s lane group lg feeds
  // channel 32w + 8lg + s (the reduction order is free), then the four partial
  // sums are added in LDS.
  {
    f32x4 accL = {0.f, 0.f, 0.f, 0.f}, accM = {0.f, 0.f, 0.f, 0.f};
    const int c0 = 32 * wave + 8 * lg;
    const f32x4 k0 = *reinterpret_cast<const f32x4*>(&sm.u1.f.kP[lc][c0]);
    const f32x4 k1 = *reinterpret_cast<const f32x4*>(&sm.u1.f.kP[lc][c0 + 4]);
    const f32x4 q0 = *reinterpret_cast<const f32x4*>(&sm.u1.f.qP[lc][c0]);
    const f32x4 q1 = *reinterpret_cast<const f32x4*>(&sm.u1.f.qP[lc][c0 + 4]);
    const f32x4 i0 = *reinterpret_cast<const f32x4*>(&sm.u1.f.kI[lc][c0]);
    const f32x4 i1 = *reinterpret_cast<const f32x4*>(&sm.u1.f.kI[lc][c0 + 4]);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      accL = mfma_f32_k4(k0[s], i0[s], accL);
      accM = mfma_f32_k4(q0[s], i0[s], accM);
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      accL = mfma_f32_k4(k1[s], i1[s], accL);
      accM = mfma_f32_k4(q1[s], i1[s], accM);
    }
    // a2 (aliased by part) was last read before the barrier above
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sm.u0.part[0][wave][4 * lg + i][lc] = accL[i];
      sm.u0.part[1][wave][4 * lg + i][lc] = accM[i];
    }
  }
  __syncthreads();
  {
    const int rr = tid >> 4, j = tid & 15;
    const float sL = sm.u0.part[0][0][rr][j] + sm.u0.part[0][1][rr][j] + sm.u0.part[0][2][rr][j] +
                     sm.u0.part[0][3][rr][j];
    const float sM = sm.u0.part[1][0][rr][j] + sm.u0.part[1][1][rr][j] + sm.u0.part[1][2][rr][j] +
                     sm.u0.part[1][3][rr][j];
    sm.L[rr][j] = j < rr ? sm.beta[rr] * sL : 0.f;
    sm.Mq[rr][j] = (_Float16)(j <= rr ? sM : 0.f);
  }
  __syncthreads();

  // ---- T = (I + L)^-1 diag(beta): column j by forward substitution
  if (tid < C) {
    const int j = tid;
    float x[C];
#pragma unroll
    for (int rr = 0; rr < C; ++rr) {
      float s = rr == j ? 1.f : 0.f;
#pragma unroll
      for (int m = 0; m < rr; ++m) s = fmaf(-sm.L[rr][m], x[m], s);
      x[rr] = s;
    }
    const float bj = sm.beta[j];
#pragma unroll
    for (int rr = 0; rr < C; ++rr) sm.Tm[rr][j] = (_Float16)(x[rr] * bj);
  }
  __syncthreads();

  // ---- W = T Khat: each wave two 16-channel tiles; store -W permuted
  {
    const f16x4 at = *reinterpret_cast<const f16x4*>(&sm.Tm[lc][4 * lg]);
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const int n0 = 32 * wave + 16 * nt;
      const f16x4 bk = *reinterpret_cast<const f16x4*>(&sm.kHt[n0 + lc][4 * lg]);
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      acc = mfma_f16_k16(at, bk, acc);
      const int c = n0 + lc;
      const int pc = (c & ~31) + kPermPos(c & 31);
#pragma unroll
      for (int i = 0; i < 4; ++i) sm.u1.nW[4 * lg + i][pc] = (_Float16)(-acc[i]);
    }
  }
  __syncthreads();

  // ---- write the record (coalesced 16-byte stores)
  char* rec = a.ws + a.lay.records + ((int64_t)h * a.lay.max_chunks + chunk) * REC_BYTES;
  {
    // Qhat and -W: 16 rows x 256 B each -> 256 threads x 16 B per matrix
    const int rr = tid >> 4, c8 = (tid & 15) * 8;
    *reinterpret_cast<u32x4*>(rec + REC_QH + (rr * K + c8) * 2) =
        *reinterpret_cast<const u32x4*>(&sm.qH[rr][c8]);
    *reinterpret_cast<u32x4*>(rec + REC_NW + (rr * K + c8) * 2) =
        *reinterpret_cast<const u32x4*>(&sm.u1.nW[rr][c8]);
    // Kbar^T: 128 rows x 32 B -> 256 threads x 16 B
    const int kr = tid >> 1, half = (tid & 1) * 8;
    *reinterpret_cast<u32x4*>(rec + REC_KBT + (kr * C + half) * 2) =
        *reinterpret_cast<const u32x4*>(&sm.kBt[kr][half]);
    // T and Mqk: 16 rows x 32 B each -> 32 threads x 16 B each
    if (tid < 32) {
      const int tr = tid >> 1, th = (tid & 1) * 8;
      *reinterpret_cast<u32x4*>(rec + REC_T + (tr * C + th) * 2) =
          *reinterpret_cast<const u32x4*>(&sm.Tm[tr][th]);
    } else if (tid < 64) {
      const int t2 = tid - 32, tr = t2 >> 1, th = (t2 & 1) * 8;
      *reinterpret_cast<u32x4*>(rec + REC_MQK + (tr * C + th) * 2) =
          *reinterpret_cast<const u32x4*>(&sm.Mq[tr][th]);
    } else if (tid < 96) {
      const int t3 = tid - 64;
      f32x4 gv4;
#pragma unroll
      for (int i = 0; i < 4; ++i) gv4[i] = fast_exp2(sm.gam2[4 * t3 + i]);
      *reinterpret_cast<f32x4*>(rec + REC_GAM + 16 * t3) = gv4;
    }
  }
}

}  // namespace

hipError_t launch_prep(const PrepArgs& a, hipStream_t s) {
  if (a.lay.max_chunks == 0) return hipSuccess;
  hipLaunchKernelGGL(prep_kernel, dim3((unsigned)a.lay.max_chunks, (unsigned)a.H), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace kda
