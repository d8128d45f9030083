// kda_prep64.hip -- chunk-prep kernel for 64-token chunks (gfx950).
//
// The token-parallel stage of the split the pages describe (P1 §二 2.2) for
// the 64-token chunk of Flash Linear Attention, which P1 §二 2.1 sets against
// its own 16: the cumulative gate of 64 tokens at lower_bound = -5 spans e^320,
// so the in-chunk decay factors cannot be formed relative to one chunk start
// in fp32.  The chunk is built from four 16-token blocks, each computed exactly
// as in the 16-token kernel relative to its own start, and every block that
// couples two of them comes out of products of bounded factors only.
//
// P1 = blog post "FlashKDA：月之暗面开源的 Kimi Delta Attention 高性能内核".
//
// One wave per block (wave w: tokens 16w .. 16w + 15).  Relative to its own
// start, block w has G_w (in-block cumulative gate), Khat'_w = kn 2^G_w,
// Qhat'_w = qn 2^G_w, Kbar'_w = kn 2^(G_w,15 - G_w), gam_w = 2^G_w,15, and
// L_ww, Mqk_ww, T_ww = (I + L_ww)^-1 diag(beta_w) as in the 16-token kernel.
// For token r of block i and j of block m < i the exponent splits into
// G'_i,r (<= 0), the whole blocks strictly between (<= 0, per channel) and
// G_m,15 - G_m,j (<= 0), so with D_mi = diag(prod_{m<l<i} gam_l):
//   X_im = Khat'_i D_mi Kbar'_m^T,  Mqk_im = Qhat'_i D_mi Kbar'_m^T   (fp32 MFMA)
// and L_im = diag(beta_i) X_im.  Block forward substitution on I + L gives
//   T_ij = -T_ii sum_{m=j}^{i-1} X_im T_mj      (i > j)
// block row by block row.  Relative to the chunk start / end:
//   Khat_i = Khat'_i prod_{l<i} gam_l, Qhat_i likewise, Kbar_i = Kbar'_i
//   prod_{l>i} gam_l, gam = prod_l gam_l,
// and -W = -T Khat over the 64 tokens (fp16 MFMA 16x16x32).  A partial chunk
// is padded with a = 0, beta = 0, q = k = 0 as in the 16-token kernel.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

constexpr int kThreads = 256;   // wave w: tokens 16w .. 16w + 15
constexpr int CH = 16;          // tokens per block
constexpr int NB = C64 / CH;    // blocks per chunk
constexpr float kEps = 1e-6f;

// Block (i, j), i >= j, of T in Smem::T; block (i, j), i > j, of X.
__device__ __forceinline__ int tri(int i, int j) { return i * (i + 1) / 2 + j; }
__device__ __forceinline__ int lowx(int i, int j) { return i * (i - 1) / 2 + j; }
// Stored column of token c (0..63) in a row of T or Mqk: the 32-token half,
// then kPermCh order within it.
__device__ __forceinline__ int pos64(int c) { return 32 * (c >> 5) + kPermPos(c & 31); }

typedef float Blk[CH][CH + 4];

// Regions that are never live at the same time share storage: Kbar' is read
// by the coupling products and the rescale, Khat and the substitution scratch
// are written only after the barrier that ends them; L_ww is dead once T_ww
// is formed, before the X blocks are written.  65.8 KB: two workgroups per CU.
struct __align__(16) Smem {
  union {
    float kbp[NB - 1][32][64];             // Kbar'_m of blocks 0..2, [channel slot 8 j + e][lane]
    struct {
      __align__(16) _Float16 kh[C64][K + 8];   // Khat relative to the chunk start (fp16), 272-byte rows
      Blk S[NB];                               // per-wave scratch of the block substitution
    } c;
  } u;
  union {
    Blk L[NB];                             // L_ww of each block
    Blk X[NB * (NB - 1) / 2];              // X_im, i > m
  } lx;
  Blk T[NB * (NB + 1) / 2];                // T_ij, i >= j, fp32
  __align__(16) _Float16 tp[C64][C64 + 8]; // T, row-major, columns at pos64 (fp16)
  __align__(16) _Float16 mp[C64][C64 + 8]; // Mqk, row-major, columns at pos64 (fp16)
  __align__(16) float gam[NB][K];          // gam of each block
  float beta[C64];
};

__device__ __forceinline__ void sync_block() { __syncthreads(); }

// gam of blocks 0..3 at the lane's 8 channels c0 .. c0 + 7.
struct Gam8 {
  f32x4 lo[NB], hi[NB];
  __device__ __forceinline__ float at(int l, int e) const { return e < 4 ? lo[l][e] : hi[l][e - 4]; }
};
__device__ __forceinline__ Gam8 gam8(const Smem& sm, int c0) {
  Gam8 g;
#pragma unroll
  for (int l = 0; l < NB; ++l) {
    g.lo[l] = *reinterpret_cast<const f32x4*>(&sm.gam[l][c0]);
    g.hi[l] = *reinterpret_cast<const f32x4*>(&sm.gam[l][c0 + 4]);
  }
  return g;
}

// The work of wave W (block W, tokens 16W .. 16W + 15) of one (chunk, head).
// Every wave passes the same sequence of workgroup barriers.
template <int W>
__device__ __forceinline__ void prep64_wave(const PrepArgs& a, Smem& sm, const ChunkEntry& ce, int chunk, int h,
                                            int tid) {
  const int lane = tid & 63;
  const int64_t H = a.H;
  const int r = lane & 15, cq = lane >> 4;
  const int lc = lane & 15, lg = lane >> 4;
  const int t = CH * W + r;                                     // token within the chunk
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
    for (int e = 0; e < 4; ++e) {
      const float q0 = bf16_lo(qw[j][e]), q1 = bf16_hi(qw[j][e]);
      const float k0 = bf16_lo(kw[j][e]), k1 = bf16_hi(kw[j][e]);
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
  char* rec = a.ws + a.lay.records + ((int64_t)chunk * a.H + h) * REC64_BYTES;   // chunk-major
  _Float16* rec_qh = reinterpret_cast<_Float16*>(rec + REC64_QH) + t * K;
  _Float16* rec_kb = reinterpret_cast<_Float16*>(rec + REC64_KB) + t * K;
  float* rec_gam = reinterpret_cast<float*>(rec + REC64_GAM);

  // ---- per channel slot of the own block: gate, scan, decay factors, L / Mqk
  f32x4 accL = {0.f, 0.f, 0.f, 0.f}, accM = {0.f, 0.f, 0.f, 0.f};
  float khv[32], qhv[32];   // Khat'_W, Qhat'_W of the lane's token at its 32 channel slots
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int c0 = 32 * j + 8 * cq;
    const f32x4 dtA = *reinterpret_cast<const f32x4*>(a.dt_bias + (int64_t)h * K + c0);
    const f32x4 dtB = *reinterpret_cast<const f32x4*>(a.dt_bias + (int64_t)h * K + c0 + 4);
    float kb[8], gm[8];
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
      khv[8 * j + e] = kP;
      qhv[8 * j + e] = qP;
      kb[e] = kI * gam;
      gm[e] = gam;
    }
    if constexpr (W < NB - 1) {
      // Kbar'_W waits for the later blocks' gam and feeds the coupling products
#pragma unroll
      for (int e = 0; e < 8; ++e) sm.u.kbp[W][8 * j + e][lane] = kb[e];
    } else {
      // the last block's Kbar' is already relative to the chunk end
      u32x4 wkb;
#pragma unroll
      for (int e = 0; e < 4; ++e) wkb[e] = pack_f16(kb[2 * e], kb[2 * e + 1]);
      *reinterpret_cast<u32x4*>(rec_kb + c0) = wkb;
    }
    if (r == 0) {
      *reinterpret_cast<f32x4*>(&sm.gam[W][c0]) = f32x4{gm[0], gm[1], gm[2], gm[3]};
      *reinterpret_cast<f32x4*>(&sm.gam[W][c0 + 4]) = f32x4{gm[4], gm[5], gm[6], gm[7]};
    }
  }

  // ---- L_WW (to LDS) and Mqk_WW (into the fp16 tile, zeros to its right);
  // lane (c, g) holds rows 4g..4g+3 of column c of the 16 x 16 block
  if (cq == 0) sm.beta[t] = beta;
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int rr = 4 * lg + i;
    sm.lx.L[W][rr][lc] = lc < rr ? sm.beta[CH * W + rr] * accL[i] : 0.f;
    sm.mp[CH * W + rr][pos64(CH * W + lc)] = (_Float16)(lc <= rr ? accM[i] : 0.f);
#pragma unroll
    for (int jb = W + 1; jb < NB; ++jb) sm.mp[CH * W + rr][pos64(CH * jb + lc)] = (_Float16)0.f;
  }
  __builtin_amdgcn_wave_barrier();

  // ---- T_WW column jc = column jc of (I + L_WW)^-1 times beta_jc (lanes 0..15)
  if (lane < CH) {
    const int jc = lane;
    float x[CH];
#pragma unroll
    for (int rr = 0; rr < CH; ++rr) {
      float sacc = rr == jc ? 1.f : 0.f;
#pragma unroll
      for (int m = 0; m < rr; ++m) sacc = fmaf(-sm.lx.L[W][rr][m], x[m], sacc);
      x[rr] = sacc;
    }
    const float bj = sm.beta[CH * W + jc];
#pragma unroll
    for (int rr = 0; rr < CH; ++rr) {
      const float tv = x[rr] * bj;
      sm.T[tri(W, W)][rr][jc] = tv;
      sm.tp[CH * W + rr][pos64(CH * W + jc)] = (_Float16)tv;
#pragma unroll
      for (int jb = W + 1; jb < NB; ++jb) sm.tp[CH * W + rr][pos64(CH * jb + jc)] = (_Float16)0.f;
    }
  }
  sync_block();   // every block's L, T_ww, gam, beta and Kbar' are visible; L is dead

  // ---- coupling blocks of the own block row, X_Wm and Mqk_Wm for m < W, and
  // the rescale of the own rows to the chunk start / end
  f32x4 accX[NB - 1], accQ[NB - 1];
#pragma unroll
  for (int m = 0; m < NB - 1; ++m) {
    accX[m] = f32x4{0.f, 0.f, 0.f, 0.f};
    accQ[m] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  u32x4 khw[4];   // Khat_W (fp16), written to LDS once Kbar' is dead
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int c0 = 32 * j + 8 * cq;
    const Gam8 g = gam8(sm, c0);
    float kv[8], qv[8], kb[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int sl = 8 * j + e;
#pragma unroll
      for (int m = 0; m < W; ++m) {
        float dmid = 1.f;   // decay of the whole blocks strictly between m and W
#pragma unroll
        for (int l = m + 1; l < W; ++l) dmid *= g.at(l, e);
        const float kbv = sm.u.kbp[m][sl][lane];   // the same (token, channel) slot as this lane's own values
        accX[m] = mfma_f32_k4(khv[sl] * dmid, kbv, accX[m]);
        accQ[m] = mfma_f32_k4(qhv[sl] * dmid, kbv, accQ[m]);
      }
      float pre = 1.f, post = 1.f;
#pragma unroll
      for (int l = 0; l < W; ++l) pre *= g.at(l, e);
#pragma unroll
      for (int l = W + 1; l < NB; ++l) post *= g.at(l, e);
      kv[e] = khv[sl] * pre;
      qv[e] = qhv[sl] * pre;
      if constexpr (W < NB - 1) kb[e] = sm.u.kbp[W][sl][lane] * post;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) khw[j][e] = pack_f16(kv[2 * e], kv[2 * e + 1]);
    const int p0 = 32 * j + kPermPos(8 * cq), p1 = 32 * j + kPermPos(8 * cq + 4);
    *reinterpret_cast<u32x2*>(rec_qh + p0) = u32x2{pack_f16(qv[0], qv[1]), pack_f16(qv[2], qv[3])};
    *reinterpret_cast<u32x2*>(rec_qh + p1) = u32x2{pack_f16(qv[4], qv[5]), pack_f16(qv[6], qv[7])};
    if constexpr (W < NB - 1) {
      u32x4 wkb;
#pragma unroll
      for (int e = 0; e < 4; ++e) wkb[e] = pack_f16(kb[2 * e], kb[2 * e + 1]);
      *reinterpret_cast<u32x4*>(rec_kb + c0) = wkb;
    }
  }
#pragma unroll
  for (int m = 0; m < W; ++m)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sm.lx.X[lowx(W, m)][4 * lg + i][lc] = accX[m][i];
      sm.mp[CH * W + 4 * lg + i][pos64(CH * m + lc)] = (_Float16)accQ[m][i];
    }
  if constexpr (W == 0) {
    for (int c = lane; c < K; c += 64)
      rec_gam[kGamSlot(c)] = sm.gam[0][c] * sm.gam[1][c] * sm.gam[2][c] * sm.gam[3][c];
  }
  sync_block();   // the X blocks and coupling blocks of Mqk are in place; Kbar' is dead

#pragma unroll
  for (int j = 0; j < 4; ++j) *reinterpret_cast<u32x4*>(&sm.u.c.kh[t][32 * j + 8 * cq]) = khw[j];

  // ---- block forward substitution, one block row at a time (row i by wave i)
#pragma unroll
  for (int i = 1; i < NB; ++i) {
    if (i == W) {
#pragma unroll
      for (int j = 0; j < i; ++j) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = j; m < i; ++m) {
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4)
            acc = mfma_f32_k4(sm.lx.X[lowx(i, m)][lc][4 * q4 + lg], sm.T[tri(m, j)][4 * q4 + lg][lc], acc);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) sm.u.c.S[W][4 * lg + e][lc] = acc[e];
        __builtin_amdgcn_wave_barrier();
        f32x4 tt = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          tt = mfma_f32_k4(sm.T[tri(i, i)][lc][4 * q4 + lg], sm.u.c.S[W][4 * q4 + lg][lc], tt);
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sm.T[tri(i, j)][4 * lg + e][lc] = -tt[e];
          sm.tp[CH * i + 4 * lg + e][pos64(CH * j + lc)] = (_Float16)(-tt[e]);
        }
      }
    }
    sync_block();   // block row i of T (and, the first time, every Khat row) is visible
  }

  // ---- -W rows of the own block: W^T tile n (channels 16n..16n+15) =
  // Khat^T T^T over the chunk's tokens, one 32-token half per MFMA, k in
  // kPermCh order (tokens 4g..4g+3 and 16+4g..16+4g+3 of the half in lane group g)
  {
    constexpr int halves = W >= 2 ? 2 : 1;   // T row block W has no tokens past its own half
    f16x8 bT[halves];
#pragma unroll
    for (int u = 0; u < halves; ++u)
      bT[u] = *reinterpret_cast<const f16x8*>(&sm.tp[CH * W + lc][32 * u + 8 * lg]);
    _Float16* rec_nw = reinterpret_cast<_Float16*>(rec + REC64_NW) + (CH * W + lc) * K;
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      f32x4 w4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int u = 0; u < halves; ++u) {
        const f16x4 k0 = lds_read_tr(&sm.u.c.kh[32 * u][16 * n], K + 8, lane);
        const f16x4 k1 = lds_read_tr(&sm.u.c.kh[32 * u + CH][16 * n], K + 8, lane);
        const f16x8 aK = {k0[0], k0[1], k0[2], k0[3], k1[0], k1[1], k1[2], k1[3]};
        w4 = mfma_f16_k32(aK, bT[u], w4);
      }
      const int c = 16 * n + 4 * lg;
      *reinterpret_cast<u32x2*>(rec_nw + (c & ~31) + kPermPos(c & 31)) =
          u32x2{pack_f16(-w4[0], -w4[1]), pack_f16(-w4[2], -w4[3])};
    }
  }

  // ---- T and Mqk to the record: 8 blocks of 16 rows x 64 B each, 16-byte pieces
  for (int i = tid; i < 512; i += kThreads) {
    const int blk = i >> 6, row = (i >> 2) & 15, piece = i & 3;
    const int tt = blk >> 1, u = blk & 1;
    *reinterpret_cast<u32x4*>(rec + REC64_T + blk * 1024 + row * 64 + piece * 16) =
        *reinterpret_cast<const u32x4*>(&sm.tp[CH * tt + row][32 * u + 8 * piece]);
    *reinterpret_cast<u32x4*>(rec + REC64_MQK + blk * 1024 + row * 64 + piece * 16) =
        *reinterpret_cast<const u32x4*>(&sm.mp[CH * tt + row][32 * u + 8 * piece]);
  }
}

__global__ __launch_bounds__(kThreads) void prep64_kernel(PrepArgs a) {
  __shared__ Smem sm;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = blockIdx.y;
  const WsHeader* hdr = reinterpret_cast<const WsHeader*>(a.ws);
  const int chunk = hdr->part_first[a.part] + (int)blockIdx.x;
  if (chunk >= hdr->part_first[a.part + 1]) return;   // the same for every wave: barriers below are safe
  const ChunkEntry ce = reinterpret_cast<const ChunkEntry*>(a.ws + a.lay.chunk_table)[chunk];
  switch (w) {
    case 0: prep64_wave<0>(a, sm, ce, chunk, h, tid); break;
    case 1: prep64_wave<1>(a, sm, ce, chunk, h, tid); break;
    case 2: prep64_wave<2>(a, sm, ce, chunk, h, tid); break;
    default: prep64_wave<3>(a, sm, ce, chunk, h, tid); break;
  }
}

}  // namespace

hipError_t launch_prep64(const PrepArgs& a, hipStream_t s) {
  if (a.grid_chunks == 0) return hipSuccess;
  hipLaunchKernelGGL(prep64_kernel, dim3((unsigned)a.grid_chunks, (unsigned)a.H), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace kda
