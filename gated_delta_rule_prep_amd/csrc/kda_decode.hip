// kda_decode.hip -- single-token (decode) step of KDA for gfx950.
//
// One new token per sequence: the recurrence itself, token by token, with no
// chunking (P1 §一: the state is decayed per channel by the activated gate,
// corrected by the beta-weighted delta-rule rank-1 update and read out by the
// query; the activations are those of the chunked kernels):
//   a = lower_bound * sigmoid(exp(A_log) * (g + dt_bias)),  beta = sigmoid(beta)
//   kn = k / |k|,  qn = scale * q / |q|                  (|x| = sqrt(sum x^2 + 1e-6))
//   S[v][k] *= exp(a[k]);  u[v] = sum_k S[v][k] kn[k];  e[v] = beta (v[v] - u[v])
//   S[v][k] += kn[k] e[v];  o[v] = sum_k S[v][k] qn[k]
// with the state stored as [N][H][V][K] (K contiguous).  The step reads and
// writes the whole 128 x 128 state of every (sequence, head) once, so it is
// bound by the state bytes.
//
// P1 = blog post "FlashKDA：月之暗面开源的 Kimi Delta Attention 高性能内核".
//
// One workgroup of four waves per (sequence, head).  Wave w owns state rows
// 32 w .. 32 w + 31; in each of its 16 loads the wave reads 1 KB of contiguous
// state (two rows): lane l holds row 32 w + 2 i + l / 32, channels
// 4 (l % 32) .. +3.  The dot products over the 128 channels are 16 partial sums
// per lane reduced over the 32 lanes of a row by a transposing butterfly (16
// exchanges for all 16 rows), after which lanes 2 i and 2 i + 1 of each half
// hold the sum of row 2 i + half.
#include "kda_device.h"
#include "kda_internal.h"
#include "../../include/kda.h"

namespace kda {
namespace {

constexpr int kThreads = 256;
constexpr float kEps = 1e-6f;

// x from lane l ^ M within each group of 32 lanes (ds_swizzle in bit-mask
// mode: and-mask 31, xor-mask M; no LDS memory is touched).
template <int M>
__device__ __forceinline__ float xor32(float x) {
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x1F | (M << 10)));
}

template <int M, int CNT, int R>
__device__ __forceinline__ void fold(float (&x)[R], int kq) {
  const bool keep_lo = (kq & M) == 0;
#pragma unroll
  for (int j = 0; j < CNT / 2; ++j) {
    const float lo = x[j], hi = x[j + CNT / 2];
    const float recv = xor32<M>(keep_lo ? hi : lo);
    x[j] = (keep_lo ? lo : hi) + recv;
  }
}

// Sum of x[i] (i < R) over the LPR lanes of a row group (LPR = 2 R), returned
// in the lanes with (lane % LPR) / 2 == i (both lanes of the pair get it).
template <int R>
__device__ __forceinline__ float row_sums(float (&x)[R], int kq) {
  if constexpr (R >= 16) fold<16, 16>(x, kq);
  if constexpr (R >= 8) fold<8, 8>(x, kq);
  fold<4, 4>(x, kq);
  fold<2, 2>(x, kq);
  return x[0] + xor32<1>(x[0]);
}

template <int M>
__device__ __forceinline__ float lanes_sum(float x) {   // sum over aligned groups of 2M lanes
  if constexpr (M >= 1) x += xor32<1>(x);
  if constexpr (M >= 2) x += xor32<2>(x);
  if constexpr (M >= 4) x += xor32<4>(x);
  if constexpr (M >= 8) x += xor32<8>(x);
  if constexpr (M >= 16) x += xor32<16>(x);
  return x;
}

// SD: dtype of the states (KDA_DTYPE_NONE when neither is given).  A lane
// moves 16 bytes of state per load: CPL = 4 fp32 or 8 bf16 channels, so a
// row spans LPR = 128 / CPL lanes and one wave load covers RPI = 64 / LPR rows.
template <int SD>
__global__ __launch_bounds__(kThreads) void decode_kernel(DecodeArgs a) {
  constexpr int CPL = SD == KDA_DTYPE_FP32 ? 4 : 8;
  constexpr int LPR = K / CPL;        // lanes per row: 32 or 16
  constexpr int RPI = 64 / LPR;       // rows per wave load: 2 or 4
  constexpr int RPL = 32 / RPI;       // rows per lane: 16 or 8
  __shared__ __align__(16) float e_sh[4][RPI][RPL];
  const int64_t pair = blockIdx.x;   // n * H + h
  const int64_t H = a.H;
  const int h = (int)(pair % H);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lr = lane / LPR, kq = lane % LPR;
  const int c0 = CPL * kq;   // this lane's channels c0 .. c0 + CPL - 1

  // ---- the token: q, k, g on this lane's channels, beta
  const int64_t tk = pair * K + c0;
  float q4[CPL], k4[CPL], g4[CPL];
#pragma unroll
  for (int w = 0; w < CPL / 4; ++w) {
    const u32x2 qw = *reinterpret_cast<const u32x2*>(a.q + tk + 4 * w);
    const u32x2 kw = *reinterpret_cast<const u32x2*>(a.k + tk + 4 * w);
    const u32x2 gw = *reinterpret_cast<const u32x2*>(a.g + tk + 4 * w);
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      q4[4 * w + 2 * e] = bf16_lo(qw[e]); q4[4 * w + 2 * e + 1] = bf16_hi(qw[e]);
      k4[4 * w + 2 * e] = bf16_lo(kw[e]); k4[4 * w + 2 * e + 1] = bf16_hi(kw[e]);
      g4[4 * w + 2 * e] = bf16_lo(gw[e]); g4[4 * w + 2 * e + 1] = bf16_hi(gw[e]);
    }
  }
  float sq = 0.f, sk = 0.f;
#pragma unroll
  for (int e = 0; e < CPL; ++e) {
    sq = fmaf(q4[e], q4[e], sq);
    sk = fmaf(k4[e], k4[e], sk);
  }
  sq = lanes_sum<LPR / 2>(sq);
  sk = lanes_sum<LPR / 2>(sk);
  const float rq = a.scale / sqrtf(sq + kEps), rk = 1.f / sqrtf(sk + kEps);
  const float beta = 1.f / (1.f + expf(-bf16_to_f32(a.beta[pair])));
  const float A2 = -expf(a.A_log[h]) * kLog2e, lb2 = a.lower_bound * kLog2e;
  float kn[CPL], qn[CPL], dec[CPL];
#pragma unroll
  for (int e = 0; e < CPL; ++e) {
    kn[e] = k4[e] * rk;
    qn[e] = q4[e] * rq;
    const float sg = fast_rcp(1.f + fast_exp2(A2 * (g4[e] + a.dt_bias[(int64_t)h * K + c0 + e])));   // sigmoid
    dec[e] = fast_exp2(lb2 * sg);                                                                      // exp(a)
  }

  // ---- state rows 32 wave + RPI i + lr, channels c0 .. c0 + CPL - 1
  const int64_t sbase = (pair * V + 32 * wave + lr) * K + c0;
  float S[RPL][CPL];
#pragma unroll
  for (int i = 0; i < RPL; ++i) {
    const int64_t idx = sbase + (int64_t)(RPI * i) * K;
    if (SD == KDA_DTYPE_NONE || a.s_in == nullptr) {
#pragma unroll
      for (int e = 0; e < CPL; ++e) S[i][e] = 0.f;
    } else if constexpr (SD == KDA_DTYPE_FP32) {
      const f32x4 w = *reinterpret_cast<const f32x4*>(static_cast<const float*>(a.s_in) + idx);
      S[i][0] = w[0]; S[i][1] = w[1]; S[i][2] = w[2]; S[i][3] = w[3];
    } else {
      const u32x4 w = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.s_in) + idx);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        S[i][2 * e] = bf16_lo(w[e]);
        S[i][2 * e + 1] = bf16_hi(w[e]);
      }
    }
  }

  // ---- decay, u = S^T kn, e = beta (v - u)
  float part[RPL];
#pragma unroll
  for (int i = 0; i < RPL; ++i) {
    float p = 0.f;
#pragma unroll
    for (int e = 0; e < CPL; ++e) {
      S[i][e] *= dec[e];
      p = fmaf(S[i][e], kn[e], p);
    }
    part[i] = p;
  }
  const float u = row_sums<RPL>(part, kq);
  const int my_row = 32 * wave + RPI * (kq >> 1) + lr;   // the row whose sums this lane holds
  const float vin = bf16_to_f32(a.v[pair * V + my_row]);
  if ((kq & 1) == 0) e_sh[wave][lr][kq >> 1] = beta * (vin - u);
  // A wave's LDS operations complete in order, so its reads below see its
  // writes above; the wave barrier keeps the compiler from reordering them.
  __builtin_amdgcn_wave_barrier();
  float ev[RPL];
#pragma unroll
  for (int i = 0; i < RPL; i += 4) {
    const f32x4 w = *reinterpret_cast<const f32x4*>(&e_sh[wave][lr][i]);
    ev[i] = w[0]; ev[i + 1] = w[1]; ev[i + 2] = w[2]; ev[i + 3] = w[3];
  }

  // ---- S += kn e^T, o = S^T qn
#pragma unroll
  for (int i = 0; i < RPL; ++i) {
    float p = 0.f;
#pragma unroll
    for (int e = 0; e < CPL; ++e) {
      S[i][e] = fmaf(kn[e], ev[i], S[i][e]);
      p = fmaf(S[i][e], qn[e], p);
    }
    part[i] = p;
  }
  const float o = row_sums<RPL>(part, kq);
  if ((kq & 1) == 0) a.out[pair * V + my_row] = f32_to_bf16(o);

  // ---- state out
  if (SD != KDA_DTYPE_NONE && a.s_out != nullptr) {
#pragma unroll
    for (int i = 0; i < RPL; ++i) {
      const int64_t idx = sbase + (int64_t)(RPI * i) * K;
      if constexpr (SD == KDA_DTYPE_FP32) {
        *reinterpret_cast<f32x4*>(static_cast<float*>(a.s_out) + idx) = f32x4{S[i][0], S[i][1], S[i][2], S[i][3]};
      } else {
        u32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = pack_bf16(S[i][2 * e], S[i][2 * e + 1]);
        *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(a.s_out) + idx) = w;
      }
    }
  }
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, hipStream_t s) {
  const int64_t pairs = a.N * a.H;
  if (pairs == 0) return hipSuccess;
  const dim3 grid((unsigned)pairs), block(kThreads);
  if (a.state_dtype == KDA_DTYPE_FP32)
    hipLaunchKernelGGL(decode_kernel<KDA_DTYPE_FP32>, grid, block, 0, s, a);
  else if (a.state_dtype == KDA_DTYPE_BF16)
    hipLaunchKernelGGL(decode_kernel<KDA_DTYPE_BF16>, grid, block, 0, s, a);
  else
    hipLaunchKernelGGL(decode_kernel<KDA_DTYPE_NONE>, grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace kda
