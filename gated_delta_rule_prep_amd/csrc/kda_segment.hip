// kda_segment.hip -- kernels of the segmented forward (kda_fwd_segmented):
// one long sequence is cut into segments whose chunk chains run in parallel
// and are joined by the affine map each segment applies to its state.
//
// Over a segment the recurrence of the FlashKDA blog post ("FlashKDA：月之暗面开源的
// Kimi Delta Attention 高性能内核", §一: decay, then the beta-weighted delta
// correction) maps its starting state affinely:
//   S_end = A S_start + B,  A = prod_t (I - beta_t kn_t kn_t^T) diag(exp(a_t)),
// with B the end state from a zero start.  Both are end states of ordinary
// runs of the segment: B with the real values and a zero start, A with zero
// values and the identity as start (both by the recurrence kernel, in one
// launch over one set of chunk records).  The segments' start states then follow
// by the prefix S_start(0) = the sequence's initial state,
// S_start(j + 1) = A_j S_start(j) + B_j, and a last run from those starts
// writes the outputs.  In the stored layout [v][k] (stored[v][k] = S[k][v]),
// the step is St_next[v][k] = sum_m St[v][m] A[k][m] + B_st[v][k]; A comes in
// its math layout A[k][m], so that the contraction index m is contiguous.
//
// A is a product of factors of spectral norm at most 1 (0 <= beta <= 1 and
// |kn| = 1 make I - beta kn kn^T a contraction, and the decay is at most 1),
// so its entries lie in [-1, 1] and it is kept in fp16; the composition runs
// on fp16 MFMA operands with fp32 accumulation and fp32 states, the rounding
// the recurrence itself applies to its state operands every chunk.
#include "kda_device.h"
#include "kda_internal.h"
#include "../../include/kda.h"

namespace kda {
namespace {

// seg_cu[n S + j] = the first row of segment j of sequence n; segments are
// ceil(len / S) tokens rounded up to whole 16-token chunks (the last ones may
// be shorter or empty); seg_cu[N S] = the total row count.
__global__ __launch_bounds__(256) void seg_cu_kernel(SegArgs a) {
  const int64_t n = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (n >= a.N) return;
  const int64_t start = a.cu ? a.cu[n] : n * a.T;
  const int64_t end = a.cu ? a.cu[n + 1] : (n + 1) * a.T;
  const int64_t len = end > start ? end - start : 0;
  const int64_t per = ((len + a.S - 1) / a.S + C - 1) / C * C;
  for (int j = 0; j < a.S; ++j) a.seg_cu[n * a.S + j] = min(start + j * per, max(end, start));
  if (n == a.N - 1) a.seg_cu[a.N * a.S] = a.cu ? a.cu[a.N] : a.N * a.T;
}

// The prefix over the segments of one (sequence, head), 16 state rows (v) per
// workgroup of eight waves; wave w computes output columns k = 16 w .. + 15.
// The contraction over m runs as four fp16 16x16x32 MFMAs, MFMA c taking
// m = 32 c + 8 g + e in element e of lane group g: lane (r, g) holds
// St[v0 + r][32 c + 8 g .. + 7] (the A operand, the same in every wave) and
// A[16 w + r][32 c + 8 g .. + 7] (the B operand, 16 bytes; the four lanes of a
// row read 64 contiguous bytes).  The accumulator holds
// St_next[v0 + 4 g + i][16 w + r].  The new rows go back to the operand layout
// through LDS, and from there, coalesced, to the next segment's start (or the
// final state).
// XCD-aware placement: id b runs on XCD b % 8; the eight row blocks of pair
// 8 q + x get ids 8 (8 q + rb) + x, so they share one L2.
constexpr int kPrefixWaves = 8;

__device__ __forceinline__ void load_ab(const uint16_t* Ah, const float* Bm, int v0, int w, int r, int g,
                                        f16x8* a, float* b) {
  const uint16_t* const arow = Ah + (16 * w + r) * K + 8 * g;
#pragma unroll
  for (int c = 0; c < 4; ++c) a[c] = __builtin_bit_cast(f16x8, *reinterpret_cast<const u32x4*>(arow + 32 * c));
#pragma unroll
  for (int i = 0; i < 4; ++i) b[i] = Bm[(v0 + 4 * g + i) * K + 16 * w + r];
}

__device__ __forceinline__ void operand_rows(const float (*tile)[K + 4], int r, int g, f16x8* st) {
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int e = 0; e < 8; ++e) st[c][e] = (_Float16)tile[r][32 * c + 8 * g + e];
}

__device__ __forceinline__ void put_rows(const float (*tile)[K + 4], int tid, void* dst, int dtype) {
  // thread tid writes row tid / 32, columns 4 (tid % 32) .. + 3 of the 16 x 128 block at dst
  const int row = tid >> 5, c4 = (tid & 31) * 4;
  const f32x4 x = *reinterpret_cast<const f32x4*>(&tile[row][c4]);
  if (dtype == KDA_DTYPE_FP32) {
    *reinterpret_cast<f32x4*>(static_cast<float*>(dst) + row * K + c4) = x;
  } else {
    u32x2 wv;
    wv[0] = pack_bf16(x[0], x[1]);
    wv[1] = pack_bf16(x[2], x[3]);
    *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(dst) + row * K + c4) = wv;
  }
}

__global__ __launch_bounds__(64 * kPrefixWaves) void prefix_kernel(PrefixArgs a) {
  __shared__ __align__(16) float tile[16][K + 4];
  const int64_t bid = blockIdx.x, x = bid & 7, q = bid >> 3;
  const int64_t nh = 8 * (q / 8) + x;
  const int v0 = 16 * (int)(q % 8);
  if (nh >= a.N * a.H) return;
  if (a.hdr->status & KDA_STATUS_BAD_CU_SEQLENS) return;   // bad cu_seqlens: leave the states alone
  const int64_t n = nh / a.H, h = nh - n * a.H;
  const int tid = threadIdx.x, lane = tid & 63, r = lane & 15, g = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t mat = (int64_t)V * K;
  const auto seg_base = [&](int j) { return ((n * a.S + j) * a.H + h) * mat; };   // [segment][head] matrix

  // the first segment's start: the sequence's initial state (or zero)
  {
    const int row = tid >> 5, c4 = (tid & 31) * 4;
    const int64_t idx = ((n * a.H + h) * V + v0 + row) * K + c4;
    f32x4 s0 = f32x4{0.f, 0.f, 0.f, 0.f};
    if (a.s_in != nullptr) {
      if (a.state_dtype == KDA_DTYPE_FP32) {
        s0 = *reinterpret_cast<const f32x4*>(static_cast<const float*>(a.s_in) + idx);
      } else {
        const u32x2 wv = *reinterpret_cast<const u32x2*>(static_cast<const uint16_t*>(a.s_in) + idx);
        s0 = f32x4{bf16_lo(wv[0]), bf16_hi(wv[0]), bf16_lo(wv[1]), bf16_hi(wv[1])};
      }
    }
    *reinterpret_cast<f32x4*>(&tile[row][c4]) = s0;
  }
  __syncthreads();
  f16x8 st[4];
  operand_rows(tile, r, g, st);
  put_rows(tile, tid, a.starts + seg_base(0) + (int64_t)v0 * K, KDA_DTYPE_FP32);
  // Two register sets of A_st / B_st, each refilled right after the segment
  // it holds is composed, so a segment's loads have the whole composition of
  // the segment before to land.  Loads past the last segment repeat it.
  f16x8 a0[4], a1[4];
  float b0[4], b1[4];
  const auto seg_ld = [&](int j, f16x8* aa, float* bb) {
    const int js = j < a.S ? j : a.S - 1;
    load_ab(a.A + seg_base(js), a.B + seg_base(js), v0, w, r, g, aa, bb);
  };
  const auto compose = [&](int j, const f16x8* aa, const float* bb) {
    // An empty segment (A = I, B = 0) leaves the state as it is, exactly;
    // the tile holds it in fp32 either way.
    const int64_t sj = (n * a.S + j);
    if (a.seg_cu[sj + 1] != a.seg_cu[sj]) {
      f32x4 acc = f32x4{bb[0], bb[1], bb[2], bb[3]};
#pragma unroll
      for (int c = 0; c < 4; ++c) acc = mfma_f16_k32(st[c], aa[c], acc);
      __syncthreads();   // every wave has read the tile of the step before
#pragma unroll
      for (int i = 0; i < 4; ++i) tile[4 * g + i][16 * w + r] = acc[i];
      __syncthreads();
      operand_rows(tile, r, g, st);
    }
    if (j + 1 < a.S) {
      put_rows(tile, tid, a.starts + seg_base(j + 1) + (int64_t)v0 * K, KDA_DTYPE_FP32);
    } else if (a.s_out != nullptr) {   // the sequence's final state
      put_rows(tile, tid, static_cast<char*>(a.s_out) +
                              ((n * a.H + h) * V + v0) * K * (a.state_dtype == KDA_DTYPE_FP32 ? 4 : 2),
               a.state_dtype);
    }
  };
  seg_ld(0, a0, b0);
  seg_ld(1, a1, b1);
  for (int j = 0; j < a.S; j += 2) {
    compose(j, a0, b0);
    seg_ld(j + 2, a0, b0);
    if (j + 1 < a.S) compose(j + 1, a1, b1);
    seg_ld(j + 3, a1, b1);
  }
}

}  // namespace

hipError_t launch_seg_cu(const SegArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(seg_cu_kernel, dim3((unsigned)((a.N + 255) / 256)), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_prefix(const PrefixArgs& a, hipStream_t s) {
  const int64_t pairs = a.N * a.H;
  if (pairs == 0) return hipSuccess;
  const int64_t grid = 64 * ((pairs + 7) / 8);   // eight 16-row blocks per pair
  if (grid > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL(prefix_kernel, dim3((unsigned)grid), dim3(64 * kPrefixWaves), 0, s, a);
  return hipGetLastError();
}

}  // namespace kda
