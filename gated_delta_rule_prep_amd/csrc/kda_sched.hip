// kda_sched.hip -- cu_seqlens work scheduler (one workgroup, integer work only).
//
// Turns the sequence boundaries into
//   * a chunk table: chunk i -> {sequence n, first flattened token row, length},
//     chunks of at most lay.chunk (16, 32 or 64) tokens that restart at every sequence start (so a
//     chunk never straddles two sequences; the pages batch variable-length
//     sequences through cu_seqlens: README mirror "内核 API", cu_seqlens row);
//   * a per-sequence table {first chunk, chunk count, first token row, length};
//   * a work order of the sequences, longest first, so that the chunk
//     recurrence starts its longest serial chains first;
//   * the first chunk of each part (parts cut the token rows into consecutive
//     ranges of part_rows rows, so that prep and recurrence can overlap);
//   * a status word: KDA_STATUS_BAD_CU_SEQLENS when cu_seqlens[0] != 0, the
//     boundaries decrease, or cu_seqlens[N] != T.  Then every sequence gets zero
//     chunks, so no later kernel touches a token;
//   * the execution path, when the caller leaves it to the library: both
//     paths' kernels are enqueued and the ones not chosen exit at once.  The
//     choice compares estimates of the two paths built from the total and the
//     longest chunk count (see choose_path).
// Without cu_seqlens sequence n is batch row n: rows [n*T, (n+1)*T).
#include "kda_internal.h"
#include "../../include/kda.h"

namespace kda {
namespace {

constexpr int kThreads = 1024;
constexpr int kRankSortMax = 2048;   // longest-first order by rank sort up to this N

__global__ __launch_bounds__(kThreads) void sched_kernel(SchedArgs a) {
  WsHeader* hdr = reinterpret_cast<WsHeader*>(a.ws);
  ChunkEntry* chunks = reinterpret_cast<ChunkEntry*>(a.ws + a.lay.chunk_table);
  SeqEntry* seqs = reinterpret_cast<SeqEntry*>(a.ws + a.lay.seq_table);
  int32_t* order = reinterpret_cast<int32_t*>(a.ws + a.lay.order);
  const int tid = threadIdx.x;
  const int64_t N = a.N;
  const int64_t C = a.lay.chunk;

  __shared__ int s_bad;
  __shared__ int32_t s_scan[kThreads];
  __shared__ int32_t s_carry;
  __shared__ int32_t s_nch[kRankSortMax];
  __shared__ int32_t s_maxc;
  if (tid == 0) {
    s_bad = 0;
    s_carry = 0;
    s_maxc = 0;
  }
  __syncthreads();

  // 1. validate the boundaries
  if (a.cu) {
    if (tid == 0 && (a.cu[0] != 0 || a.cu[N] != a.T)) s_bad = 1;
    for (int64_t n = tid; n < N; n += kThreads)
      if (a.cu[n + 1] < a.cu[n]) s_bad = 1;
  }
  __syncthreads();
  const bool bad = s_bad != 0;

  // 2. chunk counts and their exclusive prefix sum, one tile of kThreads at a time
  for (int64_t base = 0; base < N; base += kThreads) {
    const int64_t n = base + tid;
    int32_t nch = 0;
    if (n < N && !bad) {
      const int64_t len = a.cu ? a.cu[n + 1] - a.cu[n] : a.T;
      nch = (int32_t)((len + C - 1) / C);
    }
    s_scan[tid] = nch;
    if (nch > 0) atomicMax(&s_maxc, nch);
    __syncthreads();
    for (int off = 1; off < kThreads; off <<= 1) {  // Hillis-Steele inclusive scan
      const int32_t x = tid >= off ? s_scan[tid - off] : 0;
      __syncthreads();
      s_scan[tid] += x;
      __syncthreads();
    }
    if (n < N) {
      seqs[n].first_chunk = s_carry + s_scan[tid] - nch;
      seqs[n].nchunks = nch;
      seqs[n].row0 = (bad || !a.cu) ? (int32_t)(n * a.T) : (int32_t)a.cu[n];
      seqs[n].len = bad ? 0 : (int32_t)(a.cu ? a.cu[n + 1] - a.cu[n] : a.T);
    }
    __syncthreads();
    if (tid == kThreads - 1) s_carry += s_scan[tid];
    __syncthreads();
  }
  const int32_t total = s_carry;

  // 3. chunk table (the fused path, whose layout has no chunk table, skips
  // this step and the next).  Up to kThreads sequences (one scan tile, whose
  // inclusive prefix sums are still in LDS) each thread takes chunks i = tid,
  // tid + kThreads, ... and finds its sequence by binary search for the first
  // prefix sum above i, so that neither one long sequence nor many short ones
  // serialise the fill; beyond that each thread fills the chunks of its own
  // sequences.
  const bool table = a.lay.max_chunks > 0;
  if (!table) {
  } else if (N <= kThreads) {
    for (int32_t i = tid; i < total; i += kThreads) {
      int32_t lo = 0, hi = (int32_t)N - 1;
      while (lo < hi) {
        const int32_t mid = (lo + hi) >> 1;
        if (s_scan[mid] > i) hi = mid;
        else lo = mid + 1;
      }
      const int64_t n = lo;
      const int32_t c = i - (n > 0 ? s_scan[n - 1] : 0);
      const int64_t row0 = a.cu ? a.cu[n] : n * a.T;
      const int64_t len = a.cu ? a.cu[n + 1] - a.cu[n] : a.T;
      const int64_t rem = len - (int64_t)c * C;
      chunks[i] = ChunkEntry{(int32_t)n, (int32_t)(row0 + (int64_t)c * C), (int32_t)(rem < C ? rem : C)};
    }
  } else {
    for (int64_t n = tid; n < N; n += kThreads) {
      const int64_t row0 = a.cu ? a.cu[n] : n * a.T;
      const int64_t len = a.cu ? a.cu[n + 1] - a.cu[n] : a.T;
      const int32_t first = seqs[n].first_chunk, nch = seqs[n].nchunks;
      for (int32_t c = 0; c < nch; ++c) {
        const int64_t rem = len - (int64_t)c * C;
        chunks[first + c] = ChunkEntry{(int32_t)n, (int32_t)(row0 + (int64_t)c * C), (int32_t)(rem < C ? rem : C)};
      }
    }
  }
  __syncthreads();

  // 4. parts: part_first[p] = index of the first chunk whose first token row is
  // at or past p * part_rows (the chunk table is in token order)
  auto part_of = [&](int32_t row0) { return (int)min((int64_t)row0 / a.part_rows, (int64_t)a.parts - 1); };
  for (int32_t i = tid; table && i < total; i += kThreads) {
    const int pi = part_of(chunks[i].row0);
    const int pprev = i > 0 ? part_of(chunks[i - 1].row0) : -1;
    for (int p = pprev + 1; p <= pi; ++p) hdr->part_first[p] = i;
  }
  if (tid == 0 && table) {
    const int plast = total > 0 ? part_of(chunks[total - 1].row0) : -1;
    for (int p = plast + 1; p <= a.parts; ++p) hdr->part_first[p] = total;
  }

  // 5. work order, longest first (ties by index); identity beyond kRankSortMax
  const bool sort = N <= kRankSortMax;
  if (sort)
    for (int64_t n = tid; n < N; n += kThreads) s_nch[n] = seqs[n].nchunks;
  __syncthreads();
  for (int64_t n = tid; n < N; n += kThreads) {
    int64_t rank = n;
    if (sort) {
      const int32_t mine = s_nch[n];
      rank = 0;
      for (int m = 0; m < (int)N; ++m) {
        const int32_t o = s_nch[m];
        rank += (o > mine) || (o == mine && m < n);
      }
    }
    order[rank] = (int32_t)n;
  }
  if (tid == 0) {
    hdr->status = bad ? KDA_STATUS_BAD_CU_SEQLENS : KDA_STATUS_OK;
    hdr->chunk_count = total;
    hdr->path = a.path == KDA_PATH_AUTO ? choose_path(a.H, N, total, s_maxc, a.cu == nullptr, a.cus) : a.path;
  }
}

}  // namespace

hipError_t launch_sched(const SchedArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(sched_kernel, dim3(1), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace kda
