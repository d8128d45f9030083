// kda_api.cpp -- the C ABI declared in include/kda.h: host-side validation,
// workspace layout and the three kernel launches.
//
// Argument rules follow the kernel API notes of the FlashKDA README mirror
// (section "内核 API"): K = V = 128; states may be absent, bf16 or fp32 and must
// share a dtype when both are given; with cu_seqlens B must be 1 and states are
// [N, H, V, K]; without it each batch row is a sequence.  lower_bound lies in
// [-5, 0] (the same table).  Every check runs on the host before any HIP call.
#include <cmath>
#include <cstddef>
#include <cstdarg>
#include <cstdio>
#include <algorithm>
#include <atomic>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <string>

#include "../../include/kda.h"
#include "kda_internal.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int64_t align_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

// The kernels move q, k, g, v, out and the states in 16-byte vectors.
bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) != 0; }

// Device capability cache: -1 unknown, 0 unsupported, 1 gfx950.
constexpr int kMaxDevices = 64;
int g_dev_ok[kMaxDevices];
int g_dev_cus[kMaxDevices];   // compute units, 0 until read
std::once_flag g_dev_once;

int check_device(int* dev_out = nullptr) {
  std::call_once(g_dev_once, [] {
    for (int i = 0; i < kMaxDevices; ++i) g_dev_ok[i] = -1;
  });
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(KDA_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(KDA_EUNSUPPORTED, "device index %d out of range", dev);
  int ok = __atomic_load_n(&g_dev_ok[dev], __ATOMIC_ACQUIRE);
  if (ok < 0) {
    hipDeviceProp_t p;
    e = hipGetDeviceProperties(&p, dev);
    if (e != hipSuccess) return fail(KDA_EHIP, "hipGetDeviceProperties: %s", hipGetErrorString(e));
    ok = std::strncmp(p.gcnArchName, "gfx950", 6) == 0 ? 1 : 0;
    __atomic_store_n(&g_dev_ok[dev], ok, __ATOMIC_RELEASE);
  }
  if (!ok) return fail(KDA_EUNSUPPORTED, "kda: device %d is not gfx950 (MI355X)", dev);
  if (dev_out) *dev_out = dev;
  return KDA_OK;
}

// Per-device side stream and events for the overlapped path: the recurrence
// of part p runs on the side stream while the main stream computes the chunk
// records of part p + 1.  Created on first use, kept until the process ends;
// the mutex also keeps concurrent callers on one device from interleaving
// their use of the shared stream and events.
struct SideRes {
  std::mutex mu;
  bool ready = false;
  hipStream_t side = nullptr;
  hipEvent_t prep_done[kda::kMaxParts];
  hipEvent_t join;
};
SideRes g_side[kMaxDevices];

int side_resources(int dev, SideRes** out) {
  SideRes& r = g_side[dev];
  if (!r.ready) {
    hipError_t e = hipStreamCreateWithFlags(&r.side, hipStreamNonBlocking);
    for (int i = 0; e == hipSuccess && i < kda::kMaxParts; ++i)
      e = hipEventCreateWithFlags(&r.prep_done[i], hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&r.join, hipEventDisableTiming);
    if (e != hipSuccess) return fail(KDA_EHIP, "kda: side stream or event creation: %s", hipGetErrorString(e));
    r.ready = true;
  }
  *out = &r;
  return KDA_OK;
}

// Size checks shared by kda_fwd and the layout query.  N is the sequence count.
int check_sizes(int64_t B, int64_t T, int64_t H, int64_t K, int64_t V, const int64_t* cu,
                int64_t num_seqs, int has_cu, int64_t* N_out) {
  if (B < 1 || T < 0 || H < 1)
    return fail(KDA_EINVAL, "kda: need B >= 1, T >= 0, H >= 1 (got B=%lld T=%lld H=%lld)",
                (long long)B, (long long)T, (long long)H);
  if (K != kda::K || V != kda::V)
    return fail(KDA_EINVAL, "kda: K and V must both be 128 (got K=%lld V=%lld)", (long long)K, (long long)V);
  if (H > 65535) return fail(KDA_EINVAL, "kda: H=%lld exceeds 65535", (long long)H);
  const bool with_cu = cu != nullptr || has_cu;
  if (with_cu && B != 1) return fail(KDA_EINVAL, "kda: B must be 1 with cu_seqlens (got B=%lld)", (long long)B);
  if (with_cu && num_seqs < 1)
    return fail(KDA_EINVAL, "kda: num_seqs must be >= 1 with cu_seqlens (got %lld)", (long long)num_seqs);
  const int64_t N = with_cu ? num_seqs : B;
  // int32 token rows and chunk indices inside the kernels
  if (B * T >= (int64_t(1) << 31) || N >= (int64_t(1) << 30))
    return fail(KDA_EINVAL, "kda: B*T=%lld or N=%lld too large", (long long)(B * T), (long long)N);
  if (N * H >= (int64_t(1) << 31)) return fail(KDA_EINVAL, "kda: N*H too large");
  *N_out = N;
  return KDA_OK;
}

}  // namespace

namespace kda {

namespace {
std::atomic<int> g_spin_limit{kSpinLimit};
}

int device_cus() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return kCUs;
  int c = __atomic_load_n(&g_dev_cus[dev], __ATOMIC_ACQUIRE);
  if (c <= 0) {
    if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c <= 0) return kCUs;
    __atomic_store_n(&g_dev_cus[dev], c, __ATOMIC_RELEASE);
  }
  return c;
}

int spin_limit() { return g_spin_limit.load(std::memory_order_relaxed); }

bool layout_for(int64_t B, int64_t T, int64_t H, int64_t N, int chunk, Layout* L) {
  if (B < 1 || T < 0 || H < 1 || N < 0 || (chunk != C && chunk != C32 && chunk != C64)) return false;
  const int64_t rec_bytes = chunk == C ? REC_BYTES : chunk == C32 ? REC32_BYTES : REC64_BYTES;
  const int64_t max_chunks = (B * T) / chunk + N;   // sum_n ceil(len_n / chunk) <= B*T/chunk + N
  int64_t off = sizeof(WsHeader);
  L->chunk_table = off;
  off = align_up(off + max_chunks * (int64_t)sizeof(ChunkEntry), 256);
  L->seq_table = off;
  off = align_up(off + N * (int64_t)sizeof(SeqEntry), 256);
  L->order = off;
  off = align_up(off + N * 4, 256);
  L->chunk = chunk;
  L->records = off;
  L->rec_bytes = rec_bytes;
  L->max_chunks = max_chunks;
  off = align_up(off + H * max_chunks * rec_bytes, 256);
  L->state = off;
  off += N * H * V * K * (int64_t)sizeof(float);
  L->total = align_up(off, 256);
  return true;
}

// The fused path keeps only the header and the per-sequence tables: no chunk
// table, no records, no hand-over states.
bool layout_fused(int64_t B, int64_t T, int64_t H, int64_t N, Layout* L) {
  if (B < 1 || T < 0 || H < 1 || N < 0) return false;
  int64_t off = sizeof(WsHeader);
  L->chunk_table = off;
  L->seq_table = off;
  off = align_up(off + N * (int64_t)sizeof(SeqEntry), 256);
  L->order = off;
  off = align_up(off + N * 4, 256);
  L->chunk = C;
  L->records = off;
  L->rec_bytes = 0;
  L->max_chunks = 0;
  L->state = off;
  L->total = off;
  return true;
}

// Parts used when the caller leaves the choice to the library: one.  On
// MI355X the two kernels slow each other down by about as much as running
// them side by side saves (measured at T = 8192, H = 64 / 96, fixed and
// varlen: 2 to 8 parts change the step time by -2 % to +50 %), so overlap is
// left to callers that measure a gain at their own shapes.
int parts_for(int64_t) { return 1; }

// Chunk size used when the caller leaves the choice to the library.
int default_chunk() { return C; }

}  // namespace kda

namespace {

// Path a kda_fwd_ex call takes: KDA_PATH_SPLIT, KDA_PATH_FUSED, KDA_PATH_AUTO
// (both paths enqueued, the scheduler kernel picks one from the sequence
// lengths), or -1.  Measured on MI355X (T = 8192, K = V = 128, ms per call):
// the fused kernel is faster for batches of many short sequences (8 x 1024
// tokens, H = 96: 0.424 against 0.526) but slower whenever one sequence is
// long (one 8192-token sequence: 0.84 against 0.56; 12 ragged sequences with
// one of 7359 tokens: 0.91 against 0.60), and with cu_seqlens the lengths are
// only known on the device.  The library chooses only where both paths can run
// (16-token chunks, one part).
int resolve_path(int chunk, int parts, int path) {
  if (chunk != 0 && chunk != kda::C && chunk != kda::C32 && chunk != kda::C64) return -1;
  if (parts < 0) return -1;
  const bool fusable = (chunk == 0 || chunk == kda::C) && parts <= 1;
  if (path == KDA_PATH_AUTO) return fusable ? KDA_PATH_AUTO : KDA_PATH_SPLIT;
  if (path == KDA_PATH_SPLIT) return KDA_PATH_SPLIT;
  if (path == KDA_PATH_FUSED) return fusable ? KDA_PATH_FUSED : -1;
  return -1;
}

}  // namespace

extern "C" {

int kda_version(void) { return 300; }  // 0.3.0: 64-token chunks, the Neumann precision variant

const char* kda_get_last_error(void) { return g_last_error.c_str(); }

// ---- segmented forward -----------------------------------------------------

namespace {

// Workspace regions of kda_fwd_segmented (byte offsets), or false on bad sizes.
// The plain forward's workspace comes first, so its header (status, path
// taken) sits at the start as for kda_fwd.
struct SegLayout {
  int64_t inner, inner_bytes, seg_cu, A, B, starts, total;
};

bool seg_layout(int64_t B, int64_t T, int64_t H, int64_t N, int S, SegLayout* L) {
  const int64_t NS = N * S, mat = NS * H * kda::V * kda::K * (int64_t)sizeof(float);   // fp32 states
  kda::Layout inner;
  if (!kda::layout_for(1, B * T, H, NS, kda::C, &inner)) return false;
  int64_t off = 0;
  L->inner = off;
  L->inner_bytes = inner.total;
  off = align_up(off + inner.total, 256);
  L->seg_cu = off;
  off = align_up(off + (NS + 1) * 8, 256);
  L->A = off;   // the transitions, fp16
  off = align_up(off + mat / 2, 256);
  L->B = off;
  off = align_up(off + mat, 256);
  L->starts = off;
  off = align_up(off + mat, 256);
  L->total = off;
  return true;
}

// The library's segment count.  Cutting pays while the recurrence leaves
// CUs idle: one workgroup per 64 value columns of a (segment, head) chain, and
// the two-set launch doubles that.  Measured on MI355X (one sequence, H = 2 ..
// 96, T = 8192 .. 65536), the best count is the largest power of two with at
// most 128 (segment, head) chains and segments of at least 512 tokens; below
// four segments the three recurrence passes cost more than they save.  With
// cu_seqlens the mean length stands in for the lengths, which only the device
// knows.  (128 chains on the 256 CUs of a whole MI355X: half the CU count.)
int choose_segments(int64_t B, int64_t T, int64_t H, int64_t N, bool has_cu) {
  const int64_t len = has_cu ? (B * T) / (N > 0 ? N : 1) : T;
  const int64_t max_chains = kda::device_cus() / 2;
  int64_t S = 1;
  while (2 * S * N * H <= max_chains && len / (2 * S) >= 512 && 2 * S <= 4096) S *= 2;
  return S >= 4 ? (int)S : 1;
}

}  // namespace

size_t kda_fwd_workspace_bytes(int64_t B, int64_t T, int64_t H, int64_t num_seqs, int has_cu_seqlens) {
  int64_t N = 0;
  if (check_sizes(B, T, H, kda::K, kda::V, nullptr, num_seqs, has_cu_seqlens, &N) != KDA_OK) return 0;
  kda::Layout L16, L32;   // enough for either chunk size
  if (!kda::layout_for(B, T, H, N, kda::C, &L16) || !kda::layout_for(B, T, H, N, kda::C32, &L32)) return 0;
  int64_t bytes = std::max(L16.total, L32.total);
  // and for the segmented form that kda_fwd takes for B sequences of T tokens
  // when the library's segment count is above 1
  const int S = has_cu_seqlens ? 1 : choose_segments(B, T, H, N, false);
  SegLayout SL;
  if (S > 1 && seg_layout(B, T, H, N, S, &SL)) bytes = std::max(bytes, SL.total);
  return (size_t)bytes;
}

size_t kda_fwd_workspace_bytes_ex(int64_t B, int64_t T, int64_t H, int64_t num_seqs, int has_cu_seqlens,
                                  int chunk, int parts, int path) {
  int64_t N = 0;
  const int p = resolve_path(chunk, parts, path);
  if (p < 0) return 0;
  if (check_sizes(B, T, H, kda::K, kda::V, nullptr, num_seqs, has_cu_seqlens, &N) != KDA_OK) return 0;
  kda::Layout L;
  const bool ok = p == KDA_PATH_FUSED ? kda::layout_fused(B, T, H, N, &L)   // the split path's otherwise
                                      : kda::layout_for(B, T, H, N, chunk == 0 ? kda::default_chunk() : chunk, &L);
  return ok ? (size_t)L.total : 0;
}

int kda_fwd_path(int chunk, int parts, int path) { return resolve_path(chunk, parts, path); }

int kda_workspace_layout(int64_t B, int64_t T, int64_t H, int64_t num_seqs, int has_cu_seqlens, int chunk,
                         int64_t offsets[7]) {
  int64_t N = 0;
  if (offsets == nullptr) return fail(KDA_EINVAL, "kda: offsets is NULL");
  if (chunk != kda::C && chunk != kda::C32 && chunk != kda::C64)
    return fail(KDA_EINVAL, "kda: chunk must be 16, 32 or 64 (got %d)", chunk);
  int rc = check_sizes(B, T, H, kda::K, kda::V, nullptr, num_seqs, has_cu_seqlens, &N);
  if (rc != KDA_OK) return rc;
  kda::Layout L;
  if (!kda::layout_for(B, T, H, N, chunk, &L)) return fail(KDA_EINVAL, "kda: bad sizes");
  offsets[0] = L.chunk_table;
  offsets[1] = L.seq_table;
  offsets[2] = L.order;
  offsets[3] = L.records;
  offsets[4] = L.rec_bytes;
  offsets[5] = L.max_chunks;
  offsets[6] = L.total;
  return KDA_OK;
}

static int validate_common(const void* q, const void* k, const void* g, const void* beta, float scale,
                           const float* A_log, const float* dt_bias, float lower_bound,
                           const int64_t* cu, int64_t num_seqs, int64_t B, int64_t T, int64_t H,
                           int64_t K, int64_t V, void* workspace, size_t workspace_bytes, int chunk,
                           bool fused, kda::Layout* L, int64_t* N) {
  int rc = check_sizes(B, T, H, K, V, cu, num_seqs, cu != nullptr, N);
  if (rc != KDA_OK) return rc;
  // With no tokens (B * T == 0) the token tensors are empty and may be NULL.
  if (B * T > 0 && (!q || !k || !g || !beta))
    return fail(KDA_EINVAL, "kda: a required input pointer is NULL");
  if (!A_log || !dt_bias) return fail(KDA_EINVAL, "kda: A_log or dt_bias is NULL");
  if (misaligned(q) || misaligned(k) || misaligned(g) || misaligned(dt_bias))
    return fail(KDA_EINVAL, "kda: q, k, g and dt_bias must be 16-byte aligned");
  if (!std::isfinite(scale)) return fail(KDA_EINVAL, "kda: scale is not finite");
  if (!std::isfinite(lower_bound) || lower_bound < -5.0f || lower_bound > 0.0f)
    return fail(KDA_EINVAL, "kda: lower_bound must lie in [-5, 0] (got %g)", (double)lower_bound);
  if (chunk != kda::C && chunk != kda::C32 && chunk != kda::C64)
    return fail(KDA_EINVAL, "kda: chunk must be 16, 32 or 64 (got %d)", chunk);
  if (!(fused ? kda::layout_fused(B, T, H, *N, L) : kda::layout_for(B, T, H, *N, chunk, L)))
    return fail(KDA_EINVAL, "kda: bad sizes");
  if (!workspace) return fail(KDA_EINVAL, "kda: workspace is NULL");
  if ((reinterpret_cast<uintptr_t>(workspace) & 255) != 0)
    return fail(KDA_EINVAL, "kda: workspace must be 256-byte aligned");
  if ((int64_t)workspace_bytes < L->total)
    return fail(KDA_EWORKSPACE, "kda: workspace has %zu bytes, needs %lld", workspace_bytes,
                (long long)L->total);
  return KDA_OK;
}

// Parts the call uses: `requested` (clamped to 1 .. kMaxParts) or, for 0, the
// library's choice for B*T rows.
static int parts_used(int64_t B, int64_t T, int requested) {
  if (B * T == 0) return 1;
  if (requested > 0) return requested < kda::kMaxParts ? requested : kda::kMaxParts;
  return kda::parts_for(B * T);
}

static int fwd_impl(const void* q, const void* k, const void* v, const void* g, const void* beta, float scale,
                    void* out, const float* A_log, const float* dt_bias, float lower_bound,
                    const void* initial_state, int initial_state_dtype, void* final_state,
                    int final_state_dtype, const int64_t* cu_seqlens, int64_t num_seqs, int64_t B,
                    int64_t T, int64_t H, int64_t K, int64_t V, void* workspace, size_t workspace_bytes,
                    hipStream_t stream, int chunk_req, int parts_req, int path_req, hipEvent_t* ev, int n_ev,
                    hipEvent_t* ev4, int precision = 0) {
  try {
    if ((!v || !out) && B * T > 0) return fail(KDA_EINVAL, "kda: v or out is NULL");
    auto dtype_ok = [](int d) { return d == KDA_DTYPE_NONE || d == KDA_DTYPE_BF16 || d == KDA_DTYPE_FP32; };
    if (!dtype_ok(initial_state_dtype) || !dtype_ok(final_state_dtype))
      return fail(KDA_EDTYPE, "kda: state dtype codes must be KDA_DTYPE_NONE/BF16/FP32");
    if ((initial_state == nullptr) != (initial_state_dtype == KDA_DTYPE_NONE))
      return fail(KDA_EDTYPE, "kda: initial_state pointer and dtype disagree");
    if ((final_state == nullptr) != (final_state_dtype == KDA_DTYPE_NONE))
      return fail(KDA_EDTYPE, "kda: final_state pointer and dtype disagree");
    if (initial_state && final_state && initial_state_dtype != final_state_dtype)
      return fail(KDA_EDTYPE, "kda: initial_state and final_state dtypes differ");
    if (parts_req < 0) return fail(KDA_EINVAL, "kda: parts must be >= 0 (got %d)", parts_req);
    if (chunk_req != 0 && chunk_req != kda::C && chunk_req != kda::C32 && chunk_req != kda::C64)
      return fail(KDA_EINVAL, "kda: chunk must be 0, 16, 32 or 64 (got %d)", chunk_req);
    const int path = resolve_path(chunk_req, parts_req, path_req);
    if (path < 0)
      return fail(KDA_EINVAL, "kda: path %d cannot run chunk=%d with parts=%d (the fused path takes 16-token "
                  "chunks and one part)", path_req, chunk_req, parts_req);
    const bool fused = path == KDA_PATH_FUSED;   // fused kernel only
    const bool both = path == KDA_PATH_AUTO;     // the library's choice
    // With cu_seqlens only the device knows the lengths: both paths are
    // enqueued and the scheduler kernel picks (the other path's kernels exit
    // at once).  B sequences of T tokens: the host picks and enqueues one.
    const int cus = kda::device_cus();
    int host_pick = -1;
    if (both && cu_seqlens == nullptr) {
      const int64_t nc = (T + kda::C - 1) / kda::C;
      host_pick = kda::choose_path(H, B, B * nc, nc, true, cus);
    }
    const bool run_split = !both || host_pick != KDA_PATH_FUSED;
    const bool run_fused = both && host_pick != KDA_PATH_SPLIT;
    const int chunk = chunk_req == 0 ? kda::default_chunk() : chunk_req;
    kda::Layout L;
    int64_t N = 0;
    int rc = validate_common(q, k, g, beta, scale, A_log, dt_bias, lower_bound, cu_seqlens, num_seqs, B, T,
                             H, K, V, workspace, workspace_bytes, chunk, fused, &L, &N);
    if (rc != KDA_OK) return rc;
    if (misaligned(v) || misaligned(out) || misaligned(initial_state) || misaligned(final_state))
      return fail(KDA_EINVAL, "kda: v, out and the states must be 16-byte aligned");
    const int P = fused || both ? 1 : parts_used(B, T, parts_req);
    const int n_need = fused ? 4 : 2 + 4 * P + (both ? 2 : 0);
    if (ev && n_ev != n_need)
      return fail(KDA_EINVAL, "kda: %d events given, this call needs %d", n_ev, n_need);
    int dev = 0;
    rc = check_device(&dev);
    if (rc != KDA_OK) return rc;
    if (fused) {
      hipError_t e = hipSuccess;
      auto rec = [&](int i) {
        if (e == hipSuccess && ev) e = hipEventRecord(ev[i], stream);
        if (e == hipSuccess && ev4) e = hipEventRecord(ev4[i], stream);
      };
      char* ws = static_cast<char*>(workspace);
      rec(0);
      if (e == hipSuccess) {
        kda::SchedArgs sa{cu_seqlens, N, B, T, H, 1, B * T > 0 ? B * T : 1, KDA_PATH_FUSED, ws, L};
        sa.cus = cus;
        e = kda::launch_sched(sa, stream);
      }
      rec(1);
      if (e == hipSuccess && ev4) e = hipEventRecord(ev4[2], stream);
      if (e == hipSuccess && ev) e = hipEventRecord(ev[2], stream);
      if (e == hipSuccess) {
        kda::FusedArgs fa{static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                          static_cast<const uint16_t*>(v), static_cast<const uint16_t*>(g),
                          static_cast<const uint16_t*>(beta), static_cast<uint16_t*>(out), A_log, dt_bias, scale,
                          lower_bound, initial_state, final_state,
                          initial_state ? initial_state_dtype : final_state_dtype, N, H, ws, L};
        fa.cus = cus;
        e = kda::launch_fused(fa, stream);
      }
      if (e == hipSuccess && ev) e = hipEventRecord(ev[3], stream);
      if (e == hipSuccess && ev4) e = hipEventRecord(ev4[3], stream);
      if (e != hipSuccess) return fail(KDA_EHIP, "kda: launch or event call: %s", hipGetErrorString(e));
      return KDA_OK;
    }
    SideRes* side = nullptr;
    std::unique_lock<std::mutex> lock;
    if (P > 1) {
      lock = std::unique_lock<std::mutex>(g_side[dev].mu);
      rc = side_resources(dev, &side);
      if (rc != KDA_OK) return rc;
    }
    hipStream_t rstream = P > 1 ? side->side : stream;   // where the recurrence runs

    hipError_t e = hipSuccess;
    auto rec = [&](int i, hipStream_t st) {
      if (e == hipSuccess && ev) e = hipEventRecord(ev[i], st);
    };
    auto rec4 = [&](int i) {
      if (e == hipSuccess && ev4) e = hipEventRecord(ev4[i], stream);
    };
    char* ws = static_cast<char*>(workspace);
    const int64_t rows = B * T;
    const int64_t part_rows = P > 1 ? (rows + P - 1) / P : (rows > 0 ? rows : 1);
    // B sequences of T tokens on the split path in one part: the tables are
    // a function of the chunk index, so no scheduler kernel runs; the prep
    // kernel computes the entries and writes the header.
    const bool fixed = cu_seqlens == nullptr && P == 1 && chunk == kda::C && run_split && !run_fused;
    rec(0, stream);
    rec4(0);
    if (e == hipSuccess && !fixed) {
      kda::SchedArgs sa{cu_seqlens, N, B, T, H, P, part_rows,
                        both ? (host_pick >= 0 ? host_pick : KDA_PATH_AUTO) : KDA_PATH_SPLIT, ws, L};
      sa.cus = cus;
      e = kda::launch_sched(sa, stream);
    }
    rec(1, stream);
    rec4(1);
    const int sdt = initial_state ? initial_state_dtype : final_state_dtype;
    for (int p = 0; p < P && e == hipSuccess; ++p) {
      // chunks whose first row lies in the part's rows: at most one per 16 rows
      // plus one per sequence start
      const int64_t bound = P == 1 ? L.max_chunks : std::min(L.max_chunks, part_rows / chunk + N + 1);
      kda::PrepArgs pa{static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                       static_cast<const uint16_t*>(g), static_cast<const uint16_t*>(beta), A_log, dt_bias,
                       scale, lower_bound, H, p, bound, ws, L};
      if (fixed) {
        pa.fixed_T = T;
        pa.fixed_B = B;
      }
      pa.precision = precision & KDA_PREC_NEUMANN_FP16;
      rec(2 + 2 * p, stream);
      if (e == hipSuccess && run_split) e = kda::launch_prep(pa, stream);
      rec(3 + 2 * p, stream);
      if (p == P - 1) rec4(2);   // after the last chunk prep
      if (P > 1 && e == hipSuccess) {
        e = hipEventRecord(side->prep_done[p], stream);
        if (e == hipSuccess) e = hipStreamWaitEvent(rstream, side->prep_done[p], 0);
      }
      const int64_t lo = p * part_rows, hi = p == P - 1 ? (INT64_MAX / 2) : (p + 1) * part_rows;
      kda::RecurArgs ra{static_cast<const uint16_t*>(v), static_cast<uint16_t*>(out), initial_state, final_state,
                        sdt, N, H, p, lo, hi, ws, L};
      ra.precision = precision & ~KDA_PREC_NEUMANN_FP16;   // the recurrence's own bits
      ra.tiles = kda::recur_tiles(N * H, cu_seqlens == nullptr, cus);
      ra.cus = cus;
      if (fixed) ra.fixed_T = T;
      rec(2 + 2 * P + 2 * p, rstream);
      if (e == hipSuccess && run_split) e = kda::launch_recur(ra, rstream);
      rec(3 + 2 * P + 2 * p, rstream);
    }
    if (P > 1 && e == hipSuccess) {
      e = hipEventRecord(side->join, rstream);
      if (e == hipSuccess) e = hipStreamWaitEvent(stream, side->join, 0);
    }
    if (both) {   // exits at once unless the scheduler chose it (then prep and recurrence exited)
      rec(6, stream);
      if (e == hipSuccess && run_fused) {
        kda::FusedArgs fa{static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                          static_cast<const uint16_t*>(v), static_cast<const uint16_t*>(g),
                          static_cast<const uint16_t*>(beta), static_cast<uint16_t*>(out), A_log, dt_bias, scale,
                          lower_bound, initial_state, final_state, sdt, N, H, ws, L};
        fa.cus = cus;
        e = kda::launch_fused(fa, stream);
      }
      rec(7, stream);
    }
    rec4(3);
    if (e != hipSuccess) return fail(KDA_EHIP, "kda: launch or event call: %s", hipGetErrorString(e));
    return KDA_OK;
  } catch (...) {
    return fail(KDA_EHIP, "kda: unexpected C++ exception");
  }
}

int kda_fwd(const void* q, const void* k, const void* v, const void* g, const void* beta, float scale,
            void* out, const float* A_log, const float* dt_bias, float lower_bound,
            const void* initial_state, int initial_state_dtype, void* final_state,
            int final_state_dtype, const int64_t* cu_seqlens, int64_t num_seqs, int64_t B,
            int64_t T, int64_t H, int64_t K, int64_t V, void* workspace, size_t workspace_bytes,
            hipStream_t stream) {
  // B sequences of T tokens: the library's segment count is known on the
  // host; above 1 (few heads, long sequences) the call cuts the sequences
  // when the workspace holds the segmented layout.
  if (cu_seqlens == nullptr && workspace != nullptr) {
    int64_t N = 0;
    if (check_sizes(B, T, H, K, V, nullptr, num_seqs, 0, &N) == KDA_OK) {
      const int S = choose_segments(B, T, H, N, false);
      SegLayout SL;
      if (S > 1 && seg_layout(B, T, H, N, S, &SL) && (int64_t)workspace_bytes >= SL.total)
        return kda_fwd_segmented(q, k, v, g, beta, scale, out, A_log, dt_bias, lower_bound, initial_state,
                                 initial_state_dtype, final_state, final_state_dtype, nullptr, num_seqs, B, T, H,
                                 K, V, S, workspace, workspace_bytes, stream);
    }
  }
  return fwd_impl(q, k, v, g, beta, scale, out, A_log, dt_bias, lower_bound, initial_state,
                  initial_state_dtype, final_state, final_state_dtype, cu_seqlens, num_seqs, B, T, H, K, V,
                  workspace, workspace_bytes, stream, 0, 0, KDA_PATH_AUTO, nullptr, 0, nullptr);
}

int kda_fwd_profiled(const void* q, const void* k, const void* v, const void* g, const void* beta,
                     float scale, void* out, const float* A_log, const float* dt_bias, float lower_bound,
                     const void* initial_state, int initial_state_dtype, void* final_state,
                     int final_state_dtype, const int64_t* cu_seqlens, int64_t num_seqs, int64_t B,
                     int64_t T, int64_t H, int64_t K, int64_t V, void* workspace,
                     size_t workspace_bytes, hipStream_t stream, hipEvent_t events[4]) {
  if (events == nullptr || !events[0] || !events[1] || !events[2] || !events[3])
    return fail(KDA_EINVAL, "kda: kda_fwd_profiled needs four events");
  return fwd_impl(q, k, v, g, beta, scale, out, A_log, dt_bias, lower_bound, initial_state,
                  initial_state_dtype, final_state, final_state_dtype, cu_seqlens, num_seqs, B, T, H, K, V,
                  workspace, workspace_bytes, stream, 0, 0, KDA_PATH_AUTO, nullptr, 0, events);
}

int kda_fwd_precision(const void* q, const void* k, const void* v, const void* g, const void* beta, float scale,
                      void* out, const float* A_log, const float* dt_bias, float lower_bound,
                      const void* initial_state, int initial_state_dtype, void* final_state, int final_state_dtype,
                      const int64_t* cu_seqlens, int64_t num_seqs, int64_t B, int64_t T, int64_t H, int64_t K,
                      int64_t V, void* workspace, size_t workspace_bytes, hipStream_t stream, int variant) {
  const int all = KDA_PREC_BF16_STATE | KDA_PREC_BF16_INVERSE | KDA_PREC_BF16_STATE_PRODUCTS |
                  KDA_PREC_NEUMANN_FP16;
  if (variant < 0 || (variant & ~all) != 0)
    return fail(KDA_EINVAL, "kda: precision variant must be a combination of KDA_PREC_* bits (got %d)", variant);
  return fwd_impl(q, k, v, g, beta, scale, out, A_log, dt_bias, lower_bound, initial_state, initial_state_dtype,
                  final_state, final_state_dtype, cu_seqlens, num_seqs, B, T, H, K, V, workspace, workspace_bytes,
                  stream, kda::C, 1, KDA_PATH_SPLIT, nullptr, 0, nullptr, variant);
}

int kda_fwd_parts(int64_t B, int64_t T, int parts) {
  if (B < 0 || T < 0 || parts < 0) return 0;
  return parts_used(B, T, parts);
}

int kda_fwd_ex(const void* q, const void* k, const void* v, const void* g, const void* beta, float scale,
               void* out, const float* A_log, const float* dt_bias, float lower_bound,
               const void* initial_state, int initial_state_dtype, void* final_state, int final_state_dtype,
               const int64_t* cu_seqlens, int64_t num_seqs, int64_t B, int64_t T, int64_t H, int64_t K,
               int64_t V, void* workspace, size_t workspace_bytes, hipStream_t stream, int chunk,
               int parts, int path, hipEvent_t* events, int num_events) {
  if (events != nullptr)
    for (int i = 0; i < num_events; ++i)
      if (!events[i]) return fail(KDA_EINVAL, "kda: event %d is NULL", i);
  return fwd_impl(q, k, v, g, beta, scale, out, A_log, dt_bias, lower_bound, initial_state,
                  initial_state_dtype, final_state, final_state_dtype, cu_seqlens, num_seqs, B, T, H, K, V,
                  workspace, workspace_bytes, stream, chunk, parts, path, events, num_events, nullptr);
}

}  // extern "C"

// ---- the fused path without a caller workspace ------------------------------

namespace {

// The fused path's workspace is only the header and the per-sequence tables
// (layout_fused): for up to kNoAllocMaxSeqs sequences it fits in this array,
// one copy per GPU, held until the process ends.  Host code never uses the
// name `scratch` as an address (on the host it is a stand-in, not the device
// copy): g_scratch[dev] holds the device address hipGetSymbolAddress gives
// for device dev.
constexpr int64_t kNoAllocMaxSeqs = 16384;
constexpr size_t kScratchBytes = 256 + 16 * kNoAllocMaxSeqs + 4 * kNoAllocMaxSeqs;   // 320 KiB + 256 B
static_assert(sizeof(kda::WsHeader) == 256 && sizeof(kda::SeqEntry) == 16, "scratch sizing");
static __device__ __align__(256) char scratch[kScratchBytes];

char* g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of this device's scratch array (looked up once per device,
// with the device current).
int scratch_ptr(int dev, char** out) {
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(KDA_EHIP, "kda: hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    g_scratch[dev] = static_cast<char*>(p);
  }
  *out = g_scratch[dev];
  return KDA_OK;
}

}  // namespace

extern "C" {

int kda_fwd_fused_noalloc(const void* q, const void* k, const void* v, const void* g, const void* beta, float scale,
                          void* out, const float* A_log, const float* dt_bias, float lower_bound,
                          const void* initial_state, int initial_state_dtype, void* final_state,
                          int final_state_dtype, const int64_t* cu_seqlens, int64_t num_seqs, int64_t B, int64_t T,
                          int64_t H, int64_t K, int64_t V, hipStream_t stream) {
  try {
    int64_t N = 0;
    int rc = check_sizes(B, T, H, K, V, cu_seqlens, num_seqs, 0, &N);
    if (rc != KDA_OK) return rc;
    if (N > kNoAllocMaxSeqs)
      return fail(KDA_EINVAL, "kda: kda_fwd_fused_noalloc takes at most %lld sequences (got %lld)",
                  (long long)kNoAllocMaxSeqs, (long long)N);
    kda::Layout L;
    if (!kda::layout_fused(B, T, H, N, &L) || L.total > (int64_t)kScratchBytes)
      return fail(KDA_EINVAL, "kda: sizes do not fit the static scratch");
    int dev = 0;
    rc = check_device(&dev);
    if (rc != KDA_OK) return rc;
    char* ws = nullptr;
    rc = scratch_ptr(dev, &ws);
    if (rc != KDA_OK) return rc;
    return fwd_impl(q, k, v, g, beta, scale, out, A_log, dt_bias, lower_bound, initial_state, initial_state_dtype,
                    final_state, final_state_dtype, cu_seqlens, num_seqs, B, T, H, K, V, ws, kScratchBytes, stream,
                    kda::C, 0, KDA_PATH_FUSED, nullptr, 0, nullptr);
  } catch (...) {
    return fail(KDA_EHIP, "kda: unexpected C++ exception");
  }
}

int kda_fwd_num_events(int64_t B, int64_t T, int chunk, int parts, int path) {
  const int p = resolve_path(chunk, parts, path);
  if (p < 0 || B < 0 || T < 0) return 0;
  if (p == KDA_PATH_FUSED) return 4;
  if (p == KDA_PATH_AUTO) return 8;
  return 2 + 4 * parts_used(B, T, parts);
}

int kda_fwd_path_taken(const void* workspace, hipStream_t stream, int* path) {
  if (!workspace || !path) return fail(KDA_EINVAL, "kda: workspace or path is NULL");
  hipError_t e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return fail(KDA_EHIP, "kda: hipStreamSynchronize: %s", hipGetErrorString(e));
  int32_t p = 0;
  e = hipMemcpy(&p, static_cast<const char*>(workspace) + offsetof(kda::WsHeader, path), sizeof p,
                hipMemcpyDeviceToHost);
  if (e != hipSuccess) return fail(KDA_EHIP, "kda: hipMemcpy: %s", hipGetErrorString(e));
  *path = p;
  return KDA_OK;
}


int kda_fwd_segments(int64_t B, int64_t T, int64_t H, int64_t num_seqs, int has_cu_seqlens) {
  int64_t N = 0;
  if (check_sizes(B, T, H, kda::K, kda::V, nullptr, num_seqs, has_cu_seqlens, &N) != KDA_OK) return 0;
  return choose_segments(B, T, H, N, has_cu_seqlens != 0);
}

size_t kda_fwd_segmented_workspace_bytes(int64_t B, int64_t T, int64_t H, int64_t num_seqs, int has_cu_seqlens,
                                         int segments) {
  int64_t N = 0;
  if (segments < 0 || segments > 4096) return 0;
  if (check_sizes(B, T, H, kda::K, kda::V, nullptr, num_seqs, has_cu_seqlens, &N) != KDA_OK) return 0;
  if (segments == 0) segments = choose_segments(B, T, H, N, has_cu_seqlens != 0);
  if (segments == 1) return kda_fwd_workspace_bytes_ex(B, T, H, num_seqs, has_cu_seqlens, 0, 0, KDA_PATH_AUTO);
  if (N * segments >= (int64_t(1) << 30) || N * segments * H >= (int64_t(1) << 31)) return 0;
  SegLayout L;
  return seg_layout(B, T, H, N, segments, &L) ? (size_t)L.total : 0;
}

int kda_fwd_segmented(const void* q, const void* k, const void* v, const void* g, const void* beta, float scale,
                      void* out, const float* A_log, const float* dt_bias, float lower_bound,
                      const void* initial_state, int initial_state_dtype, void* final_state, int final_state_dtype,
                      const int64_t* cu_seqlens, int64_t num_seqs, int64_t B, int64_t T, int64_t H, int64_t K,
                      int64_t V, int segments, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  try {
    if (segments < 0 || segments > 4096)
      return fail(KDA_EINVAL, "kda: segments must lie in 0 .. 4096 (got %d)", segments);
    if (segments == 0) {   // the library's choice
      int64_t N0 = 0;
      const int rc0 = check_sizes(B, T, H, K, V, cu_seqlens, num_seqs, cu_seqlens != nullptr, &N0);
      if (rc0 != KDA_OK) return rc0;
      segments = choose_segments(B, T, H, N0, cu_seqlens != nullptr);
    }
    if (segments == 1)
      return fwd_impl(q, k, v, g, beta, scale, out, A_log, dt_bias, lower_bound, initial_state,
                      initial_state_dtype, final_state, final_state_dtype, cu_seqlens, num_seqs, B, T, H, K, V,
                      workspace, workspace_bytes, stream, 0, 0, KDA_PATH_AUTO, nullptr, 0, nullptr);
    // Every check of kda_fwd, on the caller's arguments, before any HIP call.
    if ((!v || !out) && B * T > 0) return fail(KDA_EINVAL, "kda: v or out is NULL");
    auto dtype_ok = [](int d) { return d == KDA_DTYPE_NONE || d == KDA_DTYPE_BF16 || d == KDA_DTYPE_FP32; };
    if (!dtype_ok(initial_state_dtype) || !dtype_ok(final_state_dtype))
      return fail(KDA_EDTYPE, "kda: state dtype codes must be KDA_DTYPE_NONE/BF16/FP32");
    if ((initial_state == nullptr) != (initial_state_dtype == KDA_DTYPE_NONE))
      return fail(KDA_EDTYPE, "kda: initial_state pointer and dtype disagree");
    if ((final_state == nullptr) != (final_state_dtype == KDA_DTYPE_NONE))
      return fail(KDA_EDTYPE, "kda: final_state pointer and dtype disagree");
    if (initial_state && final_state && initial_state_dtype != final_state_dtype)
      return fail(KDA_EDTYPE, "kda: initial_state and final_state dtypes differ");
    int64_t N = 0;
    int rc = check_sizes(B, T, H, K, V, cu_seqlens, num_seqs, cu_seqlens != nullptr, &N);
    if (rc != KDA_OK) return rc;
    if (N * segments >= (int64_t(1) << 30) || N * segments * H >= (int64_t(1) << 31))
      return fail(KDA_EINVAL, "kda: N * segments too large");
    SegLayout SL;
    if (!seg_layout(B, T, H, N, segments, &SL)) return fail(KDA_EINVAL, "kda: bad sizes");
    if (!workspace) return fail(KDA_EINVAL, "kda: workspace is NULL");
    if ((reinterpret_cast<uintptr_t>(workspace) & 255) != 0)
      return fail(KDA_EINVAL, "kda: workspace must be 256-byte aligned");
    if ((int64_t)workspace_bytes < SL.total)
      return fail(KDA_EWORKSPACE, "kda: workspace has %zu bytes, needs %lld", workspace_bytes,
                  (long long)SL.total);
    if (misaligned(v) || misaligned(out) || misaligned(initial_state) || misaligned(final_state))
      return fail(KDA_EINVAL, "kda: v, out and the states must be 16-byte aligned");
    char* ws = static_cast<char*>(workspace);
    int64_t* seg_cu = reinterpret_cast<int64_t*>(ws + SL.seg_cu);
    kda::Layout probe;
    int64_t NS = 0;
    rc = validate_common(q, k, g, beta, scale, A_log, dt_bias, lower_bound, seg_cu, N * segments, 1, B * T, H, K,
                         V, ws + SL.inner, (size_t)SL.inner_bytes, kda::C, false, &probe, &NS);
    if (rc != KDA_OK) return rc;
    rc = check_device(nullptr);
    if (rc != KDA_OK) return rc;

    uint16_t* Am = reinterpret_cast<uint16_t*>(ws + SL.A);
    float* Bm = reinterpret_cast<float*>(ws + SL.B);
    float* starts = reinterpret_cast<float*>(ws + SL.starts);
    const int64_t NS_ = N * segments, rows = B * T;
    const int sdt = initial_state ? initial_state_dtype : final_state_dtype;

    kda::Layout L;   // the plain forward's workspace for the segments
    if (!kda::layout_for(1, rows, H, NS_, kda::C, &L)) return fail(KDA_EINVAL, "kda: bad sizes");
    hipError_t e = kda::launch_seg_cu(kda::SegArgs{cu_seqlens, N, T, segments, seg_cu}, stream);
    if (e != hipSuccess) return fail(KDA_EHIP, "kda: segment launch: %s", hipGetErrorString(e));
    // The segments' chunk records: scheduler and chunk prep of the split path.
    char* const iws = ws + SL.inner;
    const int cus = kda::device_cus();
    kda::SchedArgs sa{seg_cu, NS_, 1, rows, H, 1, rows > 0 ? rows : 1, KDA_PATH_SPLIT, iws, L};
    sa.cus = cus;
    e = kda::launch_sched(sa, stream);
    if (e == hipSuccess)
      e = kda::launch_prep(kda::PrepArgs{static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                                         static_cast<const uint16_t*>(g), static_cast<const uint16_t*>(beta), A_log,
                                         dt_bias, scale, lower_bound, H, 0, L.max_chunks, iws, L},
                           stream);
    // One recurrence launch over those records, two argument sets and no
    // outputs: B_j (the values from a zero start) and A_j (zero values from
    // the identity).
    if (e == hipSuccess) {
      kda::RecurArgs ra{static_cast<const uint16_t*>(v), nullptr, nullptr, Bm, KDA_DTYPE_FP32, NS_, H, 0, 0,
                        INT64_MAX / 2, iws, L, 2, Am};
      ra.cus = cus;
      e = kda::launch_recur(ra, stream);
    }
    if (e != hipSuccess) return fail(KDA_EHIP, "kda: launch: %s", hipGetErrorString(e));
    // the segments' start states and the sequences' final states
    e = kda::launch_prefix(kda::PrefixArgs{Am, Bm, starts, initial_state, final_state, sdt, N, H, segments,
                                           reinterpret_cast<const kda::WsHeader*>(ws + SL.inner), seg_cu},
                           stream);
    if (e != hipSuccess) return fail(KDA_EHIP, "kda: prefix launch: %s", hipGetErrorString(e));
    // the outputs, every segment from its true start
    kda::RecurArgs ro{static_cast<const uint16_t*>(v), static_cast<uint16_t*>(out), starts, nullptr,
                      KDA_DTYPE_FP32, NS_, H, 0, 0, INT64_MAX / 2, iws, L};
    ro.cus = cus;
    e = kda::launch_recur(ro, stream);
    if (e != hipSuccess) return fail(KDA_EHIP, "kda: recurrence launch: %s", hipGetErrorString(e));
    return KDA_OK;
  } catch (...) {
    return fail(KDA_EHIP, "kda: unexpected C++ exception");
  }
}

int kda_debug_prep(const void* q, const void* k, const void* g, const void* beta, float scale,
                   const float* A_log, const float* dt_bias, float lower_bound, const int64_t* cu_seqlens,
                   int64_t num_seqs, int64_t B, int64_t T, int64_t H, int64_t K, void* workspace,
                   size_t workspace_bytes, hipStream_t stream, int chunk) {
  try {
    kda::Layout L;
    int64_t N = 0;
    int rc = validate_common(q, k, g, beta, scale, A_log, dt_bias, lower_bound, cu_seqlens, num_seqs, B, T,
                             H, K, kda::V, workspace, workspace_bytes, chunk, false, &L, &N);
    if (rc != KDA_OK) return rc;
    rc = check_device();
    if (rc != KDA_OK) return rc;
    char* ws = static_cast<char*>(workspace);
    kda::SchedArgs sa{cu_seqlens, N, B, T, H, 1, B * T > 0 ? B * T : 1, KDA_PATH_SPLIT, ws, L};
    hipError_t e = kda::launch_sched(sa, stream);
    if (e != hipSuccess) return fail(KDA_EHIP, "kda: scheduler launch: %s", hipGetErrorString(e));
    kda::PrepArgs pa{static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                     static_cast<const uint16_t*>(g), static_cast<const uint16_t*>(beta), A_log, dt_bias,
                     scale, lower_bound, H, 0, L.max_chunks, ws, L};
    e = kda::launch_prep(pa, stream);
    if (e != hipSuccess) return fail(KDA_EHIP, "kda: prep launch: %s", hipGetErrorString(e));
    return KDA_OK;
  } catch (...) {
    return fail(KDA_EHIP, "kda: unexpected C++ exception");
  }
}

int kda_debug_set_spin_limit(int polls) {
  kda::g_spin_limit.store(polls < 0 ? kda::kSpinLimit : polls, std::memory_order_relaxed);
  return KDA_OK;
}

int kda_decode(const void* q, const void* k, const void* v, const void* g, const void* beta, float scale,
               void* out, const float* A_log, const float* dt_bias, float lower_bound,
               const void* initial_state, int initial_state_dtype, void* final_state, int final_state_dtype,
               int64_t N, int64_t H, int64_t K, int64_t V, hipStream_t stream) {
  try {
    if (N < 0 || H < 1)
      return fail(KDA_EINVAL, "kda: need N >= 0, H >= 1 (got N=%lld H=%lld)", (long long)N, (long long)H);
    if (K != kda::K || V != kda::V)
      return fail(KDA_EINVAL, "kda: K and V must both be 128 (got K=%lld V=%lld)", (long long)K, (long long)V);
    if (N * H >= (int64_t(1) << 31)) return fail(KDA_EINVAL, "kda: N*H too large");
    if (N > 0 && (!q || !k || !v || !g || !beta || !out))
      return fail(KDA_EINVAL, "kda: a required token pointer is NULL");
    if (!A_log || !dt_bias) return fail(KDA_EINVAL, "kda: A_log or dt_bias is NULL");
    auto dtype_ok = [](int d) { return d == KDA_DTYPE_NONE || d == KDA_DTYPE_BF16 || d == KDA_DTYPE_FP32; };
    if (!dtype_ok(initial_state_dtype) || !dtype_ok(final_state_dtype))
      return fail(KDA_EDTYPE, "kda: state dtype codes must be KDA_DTYPE_NONE/BF16/FP32");
    if ((initial_state == nullptr) != (initial_state_dtype == KDA_DTYPE_NONE))
      return fail(KDA_EDTYPE, "kda: initial_state pointer and dtype disagree");
    if ((final_state == nullptr) != (final_state_dtype == KDA_DTYPE_NONE))
      return fail(KDA_EDTYPE, "kda: final_state pointer and dtype disagree");
    if (initial_state && final_state && initial_state_dtype != final_state_dtype)
      return fail(KDA_EDTYPE, "kda: initial_state and final_state dtypes differ");
    if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(g) || misaligned(out) ||
        misaligned(dt_bias) || misaligned(initial_state) || misaligned(final_state))
      return fail(KDA_EINVAL, "kda: q, k, v, g, out, dt_bias and the states must be 16-byte aligned");
    if (!std::isfinite(scale)) return fail(KDA_EINVAL, "kda: scale is not finite");
    if (!std::isfinite(lower_bound) || lower_bound < -5.0f || lower_bound > 0.0f)
      return fail(KDA_EINVAL, "kda: lower_bound must lie in [-5, 0] (got %g)", (double)lower_bound);
    int rc = check_device(nullptr);
    if (rc != KDA_OK) return rc;
    kda::DecodeArgs da{static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                       static_cast<const uint16_t*>(v), static_cast<const uint16_t*>(g),
                       static_cast<const uint16_t*>(beta), A_log, dt_bias, scale, lower_bound, initial_state,
                       final_state, initial_state ? initial_state_dtype : final_state_dtype,
                       static_cast<uint16_t*>(out), N, H};
    hipError_t e = kda::launch_decode(da, stream);
    if (e != hipSuccess) return fail(KDA_EHIP, "kda: decode launch: %s", hipGetErrorString(e));
    return KDA_OK;
  } catch (...) {
    return fail(KDA_EHIP, "kda: unexpected C++ exception");
  }
}

int kda_fwd_check_status(const void* workspace, hipStream_t stream, int* status) {
  if (!workspace || !status) return fail(KDA_EINVAL, "kda: workspace or status is NULL");
  hipError_t e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return fail(KDA_EHIP, "kda: hipStreamSynchronize: %s", hipGetErrorString(e));
  int32_t st = 0;
  e = hipMemcpy(&st, workspace, sizeof st, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return fail(KDA_EHIP, "kda: hipMemcpy: %s", hipGetErrorString(e));
  *status = st;
  return KDA_OK;
}

}  // extern "C"
