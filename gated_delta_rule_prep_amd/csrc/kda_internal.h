// kda_internal.h -- types, constants and launchers shared by the gfx950 KDA
// kernels and the C-ABI layer.  Not part of the public ABI (include/kda.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/kda.h"   // the KDA_PATH_* codes of the path choice

namespace kda {

constexpr int C = 16;     // chunk size of the 16-token kernels (tokens per chunk)
constexpr int C32 = 32;   // chunk size of the 32-token kernels
constexpr int C64 = 64;   // chunk size of the 64-token kernels
constexpr int K = 128;    // key channels
constexpr int V = 128;    // value channels

// Chunk record, one per (chunk, head), chunk-major: record (c, h) at
// (c H + h) REC_BYTES in the records region, so the records of one chunk are
// contiguous and the prep kernel's workgroups of a chunk write one stream
// (T = 8192, H = 96, 12 ragged sequences: prep 0.284 -> 0.248 ms against
// head-major).  Offsets in bytes.
constexpr int REC_QH = 0;        // Qhat  fp16 [16][128], 32-block channel order (see kPermCh)
constexpr int REC_NK = 4096;     // -Khat fp16 [16][128], same channel order
constexpr int REC_KB = 8192;     // Kbar  fp16 [16][128], token-major, natural channel order
constexpr int REC_T = 12288;     // T^T   fp16 [16][16]
constexpr int REC_MQK = 12800;   // Mqk^T fp16 [16][16]
constexpr int REC_GAM = 13312;   // gamma fp32 [128], channel c at slot kGamSlot(c)
constexpr int REC_BYTES = 13824;

// Chunk record of the 32-token kernels, one per (chunk, head), chunk-major.
// T and Mqk are row-major with the columns (tokens) of each row stored in the
// permuted order kPermCh, the same order as the channels of Qhat / -W: a lane
// of the recurrence then reads the 8 k-values of its 16x16x32 MFMA operand as
// one 16-byte piece, and the tokens it gets are exactly the accumulator rows
// (4g .. 4g+3 of both 16-token tiles) that it holds for E.
constexpr int REC32_QH = 0;        // Qhat  fp16 [32][128], channels in kPermCh order per 32-block
constexpr int REC32_NW = 8192;     // -W    fp16 [32][128], same channel order
constexpr int REC32_KB = 16384;    // Kbar  fp16 [32][128], token-major, natural channel order
constexpr int REC32_T = 24576;     // T     fp16 [32][32], row-major, columns in kPermCh order
constexpr int REC32_MQK = 26624;   // Mqk   fp16 [32][32], row-major, columns in kPermCh order
constexpr int REC32_GAM = 28672;   // gamma fp32 [128], channel c at slot kGamSlot(c)
constexpr int REC32_BYTES = 29184;

// Chunk record of the 64-token kernels, one per (chunk, head), chunk-major.
// Qhat, -W and Kbar as in the 32-token record with 64 token rows.  T and Mqk
// (64 x 64) are stored as 8 blocks of 16 rows x 32 columns, block (t, u) =
// rows 16t .. 16t + 15, token columns 32u .. 32u + 31 in kPermCh order, at
// (2t + u) x 1024 bytes, so the 16-byte operand pieces of one MFMA are one
// contiguous kilobyte.  The blocks above the diagonal (t < 2u) hold zeros.
constexpr int REC64_QH = 0;        // Qhat  fp16 [64][128], channels in kPermCh order per 32-block
constexpr int REC64_NW = 16384;    // -W    fp16 [64][128], same channel order
constexpr int REC64_KB = 32768;    // Kbar  fp16 [64][128], token-major, natural channel order
constexpr int REC64_T = 49152;     // T     fp16, 8 blocks [16][32] as above
constexpr int REC64_MQK = 57344;   // Mqk   fp16, 8 blocks [16][32] as above
constexpr int REC64_GAM = 65536;   // gamma fp32 [128], channel c at slot kGamSlot(c)
constexpr int REC64_BYTES = 66048;

// Slot of channel c = 64 r + 16 a + 4 b + i in the stored gamma: lane
// L = 16 b + 4 a + i of a recurrence wave reads slots 2L and 2L + 1 (r = 0, 1),
// i.e. exactly the decay factors that its 16-lane row (lanes with the same b)
// hands out by row broadcast.
__host__ __device__ constexpr int kGamSlot(int c) {
  return 2 * (16 * ((c >> 2) & 3) + 4 * ((c >> 4) & 3) + (c & 3)) + (c >> 6);
}

// The token rows are cut into at most kMaxParts consecutive ranges ("parts");
// the prep kernel of part p + 1 runs while the recurrence works on part p.
constexpr int kMaxParts = 8;

// Workspace header (first 256 bytes).
struct WsHeader {
  int32_t status;                   // KDA_STATUS_OK or an OR of KDA_STATUS_* bits
  int32_t chunk_count;              // number of valid chunk-table entries
  int32_t part_first[kMaxParts + 1];  // chunk-table index of the first chunk of each part; [parts] = count
  int32_t path;                     // KDA_PATH_SPLIT or KDA_PATH_FUSED: the kernels of the other path exit
  int32_t pad[52];
};
static_assert(sizeof(WsHeader) == 256, "header size");

struct ChunkEntry {     // chunk table entry
  int32_t seq;          // sequence index n
  int32_t row0;         // first flattened token row (b * T + t) of the chunk
  int32_t len;          // tokens in the chunk (1 .. chunk size)
};

struct SeqEntry {
  int32_t first_chunk;
  int32_t nchunks;
  int32_t row0;         // first flattened token row of the sequence
  int32_t len;          // tokens in the sequence
};

// B sequences of T tokens (no cu_seqlens): the scheduler's table entries
// follow from the index, so the split path with one part runs without the
// scheduler kernel and computes them itself.
__host__ __device__ inline ChunkEntry fixed_chunk(int64_t T, int64_t chunk_size, int64_t i) {
  const int64_t nc = (T + chunk_size - 1) / chunk_size, n = i / nc, c = i - n * nc;
  const int64_t rem = T - c * chunk_size;
  return ChunkEntry{(int32_t)n, (int32_t)(n * T + c * chunk_size), (int32_t)(rem < chunk_size ? rem : chunk_size)};
}
__host__ __device__ inline SeqEntry fixed_seq(int64_t T, int64_t chunk_size, int64_t n) {
  const int64_t nc = (T + chunk_size - 1) / chunk_size;
  return SeqEntry{(int32_t)(n * nc), (int32_t)nc, (int32_t)(n * T), (int32_t)T};
}

struct Layout {
  int64_t chunk_table;  // byte offsets into the workspace
  int64_t seq_table;
  int64_t order;
  int64_t chunk;        // tokens per chunk: C, C32 or C64
  int64_t records;
  int64_t rec_bytes;
  int64_t max_chunks;
  int64_t state;        // fp32 [N][H][V][K]: the state handed from one part to the next
  int64_t total;
};

// Returns false if the sizes or the chunk size (C, C32 or C64) are invalid.
bool layout_for(int64_t B, int64_t T, int64_t H, int64_t N, int chunk, Layout* out);
int parts_for(int64_t rows);   // parts used for B*T token rows when the caller does not choose
int default_chunk();           // chunk size used when the caller does not choose

// Compute units of a whole MI355X.  The launch shapes and the path estimate
// take the current device's own count (device_cus: a partitioned MI355X
// exposes fewer), kCUs only where it cannot be read.
constexpr int kCUs = 256;
int device_cus();   // host only

struct SchedArgs {
  const int64_t* cu;    // device, N + 1 entries, or nullptr
  int64_t N, B, T, H;
  int parts;            // 1 .. kMaxParts
  int64_t part_rows;    // token rows per part (the last part takes the rest)
  int path;             // KDA_PATH_SPLIT / KDA_PATH_FUSED, or KDA_PATH_AUTO: choose from the lengths
  char* ws;
  Layout lay;
  int cus = kCUs;       // compute units of the device (for the path estimate)
};

// Fused-kernel value-column tiling: 64 columns per workgroup (two per
// (sequence, head)) while two tiles per pair fit on the CUs at once, else 128.
// (A workgroup takes most of a CU's LDS, so workgroups beyond the CU count
// wait for a second round: 2 x 4096 tokens, H = 96, 0.866 ms with 384
// workgroups of 64 columns against 0.513 with 192 of 128.)
inline __host__ __device__ bool fused_two_tiles(int64_t pairs, int cus) { return 2 * pairs <= cus; }

// The recurrence's value tiles per (sequence, head) for `pairs` chains (the
// sequence-head pairs of the launch): 4 while that still gives one workgroup
// per CU, else 2; 1 when the sequences are known to be of equal length and
// two tiles per pair would not fit on the CUs at once (then throughput, not
// the longest chain, bounds the launch).
__host__ __device__ inline int recur_tiles(int64_t pairs, bool equal_lengths, int cus) {
  if (4 * pairs <= cus) return 4;
  if (2 * pairs <= cus || !equal_lengths) return 2;
  return 1;
}

// The library's path choice: estimated time (us) of each path on MI355X for H
// heads, `total` chunks over all sequences, the longest sequence's `maxc`
// chunks and N sequences (the scheduler kernel evaluates it for cu_seqlens;
// for B sequences of T tokens the host does).  The constants are a least-
// squares fit to kernel times measured on the box at K = V = 128 over 36
// batches of 8192 tokens (1 .. 128 sequences of 64 .. 8192 tokens, and 12
// ragged ones; H = 16, 32, 64, 96), with which the choice matches the faster
// path in all of them but one tie (1.6 %).  The model is empirical: each
// constant is what the fit gave, not a measured quantity on its own.
//   split: the prep kernel streams inputs and records at about 5.5 ns per
//     (chunk, head).  A recurrence workgroup costs about 13.4 us to start and
//     end (tables, state, the first chunk's latency) plus 0.37 / 0.56 / 1.0 us
//     per step with 32 / 64 / 128 columns; the recurrence is the longest chain
//     or, with more workgroups than CUs, throughput: two 64-column workgroups
//     share a CU, at 3.76 us of start per workgroup and 0.64 us per step and
//     tile of CU time, the chain then at 0.47 us per step;
//   fused: a workgroup step costs 1.75 us (64 columns, two workgroups per
//     pair) or 2.20 us (128 columns) of CU time, and the longest sequence's
//     chain 1.60 / 1.88 us per step; each sequence takes five pipeline steps
//     more than its chunk count plus 1.75 us, and the work spreads over the
//     CUs, one workgroup per CU.
__host__ __device__ inline double recur_estimate(int64_t H, int64_t N, int64_t total, int64_t maxc,
                                                 bool equal_lengths, int cus) {
  const double chunk_heads = (double)total * (double)H, pairs = (double)N * (double)H;
  const int tiles = recur_tiles(N * H, equal_lengths, cus);
  const double step = tiles == 4 ? 0.37 : tiles == 2 ? 0.56 : 1.0;
  const double chain = 13.4 + step * (double)maxc;
  if (tiles * pairs <= cus) return chain;
  if (tiles == 2) return fmax(13.4 + 0.47 * (double)maxc, 2.0 * (3.76 * pairs + 0.64 * chunk_heads) / cus);
  return fmax(chain, (13.4 * pairs + step * chunk_heads) / cus);
}

__host__ __device__ inline double fused_estimate(int64_t H, int64_t N, int64_t total, int64_t maxc, int cus) {
  const double chunk_heads = (double)total * (double)H, pairs = (double)N * (double)H;
  const bool two = fused_two_tiles(N * H, cus);
  const double step = two ? 1.75 : 2.20, chain_step = two ? 1.60 : 1.88;
  const double chain = 1.75 + chain_step * (double)(maxc + 5);
  return fmax(chain, (two ? 2.0 : 1.0) * (1.75 * pairs + step * (chunk_heads + 5.0 * pairs)) / cus);
}

__host__ __device__ inline int choose_path(int64_t H, int64_t N, int64_t total, int64_t maxc, bool equal_lengths,
                                           int cus) {
  const double split = 5.5e-3 * (double)total * (double)H + recur_estimate(H, N, total, maxc, equal_lengths, cus);
  return fused_estimate(H, N, total, maxc, cus) < split ? KDA_PATH_FUSED : KDA_PATH_SPLIT;
}


struct PrepArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* g;
  const uint16_t* beta;
  const float* A_log;
  const float* dt_bias;
  float scale;
  float lower_bound;
  int64_t H;
  int part;             // chunks part_first[part] .. part_first[part + 1] - 1
  int64_t grid_chunks;  // workgroup columns launched (a bound on the part's chunk count)
  char* ws;
  Layout lay;
  // > 0: fixed_B sequences of fixed_T tokens, one part, and no scheduler
  // kernel ran: chunk entries come from fixed_chunk, and the first workgroup
  // writes the header (status OK, path split, chunk count, part bounds)
  int64_t fixed_T = 0, fixed_B = 0;
  // KDA_PREC_NEUMANN_FP16 set: the precision study's form of the inverse
  int precision = 0;
};

struct RecurArgs {
  const uint16_t* v;
  uint16_t* out;
  const void* s_in;
  void* s_out;
  int state_dtype;      // KDA_DTYPE_*
  int64_t N, H;
  int part;             // chunks whose first token row lies in [row_lo, row_hi)
  int64_t row_lo, row_hi;
  char* ws;
  Layout lay;
  // sets == 2 (16-token chunks, one part): a second recurrence over the same
  // chunk records in the same launch, pairs N H .. 2 N H - 1, that computes
  // each pair's transition: zero values from the identity state, written as
  // fp16 to s_out2 in math layout [n][h][k][v] (the values are read from v
  // and ignored).  A NULL output pointer skips the outputs (always, for the
  // second set).
  int sets;
  uint16_t* s_out2;
  // Precision variant of the chunk step (KDA_PREC_*, 16-token chunks only);
  // 0 is the library's own arithmetic.
  int precision;
  // Value tiles per (sequence, head) for 16-token chunks: 1, 2 or 4 (128, 64
  // or 32 columns per workgroup), or 0 for recur_tiles(pairs, false, cus).
  int tiles;
  // > 0: N sequences of fixed_T tokens with no scheduler tables (the prep
  // kernel wrote the header): sequence entries from fixed_seq, order = index
  int64_t fixed_T = 0;
  // Polls after which a wait between the waves of a workgroup gives up (set
  // by the launch from spin_limit()).
  int spin_limit = 0;
  int cus = kCUs;       // compute units of the device (launch shape)
};

// Waits between the waves of a recurrence or fused workgroup give up after
// kSpinLimit polls, or after the count a test set with
// kda_debug_set_spin_limit (spin_limit() returns the one in force).
constexpr int kSpinLimit = 1 << 21;
int spin_limit();

// Fused chunk prep + recurrence (one kernel, records kept in LDS): the
// inputs and outputs of kda_fwd, the scheduler's tables in `ws`.
struct FusedArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* g;
  const uint16_t* beta;
  uint16_t* out;
  const float* A_log;
  const float* dt_bias;
  float scale;
  float lower_bound;
  const void* s_in;
  void* s_out;
  int state_dtype;      // KDA_DTYPE_* of whichever state is given
  int64_t N, H;
  char* ws;
  Layout lay;
  // Polls after which a wait between the waves of a workgroup gives up (set
  // by the launch from spin_limit()).
  int spin_limit = 0;
  int cus = kCUs;       // compute units of the device (launch shape)
};

// Segmented forward: segment boundaries and the prefix over the segments'
// affine state maps (kda_segment.hip).
struct SegArgs {
  const int64_t* cu;    // the caller's cu_seqlens (device) or nullptr (N rows of T tokens)
  int64_t N, T;
  int S;                // segments per sequence
  int64_t* seg_cu;      // written: N S + 1 boundaries
};

struct PrefixArgs {
  const uint16_t* A;    // [N S][H][K][K]: transition of each (segment, head), fp16, math layout A[k][m]
  const float* B;       // [N S][H][V][K]: end state from a zero start
  float* starts;        // written: [N S][H][V][K] start state of each segment
  const void* s_in;     // the caller's initial state [N][H][V][K] or nullptr
  void* s_out;          // the caller's final state or nullptr
  int state_dtype;      // KDA_DTYPE_* of the caller's states
  int64_t N, H;
  int S;
  const WsHeader* hdr;  // the forward's header: nothing is written unless its status is OK
  const int64_t* seg_cu;  // N S + 1 segment boundaries: an empty segment passes its state through
};

// Single-token step: token n of every sequence is row n of q, k, v, g, beta
// ([N][H][128], [N][H]) and of out.
struct DecodeArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* g;
  const uint16_t* beta;
  const float* A_log;
  const float* dt_bias;
  float scale;
  float lower_bound;
  const void* s_in;
  void* s_out;
  int state_dtype;      // KDA_DTYPE_* of whichever state is given
  uint16_t* out;
  int64_t N, H;
};

hipError_t launch_sched(const SchedArgs& a, hipStream_t s);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t s);
hipError_t launch_fused(const FusedArgs& a, hipStream_t s);
hipError_t launch_seg_cu(const SegArgs& a, hipStream_t s);
hipError_t launch_prefix(const PrefixArgs& a, hipStream_t s);
// The launchers pick the 16-, 32- or 64-token kernels by a.lay.chunk.
hipError_t launch_prep(const PrepArgs& a, hipStream_t s);
hipError_t launch_recur(const RecurArgs& a, hipStream_t s);
hipError_t launch_prep32(const PrepArgs& a, hipStream_t s);
hipError_t launch_recur32(const RecurArgs& a, hipStream_t s);
hipError_t launch_prep64(const PrepArgs& a, hipStream_t s);
hipError_t launch_recur64(const RecurArgs& a, hipStream_t s);

}  // namespace kda
