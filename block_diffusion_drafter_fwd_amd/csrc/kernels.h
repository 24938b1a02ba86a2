// Argument blocks and launchers of the gfx950 kernels of the drafter forward.
// Every kernel takes its arguments by value; per-call tables (sequence and row
// descriptors) live in the caller's workspace and are written there by the
// upload kernel, so no launch needs a host round trip.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace dflash {
namespace kern {

constexpr int kMaxSeg = 32;        // column segments of one GEMM launch
constexpr int kMaxOut = 16;        // outputs of one norm launch
constexpr int kMaxL = 16;          // layers of one head-finish launch
constexpr int kUploadWords = 960;  // 3840-byte payload of one upload launch (kernel arguments: 4 KiB)
constexpr int kHistRing = 512;     // slots of a session's committed-token ring (penalty history)

// One sequence (session) of a batched call.
struct SeqDesc {
    void* cache;          // arena base, [L][2][Hkv][cap][D] of the config dtype
    int32_t* hist;        // committed-token ring (sampler)
    uint64_t seed, stream;
    int32_t cap, ring;    // slots; ring != 0: slot = position mod cap
    int32_t F, M;         // block anchor position, block rows
    int32_t q_row0;       // first block row of this sequence
    int32_t out_row0;     // first logits row (block rows minus anchors before it)
    int32_t key_lo;       // first key position visible to the block
    int32_t item0, nitems;// attention work items
    int32_t current;      // anchor token
    int32_t hist_n, hist_head;
};
static_assert(sizeof(SeqDesc) == 80, "SeqDesc layout");

struct RowInfo {
    int32_t seq;          // index into the SeqDesc table
    int32_t pos;          // absolute position (context/block) or row index (sampler)
};

// C[:, c_col0 : c_col0+N] (+)= A[M, K] . B[N, K]^T, one entry per segment.
struct GemmSeg {
    const void* A;
    const void* B;
    int32_t lda, ldb, N, c_col0, tile0, pad;
};

// epilogues: C = acc, C += acc, out = silu(acc of segment 0) * (acc of
// segment 1) for the paired gate|up projection, or kPartial: K is split over
// workgroups and split s writes its share to C + s * M * ldc (at most
// max_splits slices); the consumer of C adds the slices
enum GemmMode { kStore = 0, kAccumulate = 1, kSwiGLU = 2, kPartial = 3 };

struct GemmHead {
    int32_t M, K, kc, splits;
    float* C;
    int32_t ldc, accumulate;
    int32_t mode, ldo;
    void* out;                // kSwiGLU output [M, ldo]
    int32_t out_bf16, max_splits;
    const int32_t* a_rows;    // optional: A row of output row m (all segments)
    float* part;              // split-K partials [splits][M][ldc]
    int32_t nseg, ntiles;
    int32_t col_lo, col_hi;   // columns covered by the segments
    int32_t xcd_remap, pad;   // tiled kernels: gather the items that share A onto one XCD
};

// The argument block is copied to the device at every launch and its cache
// lines are fetched by every workgroup at start-up, so launches with few
// segments use a short form (the launcher converts).
template <int NS>
struct GemmArgsT : GemmHead {
    GemmSeg seg[NS];
};
constexpr int kFewSeg = 4;
using GemmArgs = GemmArgsT<kMaxSeg>;

// y = RMSNorm(x) * gain with x = in[row] (optional) + sum of nsplit fp32
// slices part[s * part_stride + row * in_stride]; x is written back to
// `writeback` when given (fused residual add).  Rows are at most kNormMaxW wide.
constexpr int kNormMaxW = 8192;
struct NormArgs {
    const void* in;
    int64_t in_stride;        // elements between rows (of in, part and writeback)
    const int32_t* row_src;   // optional: input row of each output row
    const float* part;
    int64_t part_stride;
    float* writeback;
    int32_t nsplit, pad;
    int32_t in_bf16, rows, width, groups;
    float eps;
    int32_t gain_bf16, nout, out_bf16;
    int64_t gain_group_stride;
    int64_t out_stride;
    const void* gain[kMaxOut];
    void* out[kMaxOut];
};

struct HeadArgs {
    const float* src;         // projection output rows: nsplit slices of src_stride floats, summed
    const RowInfo* rows;
    const SeqDesc* seqs;
    void* q_out;              // [rows][Hq][D]
    const void* q_norm;
    const void* k_norm[kMaxL];
    int32_t ld, nrows, D, Hq, Hkv, L;
    int32_t q_col;            // -1: no q heads in this launch
    int32_t k_col[kMaxL], v_col[kMaxL], layer[kMaxL];
    int32_t qk_norm, w_bf16, cache_bf16, q_bf16;
    int32_t nsplit, pad;
    int64_t src_stride;
    float eps;
    // rows == nullptr: one run of rows, row r at position pos0 + r of the
    // session whose cache, slot count and ring mode follow (no tables)
    int32_t pos0;
    void* cache0;
    int32_t cap0, ring0;
    double inv_freq[64];      // theta^(-2d/D), d < D/2, computed on the host in fp64
};

// h[row] = table[token of row]; when `gain` is set, also out[row] =
// RMSNorm(h[row]) * gain (the first layer's input norm), out_bf16 typed
struct EmbedArgs {
    const void* table;
    float* h;
    const RowInfo* rows;      // nullptr: one block, row 0 the anchor `current`, the rest mask tokens
    const SeqDesc* seqs;
    int32_t H, nrows, mask_id, w_bf16;
    const void* gain;
    void* out;
    float eps;
    int32_t out_bf16;
    int32_t vec4;             // set by the launcher: rows read four elements at a time
    int32_t current;
};

struct AttnArgs {
    const void* Q;            // [rows][Hq][D]
    const SeqDesc* seqs;
    const RowInfo* rows;
    float* part_o;            // [items][Hkv][64][D]
    float* part_ml;           // [items][Hkv][64][2]
    const float* gate_src;    // projection rows holding the g columns (gate_nsplit slices, summed)
    const uint32_t* order;    // [total_items]: (sequence << 16 | item), largest chunks first
    void* out;                // [rows][Hq*D]
    int32_t nseq, nrows, layer, L, Hq, Hkv, D, causal, window, chunk, total_items;
    int32_t gate, gate_ld, gate_col, out_bf16;
    int32_t gate_nsplit;
    int32_t strided;          // item c of a sequence takes its tiles c, c + nitems, ... (else one run of chunk keys)
    int64_t gate_stride;
    float scale;
    int32_t pad2;
    SeqDesc seq0;             // rows == nullptr: one session, block row r at position seq0.F + r, items in order
};

struct SampleArgs {
    const float* logits;
    const SeqDesc* seqs;
    const RowInfo* rows;      // seq, row within the session's block
    uint32_t* bitmap;         // [nseq][words]
    float* stats;             // [R][nchunk][4]
    int32_t* ids;
    float* probs;
    int32_t V, R, nseq, words, chunk, nchunk, round, use_penalty;
    float temperature, rho;
    SeqDesc seq0;             // rows == nullptr: one session, row r is its row r
};

// Speculative verification of drafted blocks: session k drafted
// offs[k+1] - offs[k] tokens and has that many + 1 target rows, from target
// row offs[k] + k on.
struct VerifyArgs {
    const float* target;      // [Rt][V] target logits
    const int32_t* draft_ids; // [Rd]
    const float* draft_probs; // [Rd][V] (temperature > 0)
    const SeqDesc* seqs;      // seed, stream
    const RowInfo* rows;      // per target row: session, row within its block
    const int32_t* offs;      // [nseq + 1]
    float* stats;             // [Rt][nchunk][4]: max / sum-exp of row / T, argmax
    float* stats2;            // [Rt][nchunk][4]: best Gumbel key of the next-token draw
    int32_t* accepted;        // [nseq]
    int32_t* next;            // [nseq]
    int32_t V, Rt, nseq, chunk, nchunk, round;
    float temperature;
    int32_t n0;               // rows == nullptr: one session with n0 drafts,
    SeqDesc seq0;             // its descriptor (no tables)
};

// DFlash2 candidate selector: per (row, 4096-token chunk) the chunk's top-K,
// then per session a walk over its rows in order (merge to the row's top-K,
// bigram scores against the previous choice, softmax / Gumbel-max).
constexpr int kSelMaxK = 16;            // candidates per row, at most
constexpr int kSelMaxEntries = 1024;    // chunk candidates merged per row (nchunk * K), at most
constexpr int kSelMaxDs = 256;          // selector table width, at most
// per row, written by the preparation pass and read by the walk: the row's
// candidate ids (int bits) and logits by rank, then the bigram terms
// <P[p], Q[c]> for candidate rank p of the row before (the anchor: p = 0)
// and rank c of this row, p-major
constexpr int kSelPrepStride = 2 * kSelMaxK + kSelMaxK * kSelMaxK;
struct SelectArgs {
    const float* logits;      // [R][V]
    const void* P;            // [V][Ds] predecessor table (bf16 or fp32)
    const void* Q;            // [V][Ds] candidate table
    const SeqDesc* seqs;      // [nseq]: seed, stream (null with offs and anchors: one session, seq0)
    const int32_t* offs;      // [nseq + 1] row offsets
    const int32_t* anchors;   // [nseq]
    float* cand;              // [R][nchunk][kSelMaxK][2]: chunk top-K (value, id bits)
    int32_t* tokens;          // [R]
    int32_t* cand_ids;        // [R][K]
    float* cand_probs;        // [R][K] or null
    float* dense;             // [R][V] or null: zeroed, then the candidates' probabilities
    float* prep;              // [R][kSelPrepStride]
    int32_t V, R, nseq, K, Ds, chunk, nchunk, round, w_bf16, pad;
    float temperature;
    SeqDesc seq0;             // one session (seqs null): rows 0..R-1, anchor seq0.current
};

struct UploadArgs {
    uint32_t* dst;
    int32_t nwords, pad;
    uint32_t data[kUploadWords];
};

// history tokens (payload in the kernel arguments) + a 16-byte-aligned copy
constexpr int kCommitTokens = 256;
struct CommitArgs {
    int32_t* hist;
    const uint4* src;
    uint4* dst;
    int64_t n16;              // 16-byte units to copy
    int32_t count, pad;
    int32_t tokens[kCommitTokens];
};

// Commits of several sessions in one launch: item i writes its tokens
// tokens[tok0 .. tok0+count) to hist[(slot0 + j) mod kHistRing] and copies n16
// 16-byte units from src to dst.  Everything rides in the kernel arguments.
constexpr int kCommitItems = 32, kCommitBatchTokens = 512;
struct CommitItemArgs {
    int32_t* hist;
    const uint4* src;
    uint4* dst;
    int64_t n16;
    int32_t slot0, tok0, count, pad;
};
struct CommitBatchArgs {
    int32_t n, pad;
    CommitItemArgs item[kCommitItems];
    int32_t tokens[kCommitBatchTokens];
};

// launchers (return hipError_t of the launch)
// tag 1 launches a separate instantiation (the unembedding) so that profilers
// can tell it apart from the per-layer GEMMs
// splits_out (optional) receives the number of K slices written in kPartial mode
hipError_t gemm(GemmArgs a, bool bf16, size_t part_cap_floats, int num_cus, hipStream_t st, int tag = 0,
                int* splits_out = nullptr);
hipError_t rmsnorm(const NormArgs& a, hipStream_t st);
hipError_t commit_batch(const CommitBatchArgs& a, hipStream_t st);
hipError_t head_finish(const HeadArgs& a, int nlayer, hipStream_t st);
hipError_t embed(const EmbedArgs& a, hipStream_t st);
// part: 0 both launches, 1 the partials only, 2 the combine only (bf16 path)
hipError_t attention(const AttnArgs& a, bool bf16, hipStream_t st, int part = 0);
hipError_t sample(const SampleArgs& a, hipStream_t st);
hipError_t verify(const VerifyArgs& a, hipStream_t st);
hipError_t select(const SelectArgs& a, hipStream_t st);
hipError_t gather_rows(void* dst, const uint64_t* src_ptrs, int32_t rows, size_t row_bytes, hipStream_t st);
hipError_t upload(void* dst, const void* host, size_t bytes, hipStream_t st);
// count <= kCommitTokens tokens to hist, then bytes from src to dst; returns
// hipErrorInvalidValue (nothing launched) when bytes or a pointer is not
// 16-byte aligned
hipError_t commit_rows(int32_t* hist, const int32_t* tokens, int32_t count, void* dst, const void* src, size_t bytes,
                       hipStream_t st);
hipError_t cache_read(const void* cache, int32_t cap, int32_t ring, int32_t Hkv, int32_t D, int32_t layer,
                      int32_t pos0, int32_t count, int32_t bf16, float* k_out, float* v_out, hipStream_t st);

}  // namespace kern
}  // namespace dflash
