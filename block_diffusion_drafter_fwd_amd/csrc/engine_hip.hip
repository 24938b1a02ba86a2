// HIP backend of the drafter: plans and enqueues the kernels of the context
// pass, the block pass and the sampler.  All device memory is the caller's:
// the per-call tables and every intermediate live in the workspace whose
// layout is computed here.
//
// Context pass (rows of one or more sessions):
//   [aux tap norms] -> fc GEMM (K slices) -> hidden_norm (sums the slices)
//   -> [per-layer input_layernorm] -> every layer's k|v in one GEMM (K slices)
//   -> head_finish (sums slices; k-norm, RoPE, slot write of K and V)
// Block pass (anchor + n mask rows per sequence):
//   embed -> norm -> per layer: QKV(+g) GEMM (slices) -> head_finish (q to the
//   query buffer, block K/V to the cache) -> attention partials -> combine
//   (+ gate) -> o_proj (slices) -> residual add + post norm -> gate|up GEMM
//   with SwiGLU epilogue -> down_proj (slices) -> residual add + next norm
//   (the final norm after the last layer) -> unembedding of rows 1..n.
// Splitting K over workgroups lets the small-N weight-streaming GEMMs use all
// CUs; the slices are added by whichever kernel reads the result next, so no
// reduction pass is launched.
#include <algorithm>
#include <functional>
#include <mutex>
#include <queue>
#include <cmath>
#include <cstring>
#include <string>
#include <vector>

#include "engine.h"
#include "kernels.h"

namespace dflash {

// the static scratch array of dflash_verify_noalloc (4 MiB per GPU); see
// scratch_address below for how host code obtains its device address
static __device__ __align__(256) char scratch[size_t(4) << 20];

namespace {

using namespace kern;

size_t al(size_t x) { return (x + 255) & ~size_t(255); }

static_assert(kHistory == kHistRing, "the kernels index the history ring with kHistRing slots");

// Device memory for the calls that take no workspace (dflash_verify_noalloc):
// one array per GPU for the process's lifetime.  Host code never passes the
// array's name to a kernel (on the host it is a stand-in, not a device
// address): each device's address comes from hipGetSymbolAddress, resolved
// once per device with that device current, and only that pointer is used.
constexpr size_t kScratchBytes = sizeof(scratch);

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// the current device's scratch address (resolved on the first call per device)
hipError_t scratch_address(int dev, void** out) {
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

constexpr int kSampleChunk = 4096;
constexpr int kAttnMinChunk = 64;                    // keys per attention work item, at least (one tile)
constexpr int kAttnShortChunk = 256;                 // below: one attention workgroup per CU
constexpr int kAttnRoundChunk = 4096;                // longest chunk worth a single resident round
constexpr int kAttnManyLo = 1024, kAttnManyHi = 4096;  // chunk range when the split runs in several rounds
constexpr int kAttnItemStartTiles = 6;               // an item's start-up, in 64-key tiles (measured fit)
constexpr size_t kPartCapFloats = size_t(8) << 20;   // tiled split-K partials: 32 MiB
constexpr int kMaxSlicesFc = 8;                      // K slices of the fc GEMM
constexpr int kMaxSlicesKv = 4;                      // K slices of the context k|v GEMM

// The context-path buffers come twice (lane 0 and lane 1): the passes of one
// call alternate between the session's stream and a second one, which run
// them at the same time.
struct CtxBufs {
    size_t tables, stage, fc, c, x, kv;
};
struct WsLayout {
    size_t tables;
    size_t ctx_stage, ctx_fc, ctx_c, ctx_x, ctx_kv;
    CtxBufs lane1;
    size_t blk_h, blk_x, blk_qkv, blk_q, blk_attn, blk_part, blk_mlp, blk_act;
    size_t attn_o, attn_ml, part, bitmap, stats, stats2, sel, sel_prep;
    size_t total;
    int32_t r_ctx, r_blk, items_cap, nchunk_max, blk_slices;
};

#define HIP_OK(expr)                                                                    \
    do {                                                                                \
        hipError_t e_ = (expr);                                                         \
        if (e_ != hipSuccess) return fail(DFLASH_E_HIP, std::string(#expr) + ": " +     \
                                                         hipGetErrorString(e_));        \
    } while (0)

class HipEngine : public Engine {
public:
    HipEngine(const Model& m, int num_cus, void* scratch) : m_(m), cus_(num_cus), scratch_(scratch) {}

    WsLayout layout(int32_t ms) const {
        const dflash_config& c = m_.cfg;
        WsLayout w{};
        const size_t act = m_.elem;
        w.r_blk = ms * c.block_size;
        w.r_ctx = std::max(c.flush_rows, w.r_blk);
        // K slices of the block path's split GEMMs, at most four: every
        // slice is read again by the norm or head finish that follows, and
        // with eight the o_proj / down norms of a 4096-wide model cost more
        // than the wider splits saved (long 679 -> 689 blocks/s, qwen 1867
        // -> 1873 at four; at two qwen's 2048-deep GEMMs leave CUs idle, 1781)
        w.blk_slices = std::max(1, std::min(4, 4096 / w.r_blk));
        const int32_t rmax = std::max(w.r_ctx, w.r_blk);
        const int32_t L = c.layers, H = c.hidden, I = c.intermediate;
        w.items_cap = 4 * std::max(1, attn_target_wg() / c.kv_heads) + ms;
        w.nchunk_max = (c.vocab + kSampleChunk - 1) / kSampleChunk;
        size_t o = 0;
        auto put = [&](size_t bytes) { size_t at = o; o += al(bytes); return at; };
        w.tables = put(sizeof(SeqDesc) * (size_t)ms + sizeof(RowInfo) * (size_t)rmax +
                       sizeof(int32_t) * (size_t)w.r_blk + sizeof(uint64_t) * (size_t)w.r_ctx +
                       sizeof(uint32_t) * (size_t)w.items_cap + 128);
        w.ctx_stage = put(act * (size_t)w.r_ctx * m_.fc_in);
        w.ctx_fc = put(4 * (size_t)kMaxSlicesFc * w.r_ctx * H);
        w.ctx_c = put(4 * (size_t)w.r_ctx * H);
        w.ctx_x = put(act * (size_t)(c.ctx_input_norm ? L : 1) * w.r_ctx * H);
        w.ctx_kv = put(4 * (size_t)kMaxSlicesKv * w.r_ctx * L * 2 * m_.kd);
        w.lane1.tables = put(sizeof(SeqDesc) * (size_t)ms + sizeof(RowInfo) * (size_t)w.r_ctx +
                             sizeof(uint64_t) * (size_t)w.r_ctx + 128);
        w.lane1.stage = put(act * (size_t)w.r_ctx * m_.fc_in);
        w.lane1.fc = put(4 * (size_t)kMaxSlicesFc * w.r_ctx * H);
        w.lane1.c = put(4 * (size_t)w.r_ctx * H);
        w.lane1.x = put(act * (size_t)(c.ctx_input_norm ? L : 1) * w.r_ctx * H);
        w.lane1.kv = put(4 * (size_t)kMaxSlicesKv * w.r_ctx * L * 2 * m_.kd);
        w.blk_h = put(4 * (size_t)w.r_blk * H);
        w.blk_x = put(act * (size_t)w.r_blk * H);
        w.blk_qkv = put(4 * (size_t)w.blk_slices * w.r_blk * qkv_ld());
        w.blk_q = put(act * (size_t)w.r_blk * m_.qd);
        w.blk_attn = put(act * (size_t)w.r_blk * m_.qd);
        w.blk_part = put(4 * (size_t)w.blk_slices * w.r_blk * H);
        w.blk_mlp = put(4 * (size_t)w.r_blk * 2 * I);
        w.blk_act = put(act * (size_t)w.r_blk * I);
        const bool bf16 = c.dtype == DFLASH_BF16;
        w.attn_o = put(bf16 ? 4 * (size_t)w.items_cap * c.kv_heads * 64 * c.head_dim : 0);
        w.attn_ml = put(bf16 ? 4 * (size_t)w.items_cap * c.kv_heads * 64 * 2 : 0);
        w.part = put(bf16 ? 4 * kPartCapFloats : 0);
        w.bitmap = put(4 * (size_t)ms * ((c.vocab + 31) / 32));
        w.stats = put(16 * (size_t)w.r_blk * w.nchunk_max);
        w.stats2 = put(16 * (size_t)w.r_blk * w.nchunk_max);   // verification's second pass
        w.sel = put(c.sel_candidates ? 8 * (size_t)kSelMaxK * w.r_blk * w.nchunk_max : 0);
        w.sel_prep = put(c.sel_candidates ? 4 * (size_t)kSelPrepStride * w.r_blk : 0);
        w.total = o;
        return w;
    }

    // attention work items per call: two workgroups per CU over all kv heads,
    // the number that are resident together (64 KiB of LDS each), so the
    // whole split runs as one round
    int32_t attn_target_wg() const { return 2 * cus_; }

    int32_t qkv_ld() const { return m_.qd + 2 * m_.kd + (m_.cfg.gate ? m_.cfg.q_heads : 0); }

    size_t workspace_bytes(int32_t ms) const override { return layout(ms).total; }

    int copy_rows(void* dst, const void* src, size_t bytes, void* stream) override {
        if (!bytes) return 0;
        HIP_OK(hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToDevice, (hipStream_t)stream));
        return 0;
    }

    int write_history(const SessView& s, int32_t slot0, const int32_t* tokens, int32_t count,
                      void* stream) override {
        HIP_OK(upload(s.hist + slot0, tokens, sizeof(int32_t) * (size_t)count, (hipStream_t)stream));
        return 0;
    }

    int commit_rows(const SessView& s, int32_t slot0, const int32_t* tokens, int32_t count, void* dst,
                    const void* src, size_t bytes, void* stream) override {
        if (count <= kCommitTokens && bytes % 16 == 0 && ((uintptr_t)src & 15) == 0 && ((uintptr_t)dst & 15) == 0) {
            HIP_OK(kern::commit_rows(s.hist + slot0, tokens, count, dst, src, bytes, (hipStream_t)stream));
            return 0;
        }
        return Engine::commit_rows(s, slot0, tokens, count, dst, src, bytes, stream);
    }

    // every session's history tokens and feature rows from the kernel
    // arguments of one launch per kCommitItems sessions / kCommitBatchTokens
    // tokens; an item that does not fit a launch's rules goes alone
    int commit_many(const std::vector<CommitItem>& items, void* stream) override {
        CommitBatchArgs a{};
        int32_t ntok = 0;
        auto launch = [&]() -> int {
            if (a.n) HIP_OK(kern::commit_batch(a, (hipStream_t)stream));
            a.n = 0;
            ntok = 0;
            return 0;
        };
        for (const CommitItem& c : items) {
            const bool fits = c.count <= kCommitBatchTokens && c.bytes % 16 == 0 &&
                              ((uintptr_t)c.src & 15) == 0 && ((uintptr_t)c.dst & 15) == 0;
            if (!fits) {
                if (int rc = Engine::commit_many({c}, stream)) return rc;
                continue;
            }
            if (a.n == kCommitItems || ntok + c.count > kCommitBatchTokens)
                if (int rc = launch()) return rc;
            CommitItemArgs& it = a.item[a.n++];
            it.hist = c.hist;
            it.src = (const uint4*)c.src;
            it.dst = (uint4*)c.dst;
            it.n16 = (int64_t)(c.bytes / 16);
            it.slot0 = c.slot0;
            it.tok0 = ntok;
            it.count = c.count;
            for (int32_t j = 0; j < c.count; ++j) a.tokens[ntok + j] = c.tokens[j];
            ntok += c.count;
        }
        return launch();
    }

    int ctx_forward(const std::vector<SessView>& sess, const std::vector<CtxSeg>& segs, void* ws,
                    int32_t ws_sessions, void* stream, int lane) override;

    struct Aux {
        hipStream_t st = nullptr;
        hipEvent_t fork = nullptr, join = nullptr;
    };
    int aux_open(void** out) override {
        *out = nullptr;
        Aux* a = new Aux;
        // default priority (a stream of another priority is not used here)
        if (hipStreamCreateWithFlags(&a->st, hipStreamNonBlocking) != hipSuccess ||
            hipEventCreateWithFlags(&a->fork, hipEventDisableTiming) != hipSuccess ||
            hipEventCreateWithFlags(&a->join, hipEventDisableTiming) != hipSuccess) {
            aux_close(a);
            return fail(DFLASH_E_HIP, "second stream of the session could not be created");
        }
        *out = a;
        return 0;
    }
    void aux_close(void* p) override {
        Aux* a = (Aux*)p;
        if (!a) return;
        if (a->st) {
            (void)hipStreamSynchronize(a->st);
            (void)hipStreamDestroy(a->st);
        }
        if (a->fork) (void)hipEventDestroy(a->fork);
        if (a->join) (void)hipEventDestroy(a->join);
        delete a;
    }
    void* aux_stream(void* p) override { return p ? (void*)((Aux*)p)->st : nullptr; }
    int aux_fork(void* p, void* stream) override {
        Aux* a = (Aux*)p;
        HIP_OK(hipEventRecord(a->fork, (hipStream_t)stream));
        HIP_OK(hipStreamWaitEvent(a->st, a->fork, 0));
        return 0;
    }
    int aux_join(void* p, void* stream) override {
        Aux* a = (Aux*)p;
        HIP_OK(hipEventRecord(a->join, a->st));
        HIP_OK(hipStreamWaitEvent((hipStream_t)stream, a->join, 0));
        return 0;
    }
    int block_forward(const std::vector<SessView>& sess, const std::vector<BlockSeq>& seqs, float* logits,
                      float* hidden, void* ws, int32_t ws_sessions, void* stream) override;
    int sample(const std::vector<SessView>& sess, const int32_t* row_offsets, const float* logits,
               const dflash_sample_params& p, int32_t* ids, float* probs, void* ws, int32_t ws_sessions,
               void* stream) override;

    int verify(const std::vector<SessView>& sess, const int32_t* draft_offsets, const float* target,
               const int32_t* draft_ids, const float* draft_probs, const dflash_verify_params& p, int32_t* accepted,
               int32_t* next, void* ws, int32_t ws_sessions, void* stream) override;
    int verify_scratch(const std::vector<SessView>& sess, const int32_t* draft_offsets, const float* target,
                       const int32_t* draft_ids, const float* draft_probs, const dflash_verify_params& p,
                       int32_t* accepted, int32_t* next, void* stream) override;
    int select(const std::vector<SessView>& sess, const int32_t* row_offsets, const float* logits,
               const int32_t* current, const dflash_select_params& p, int32_t* tokens, int32_t* cand_ids,
               float* cand_probs, float* dense, void* ws, int32_t ws_sessions, void* stream) override;

    int cache_read(const SessView& s, int32_t layer, int32_t pos0, int32_t count, float* k_out, float* v_out,
                   void* stream) override {
        const dflash_config& c = m_.cfg;
        HIP_OK(kern::cache_read(s.cache, s.cap, s.ring, c.kv_heads, c.head_dim, layer, pos0, count,
                                c.dtype == DFLASH_BF16, k_out, v_out, (hipStream_t)stream));
        return 0;
    }

    int profile_begin(const std::string& stage) override {
        stage_ = stage;
        ev_used_ = 0;
        return 0;
    }

    int profile_end(double* total_ms, int32_t* launches) override {
        *total_ms = 0.0;
        *launches = (int32_t)(ev_used_ / 2);
        stage_.clear();
        if (ev_used_ >= 2) HIP_OK(hipEventSynchronize(ev_[ev_used_ - 1]));
        for (size_t i = 0; i + 1 < ev_used_; i += 2) {
            float ms = 0.f;
            HIP_OK(hipEventElapsedTime(&ms, ev_[i], ev_[i + 1]));
            *total_ms += ms;
        }
        ev_used_ = 0;
        return 0;
    }

    ~HipEngine() override {
        for (hipEvent_t e : ev_) (void)hipEventDestroy(e);
    }

private:
    int verify_in(const std::vector<SessView>& sess, const int32_t* draft_offsets, const float* target,
                  const int32_t* draft_ids, const float* draft_probs, const dflash_verify_params& p, int32_t* accepted,
                  int32_t* next, char* tab, float* stats, float* stats2, void* stream);
    size_t verify_scratch_bytes(int32_t count, int32_t Rt) const;
    size_t verify_table_bytes(int32_t count, int32_t Rt) const;

    // Brackets the launches of one stage with events while that stage is profiled.
    struct Timed {
        HipEngine* e;
        hipStream_t st;
        bool on;
        Timed(HipEngine* eng, const char* stage, hipStream_t s) : e(eng), st(s), on(eng->stage_ == stage) {
            if (on) e->record(st);
        }
        ~Timed() {
            if (on) e->record(st);
        }
    };
    void record(hipStream_t st) {
        if (ev_used_ == ev_.size()) {
            hipEvent_t ev;
            if (hipEventCreate(&ev) != hipSuccess) return;
            ev_.push_back(ev);
        }
        (void)hipEventRecord(ev_[ev_used_++], st);
    }

    bool bf16() const { return m_.cfg.dtype == DFLASH_BF16; }

    NormArgs norm_args(const void* in, int in_bf16, int64_t in_stride, int rows, int width) const {
        NormArgs n{};
        n.in = in;
        n.in_bf16 = in_bf16;
        n.in_stride = in_stride;
        n.rows = rows;
        n.width = width;
        n.groups = 1;
        n.eps = m_.cfg.rms_eps;
        n.gain_bf16 = bf16();
        n.out_bf16 = bf16();
        n.out_stride = width;
        return n;
    }

    GemmArgs gemm_args(int32_t M, int32_t K, float* C, int32_t ldc, GemmMode mode, float* part,
                       int32_t max_slices) const {
        GemmArgs g{};
        g.M = M;
        g.K = K;
        g.C = C;
        g.ldc = ldc;
        g.mode = mode;
        g.part = part;
        g.max_splits = max_slices;
        return g;
    }

    // Per-call tables, packed and written by one upload (a few for long tables).
    struct Tables {
        std::vector<uint8_t> blob;
        size_t add(const void* p, size_t n) {
            const size_t off = (blob.size() + 15) & ~size_t(15);
            blob.resize(off + n);
            if (n) std::memcpy(blob.data() + off, p, n);
            return off;
        }
    };

    void fill_inv_freq(HeadArgs& h) const {
        const dflash_config& c = m_.cfg;
        for (int d = 0; d < c.head_dim / 2 && d < 64; ++d)
            h.inv_freq[d] = std::pow((double)c.rope_theta, -2.0 * d / (double)c.head_dim);
    }

    SeqDesc desc_of(const SessView& s) const {
        SeqDesc d{};
        d.cache = s.cache;
        d.hist = s.hist;
        d.seed = s.seed;
        d.stream = s.stream_id;
        d.cap = s.cap;
        d.ring = s.ring;
        return d;
    }

    Model m_;
    int cus_;
    void* scratch_ = nullptr;    // this device's static scratch array (device address)
    std::string stage_;
    std::vector<hipEvent_t> ev_;
    size_t ev_used_ = 0;
};

int HipEngine::ctx_forward(const std::vector<SessView>& sess, const std::vector<CtxSeg>& segs, void* ws,
                           int32_t ws_sessions, void* stream, int lane) {
    const dflash_config& c = m_.cfg;
    const WsLayout w = layout(ws_sessions);
    const CtxBufs b = lane ? w.lane1 : CtxBufs{w.tables, w.ctx_stage, w.ctx_fc, w.ctx_c, w.ctx_x, w.ctx_kv};
    hipStream_t st = (hipStream_t)stream;
    char* base = (char*)ws;
    const int32_t H = c.hidden, L = c.layers, kd = m_.kd;
    const size_t rb = (size_t)m_.fc_in * m_.elem;
    float* part = (float*)(base + w.part);
    size_t si = 0;
    while (si < segs.size()) {
        // a group of whole segments with at most r_ctx rows
        size_t sj = si;
        int32_t rows = 0;
        while (sj < segs.size() && rows + segs[sj].nrows <= w.r_ctx) rows += segs[sj++].nrows;
        if (sj == si) return fail(DFLASH_E_CAPACITY, "context segment larger than the workspace");
        std::vector<SeqDesc> descs;
        std::vector<RowInfo> info;
        std::vector<uint64_t> srcs;
        std::vector<int32_t> map(sess.size(), -1);
        for (size_t k = si; k < sj; ++k) {
            const CtxSeg& g = segs[k];
            if (map[g.sess] < 0) {
                map[g.sess] = (int32_t)descs.size();
                descs.push_back(desc_of(sess[g.sess]));
            }
            for (int32_t r = 0; r < g.nrows; ++r) {
                info.push_back({map[g.sess], g.pos0 + r});
                srcs.push_back((uint64_t)((const char*)g.rows + (size_t)r * rb));
            }
        }
        // one segment (a session's flush): its rows' positions and cache go
        // to the head finish in the kernel arguments, and no table is uploaded
        const bool one = sj - si == 1;
        char* tab = base + b.tables;
        const SeqDesc* d_desc = nullptr;
        const RowInfo* d_info = nullptr;
        size_t o_src = 0;
        if (!one) {
            Tables tb;
            const size_t o_desc = tb.add(descs.data(), sizeof(SeqDesc) * descs.size());
            const size_t o_info = tb.add(info.data(), sizeof(RowInfo) * info.size());
            o_src = tb.add(srcs.data(), sizeof(uint64_t) * srcs.size());
            HIP_OK(upload(tab, tb.blob.data(), tb.blob.size(), st));
            d_desc = (const SeqDesc*)(tab + o_desc);
            d_info = (const RowInfo*)(tab + o_info);
        }

        // A operand of fc: the segment rows themselves, or gathered / aux-normed
        const void* A = segs[si].rows;
        if (sj - si > 1) {
            HIP_OK(gather_rows(base + b.stage, (const uint64_t*)(tab + o_src), rows, rb, st));
            A = base + b.stage;
        }
        if (c.aux_norms) {
            NormArgs n = norm_args(A, bf16(), m_.fc_in, rows, m_.fc_in);
            n.groups = c.taps;
            n.gain_group_stride = c.target_hidden;
            n.nout = 1;
            n.gain[0] = m_.aux_norms;
            n.out[0] = base + b.stage;
            n.out_stride = m_.fc_in;
            HIP_OK(rmsnorm(n, st));
            A = base + b.stage;
        }
        float* fc_out = (float*)(base + b.fc);
        int fc_slices = 1;
        {
            GemmArgs g = gemm_args(rows, m_.fc_in, fc_out, H, kPartial, part, kMaxSlicesFc);
            g.nseg = 1;
            g.seg[0] = GemmSeg{A, m_.fc, m_.fc_in, m_.fc_in, H, 0, 0, 0};
            Timed tm(this, "flush_fc", st);
            HIP_OK(gemm(g, bf16(), kPartCapFloats, cus_, st, 0, &fc_slices));
        }
        // hidden_norm over the summed slices, then (Laguna) every layer's input_layernorm
        char* xs = base + b.x;
        const size_t xstride = m_.elem * (size_t)w.r_ctx * H;
        {
            NormArgs n = norm_args(nullptr, 0, H, rows, H);
            n.part = fc_out;
            n.nsplit = fc_slices;
            n.part_stride = (int64_t)rows * H;
            n.nout = 1;
            n.gain[0] = m_.hidden_norm;
            if (c.ctx_input_norm) {
                n.out[0] = base + b.c;
                n.out_bf16 = 0;
            } else {
                n.out[0] = xs;
            }
            HIP_OK(rmsnorm(n, st));
        }
        if (c.ctx_input_norm) {
            for (int32_t l0 = 0; l0 < L; l0 += kMaxOut) {
                NormArgs n2 = norm_args(base + b.c, 0, H, rows, H);
                n2.nout = std::min(kMaxOut, L - l0);
                for (int32_t j = 0; j < n2.nout; ++j) {
                    n2.gain[j] = m_.layer[l0 + j].in_ln;
                    n2.out[j] = xs + (size_t)(l0 + j) * xstride;
                }
                HIP_OK(rmsnorm(n2, st));
            }
        }
        // every layer's K|V in one GEMM (up to 16 layers per launch)
        const int32_t ldkv = L * 2 * kd;
        float* kv_out = (float*)(base + b.kv);
        for (int32_t l0 = 0; l0 < L; l0 += kMaxSeg / 2) {
            const int32_t nl = std::min<int32_t>(kMaxSeg / 2, L - l0);
            GemmArgs g = gemm_args(rows, H, kv_out, ldkv, kPartial, part, kMaxSlicesKv);
            g.nseg = 2 * nl;
            for (int32_t j = 0; j < nl; ++j) {
                const int32_t l = l0 + j;
                const void* x = xs + (c.ctx_input_norm ? (size_t)l * xstride : 0);
                g.seg[2 * j] = GemmSeg{x, m_.layer[l].k, H, H, kd, l * 2 * kd, 0, 0};
                g.seg[2 * j + 1] = GemmSeg{x, m_.layer[l].v, H, H, kd, l * 2 * kd + kd, 0, 0};
            }
            int kv_slices = 1;
            {
                Timed tm(this, "flush_kv", st);
                HIP_OK(gemm(g, bf16(), kPartCapFloats, cus_, st, 0, &kv_slices));
            }
            HeadArgs h{};
            h.src = kv_out;
            h.nsplit = kv_slices;
            h.src_stride = (int64_t)rows * ldkv;
            h.rows = d_info;
            h.seqs = d_desc;
            if (one) {
                h.pos0 = segs[si].pos0;
                h.cache0 = descs[0].cache;
                h.cap0 = descs[0].cap;
                h.ring0 = descs[0].ring;
            }
            h.ld = ldkv;
            h.nrows = rows;
            h.D = c.head_dim;
            h.Hq = c.q_heads;
            h.Hkv = c.kv_heads;
            h.L = L;
            h.q_col = -1;
            for (int j = 0; j < nl; ++j) {
                h.k_col[j] = (l0 + j) * 2 * kd;
                h.v_col[j] = (l0 + j) * 2 * kd + kd;
                h.layer[j] = l0 + j;
                h.k_norm[j] = m_.layer[l0 + j].k_norm;
            }
            h.qk_norm = c.qk_norm;
            h.w_bf16 = bf16();
            h.cache_bf16 = bf16();
            h.eps = c.rms_eps;
            fill_inv_freq(h);
            HIP_OK(head_finish(h, nl, st));
        }
        si = sj;
    }
    return 0;
}

int HipEngine::block_forward(const std::vector<SessView>& sess, const std::vector<BlockSeq>& seqs, float* logits,
                             float* hidden, void* ws, int32_t ws_sessions, void* stream) {
    const dflash_config& c = m_.cfg;
    const WsLayout w = layout(ws_sessions);
    hipStream_t st = (hipStream_t)stream;
    char* base = (char*)ws;
    const int32_t H = c.hidden, I = c.intermediate, qd = m_.qd, kd = m_.kd;

    // tables: one SeqDesc per block, one RowInfo per block row, the row of
    // every unembedded row (rows 1..n of each block), the attention work split
    std::vector<SeqDesc> descs;
    std::vector<RowInfo> info;
    std::vector<int32_t> rowsrc;
    int32_t R = 0, Rout = 0;
    int64_t total_keys = 0;
    for (const BlockSeq& b : seqs) {
        SeqDesc d = desc_of(sess[b.sess]);
        d.F = b.F;
        d.M = b.M;
        d.q_row0 = R;
        d.out_row0 = Rout;
        d.key_lo = c.window ? std::max(0, b.F - c.window + 1) : 0;
        d.current = b.current;
        total_keys += b.F + b.M - d.key_lo;
        for (int32_t i = 0; i < b.M; ++i) info.push_back({(int32_t)descs.size(), b.F + i});
        for (int32_t i = 1; i < b.M; ++i) rowsrc.push_back(R + i);
        R += b.M;
        Rout += b.M - 1;
        descs.push_back(d);
    }
    if (R > w.r_blk) return fail(DFLASH_E_CAPACITY, "block rows exceed the workspace");
    // attention split: every sequence's keys in chunks of one size.  If one
    // resident round of workgroups (target_items per kv head) can hold the
    // whole split with chunks of at most kAttnRoundChunk keys, use that (one
    // round, no tail).  Otherwise (many sequences, or very long ones) split
    // into chunks of 1024..4096 keys over several rounds, so that one long
    // sequence does not leave the other workgroups idle, the size chosen by
    // the schedule model below; the workspace bounds the item count.  When
    // that gives short chunks (little work in
    // all), one workgroup per CU instead: a second one on a CU only splits
    // its bandwidth, and every extra item costs a partial to write and to
    // combine.
    const int32_t nseq = (int32_t)seqs.size();
    // Several rounds: items are dispatched largest first (every kv head of an
    // item side by side), so the chunk decides how evenly the resident slots
    // finish.  Each candidate's schedule is simulated on the host (an item
    // costs its 64-key tiles plus a fixed start-up) and the earliest finish
    // wins; on the batched workload it picks 4096 keys, the fastest of the
    // measured chunks (1536..8192 keys).
    auto many_chunk = [&](int32_t slots, int64_t min_chunk) {
        int32_t best = 0;
        int64_t best_t = 0;
        std::vector<int32_t> sizes;
        for (int32_t ch = kAttnManyLo; ch <= kAttnManyHi; ch += 512) {
            if (ch < min_chunk) continue;
            sizes.clear();
            for (const SeqDesc& d : descs) {
                const int32_t nk = d.F + d.M - d.key_lo;
                // item i of ni takes tiles i, i + ni, ... of the sequence's T tiles
                const int32_t ni = (nk + ch - 1) / ch, T = (nk + 63) / 64;
                for (int32_t i = 0; i < ni; ++i) sizes.push_back((T - i + ni - 1) / ni);
            }
            if ((int64_t)sizes.size() > w.items_cap) continue;
            std::sort(sizes.begin(), sizes.end(), std::greater<int32_t>());
            std::priority_queue<int64_t, std::vector<int64_t>, std::greater<int64_t>> fin;
            for (int32_t i = 0; i < slots; ++i) fin.push(0);
            int64_t t_end = 0;
            for (int32_t tiles : sizes) {
                const int64_t t = fin.top() + tiles + kAttnItemStartTiles;
                fin.pop();
                fin.push(t);
                t_end = std::max(t_end, t);
            }
            if (!best || t_end < best_t) {
                best = ch;
                best_t = t_end;
            }
        }
        return best ? best : kAttnManyHi;
    };
    auto pick_chunk = [&](int32_t target_wg) {
        const int32_t target_items = std::max(1, target_wg / c.kv_heads);
        int64_t chunk64 = target_items > nseq ? (total_keys + target_items - nseq - 1) / (target_items - nseq)
                                              : (int64_t)kAttnRoundChunk + 1;
        if (chunk64 > kAttnRoundChunk) {
            const int64_t room = std::max<int64_t>(1, (int64_t)w.items_cap - nseq);
            const int64_t need = (total_keys + room - 1) / room;   // the workspace bounds the item count
            chunk64 = need > kAttnManyHi ? need : many_chunk(target_items, need);
        }
        return (int32_t)std::max<int64_t>(kAttnMinChunk, (chunk64 + 63) / 64 * 64);
    };
    int32_t chunk = pick_chunk(attn_target_wg());
    const bool long_chunks = chunk >= kAttnShortChunk;
    if (!long_chunks) chunk = pick_chunk(cus_);
    int32_t items = 0;
    for (SeqDesc& d : descs) {
        const int32_t nk = d.F + d.M - d.key_lo;
        d.item0 = items;
        d.nitems = (nk + chunk - 1) / chunk;
        items += d.nitems;
    }
    if (bf16() && items > w.items_cap) return fail(DFLASH_E_CAPACITY, "attention work exceeds the workspace");
    // Long chunks: each item takes every nitems-th 64-key tile of its
    // sequence instead of one run, so the workgroups of a kv head read
    // neighbouring tiles together (131072-key context: 97.1 -> 94.2 us per
    // layer; batched, several rounds: 295 -> 292 us, with the schedule model
    // and the dispatch order below counting the interleaved items' tiles).
    const int32_t strided = long_chunks;
    if (items > 0xffff || nseq > 0xffff) return fail(DFLASH_E_CAPACITY, "attention work items exceed 16-bit indices");
    // One session (bf16): its block's kernels take the descriptor, the anchor
    // and the first position from their arguments, so no table is uploaded
    // (one launch fewer, and no kernel starts with two dependent table loads).
    const bool one = nseq == 1 && bf16();
    const SeqDesc* d_desc = nullptr;
    const RowInfo* d_info = nullptr;
    const int32_t* d_rowsrc = nullptr;
    const uint32_t* d_order = nullptr;
    if (!one) {
        // dispatch order of the attention items: largest chunks first (stable),
        // so the partial chunks at the sequences' ends fill the launch's tail
        std::vector<uint32_t> order;
        order.reserve(items);
        for (int32_t s = 0; s < nseq; ++s)
            for (int32_t i = 0; i < descs[s].nitems; ++i)
                order.push_back(((uint32_t)s << 16) | (uint32_t)(descs[s].item0 + i));
        auto item_keys = [&](uint32_t od) {   // (in 64-key tiles when the items interleave)
            const SeqDesc& d = descs[od >> 16];
            const int32_t i = (int32_t)(od & 0xffffu) - d.item0;
            if (strided) return ((d.F + d.M - d.key_lo + 63) / 64 - i + d.nitems - 1) / d.nitems;
            return std::min(chunk, d.F + d.M - d.key_lo - i * chunk);
        };
        std::stable_sort(order.begin(), order.end(),
                         [&](uint32_t x, uint32_t y) { return item_keys(x) > item_keys(y); });
        Tables tb;
        const size_t o_desc = tb.add(descs.data(), sizeof(SeqDesc) * descs.size());
        const size_t o_info = tb.add(info.data(), sizeof(RowInfo) * info.size());
        const size_t o_src = tb.add(rowsrc.data(), sizeof(int32_t) * rowsrc.size());
        const size_t o_ord = tb.add(order.data(), sizeof(uint32_t) * order.size());
        char* tab = base + w.tables;
        HIP_OK(upload(tab, tb.blob.data(), tb.blob.size(), st));
        d_desc = (const SeqDesc*)(tab + o_desc);
        d_info = (const RowInfo*)(tab + o_info);
        d_rowsrc = (const int32_t*)(tab + o_src);
        d_order = (const uint32_t*)(tab + o_ord);
    }

    float* h = (float*)(base + w.blk_h);
    void* x = base + w.blk_x;
    float* qkv = (float*)(base + w.blk_qkv);
    float* hpart = (float*)(base + w.blk_part);
    float* part = (float*)(base + w.part);
    const int32_t ldq = qkv_ld();
    {
        // embedding rows and the first layer's input norm in one pass
        EmbedArgs e{m_.embed, h, d_info, d_desc, H, R, c.mask_id, bf16(), m_.layer[0].in_ln, x, c.rms_eps, bf16()};
        e.current = descs[0].current;   // (rows == nullptr: one block, anchor first)
        HIP_OK(embed(e, st));
    }
    for (int32_t l = 0; l < c.layers; ++l) {
        const LayerW& lw = m_.layer[l];
        int qkv_slices = 1;
        {
            GemmArgs g = gemm_args(R, H, qkv, ldq, kPartial, part, w.blk_slices);
            g.seg[0] = GemmSeg{x, lw.q, H, H, qd, 0, 0, 0};
            g.seg[1] = GemmSeg{x, lw.k, H, H, kd, qd, 0, 0};
            g.seg[2] = GemmSeg{x, lw.v, H, H, kd, qd + kd, 0, 0};
            g.nseg = 3;
            if (c.gate) g.seg[g.nseg++] = GemmSeg{x, lw.g, H, H, c.q_heads, qd + 2 * kd, 0, 0};
            Timed tg(this, "layer_gemms", st);
            HIP_OK(gemm(g, bf16(), kPartCapFloats, cus_, st, 0, &qkv_slices));
        }
        {
            HeadArgs hd{};
            hd.src = qkv;
            hd.nsplit = qkv_slices;
            hd.src_stride = (int64_t)R * ldq;
            hd.rows = d_info;
            hd.seqs = d_desc;
            if (one) {   // rows F, F + 1, ... of the one session
                hd.pos0 = descs[0].F;
                hd.cache0 = descs[0].cache;
                hd.cap0 = descs[0].cap;
                hd.ring0 = descs[0].ring;
            }
            hd.q_out = base + w.blk_q;
            hd.q_norm = lw.q_norm;
            hd.k_norm[0] = lw.k_norm;
            hd.ld = ldq;
            hd.nrows = R;
            hd.D = c.head_dim;
            hd.Hq = c.q_heads;
            hd.Hkv = c.kv_heads;
            hd.L = c.layers;
            hd.q_col = 0;
            hd.k_col[0] = qd;
            hd.v_col[0] = qd + kd;
            hd.layer[0] = l;
            hd.qk_norm = c.qk_norm;
            hd.w_bf16 = bf16();
            hd.cache_bf16 = bf16();
            hd.q_bf16 = bf16();
            hd.eps = c.rms_eps;
            fill_inv_freq(hd);
            HIP_OK(head_finish(hd, 1, st));
        }
        {
            AttnArgs a{};
            a.Q = base + w.blk_q;
            a.seqs = d_desc;
            a.rows = d_info;
            a.part_o = (float*)(base + w.attn_o);
            a.part_ml = (float*)(base + w.attn_ml);
            a.gate_src = qkv;
            a.order = d_order;
            a.seq0 = descs[0];              // (rows == nullptr: one session)
            a.gate_nsplit = qkv_slices;
            a.gate_stride = (int64_t)R * ldq;
            a.out = base + w.blk_attn;
            a.nseq = (int32_t)descs.size();
            a.nrows = R;
            a.layer = l;
            a.L = c.layers;
            a.Hq = c.q_heads;
            a.Hkv = c.kv_heads;
            a.D = c.head_dim;
            a.causal = c.causal;
            a.window = c.window;
            a.chunk = chunk;
            a.strided = strided;
            a.total_items = items;
            a.gate = c.gate;
            a.gate_ld = ldq;
            a.gate_col = qd + 2 * kd;
            a.out_bf16 = bf16();
            a.scale = 1.f / sqrtf((float)c.head_dim);
            Timed tm(this, "attention", st);
            if (bf16() && stage_ == "attention_partial") {
                {
                    Timed tp(this, "attention_partial", st);
                    HIP_OK(attention(a, true, st, 1));
                }
                HIP_OK(attention(a, true, st, 2));
            } else {
                HIP_OK(attention(a, bf16(), st));
            }
        }
        int o_slices = 1;
        {
            GemmArgs g = gemm_args(R, qd, hpart, H, kPartial, part, w.blk_slices);
            g.seg[0] = GemmSeg{base + w.blk_attn, lw.o, qd, qd, H, 0, 0, 0};
            g.nseg = 1;
            Timed tg(this, "layer_gemms", st);
            HIP_OK(gemm(g, bf16(), kPartCapFloats, cus_, st, 0, &o_slices));
        }
        {   // h += attention output; x = post-attention norm of h
            NormArgs n = norm_args(h, 0, H, R, H);
            n.part = hpart;
            n.nsplit = o_slices;
            n.part_stride = (int64_t)R * H;
            n.writeback = h;
            n.nout = 1;
            n.gain[0] = lw.post_ln;
            n.out[0] = x;
            HIP_OK(rmsnorm(n, st));
        }
        {
            GemmArgs g = gemm_args(R, H, (float*)(base + w.blk_mlp), 2 * I, kSwiGLU, part, 1);
            g.seg[0] = GemmSeg{x, lw.gate, H, H, I, 0, 0, 0};
            g.seg[1] = GemmSeg{x, lw.up, H, H, I, I, 0, 0};
            g.nseg = 2;
            g.out = base + w.blk_act;        // act = silu(x W_gate^T) * (x W_up^T)
            g.ldo = I;
            g.out_bf16 = bf16();
            Timed tg(this, "layer_gemms", st);
            HIP_OK(gemm(g, bf16(), kPartCapFloats, cus_, st));
        }
        int d_slices = 1;
        {
            GemmArgs g = gemm_args(R, I, hpart, H, kPartial, part, w.blk_slices);
            g.seg[0] = GemmSeg{base + w.blk_act, lw.down, I, I, H, 0, 0, 0};
            g.nseg = 1;
            Timed tg(this, "layer_gemms", st);
            HIP_OK(gemm(g, bf16(), kPartCapFloats, cus_, st, 0, &d_slices));
        }
        {   // h += MLP output; x = next layer's input norm (the final norm after the last)
            NormArgs n = norm_args(h, 0, H, R, H);
            n.part = hpart;
            n.nsplit = d_slices;
            n.part_stride = (int64_t)R * H;
            n.writeback = h;
            n.nout = 1;
            n.gain[0] = l + 1 < c.layers ? m_.layer[l + 1].in_ln : m_.norm;
            n.out[0] = x;
            HIP_OK(rmsnorm(n, st));
        }
    }
    if (hidden) HIP_OK(hipMemcpyAsync(hidden, h, sizeof(float) * (size_t)R * H, hipMemcpyDeviceToDevice, st));
    if (Rout > 0) {
        GemmArgs g = gemm_args(Rout, H, logits, c.vocab, kStore, part, 1);
        g.a_rows = d_rowsrc;                 // rows 1..n of every block
        g.seg[0] = GemmSeg{x, m_.lm_head, H, H, c.vocab, 0, 0, 0};
        if (one) g.seg[0].A = (const uint16_t*)x + H;   // one block: rows 1..n are contiguous
        g.nseg = 1;
        Timed tm(this, "unembed", st);
        HIP_OK(gemm(g, bf16(), kPartCapFloats, cus_, st, 1));
    }
    return 0;
}

int HipEngine::verify(const std::vector<SessView>& sess, const int32_t* draft_offsets, const float* target,
                      const int32_t* draft_ids, const float* draft_probs, const dflash_verify_params& p,
                      int32_t* accepted, int32_t* next, void* ws, int32_t ws_sessions, void* stream) {
    const WsLayout w = layout(ws_sessions);
    const int32_t count = (int32_t)sess.size();
    const int32_t Rt = draft_offsets[count] + count;     // target rows: n_k + 1 per session
    if (Rt > w.r_blk) return fail(DFLASH_E_CAPACITY, "verified rows exceed the workspace");
    char* base = (char*)ws;
    return verify_in(sess, draft_offsets, target, draft_ids, draft_probs, p, accepted, next, base + w.tables,
                     (float*)(base + w.stats), (float*)(base + w.stats2), stream);
}

// The scratch a verification needs: its tables, then two [Rt][nchunk][4]
// float statistics arrays (every element is written before it is read).
size_t HipEngine::verify_scratch_bytes(int32_t count, int32_t Rt) const {
    const size_t stats = 16 * (size_t)Rt * ((m_.cfg.vocab + kSampleChunk - 1) / kSampleChunk);
    return al(verify_table_bytes(count, Rt)) + 2 * al(stats);
}

size_t HipEngine::verify_table_bytes(int32_t count, int32_t Rt) const {
    return sizeof(SeqDesc) * (size_t)count + sizeof(RowInfo) * (size_t)Rt + sizeof(int32_t) * (count + 1) + 64;
}

int HipEngine::verify_scratch(const std::vector<SessView>& sess, const int32_t* draft_offsets, const float* target,
                              const int32_t* draft_ids, const float* draft_probs, const dflash_verify_params& p,
                              int32_t* accepted, int32_t* next, void* stream) {
    if (!scratch_) return fail(DFLASH_E_HIP, "no scratch array on this device");
    const int32_t count = (int32_t)sess.size();
    const int32_t Rt = draft_offsets[count] + count;
    if (verify_scratch_bytes(count, Rt) > kScratchBytes)
        return fail(DFLASH_E_CAPACITY, "verification exceeds the static scratch array (" +
                                           std::to_string(kScratchBytes >> 20) + " MiB)");
    const size_t stats = al(16 * (size_t)Rt * ((m_.cfg.vocab + kSampleChunk - 1) / kSampleChunk));
    char* base = (char*)scratch_;
    char* tab = base;
    char* s1 = base + al(verify_table_bytes(count, Rt));
    return verify_in(sess, draft_offsets, target, draft_ids, draft_probs, p, accepted, next, tab, (float*)s1,
                     (float*)(s1 + stats), stream);
}

int HipEngine::verify_in(const std::vector<SessView>& sess, const int32_t* draft_offsets, const float* target,
                         const int32_t* draft_ids, const float* draft_probs, const dflash_verify_params& p,
                         int32_t* accepted, int32_t* next, char* tab, float* stats, float* stats2, void* stream) {
    const dflash_config& c = m_.cfg;
    hipStream_t st = (hipStream_t)stream;
    const int32_t count = (int32_t)sess.size();
    const int32_t Rt = draft_offsets[count] + count;
    std::vector<SeqDesc> descs(count);
    std::vector<RowInfo> info;
    for (int32_t k = 0; k < count; ++k) {
        descs[k] = desc_of(sess[k]);
        for (int32_t i = 0; i <= draft_offsets[k + 1] - draft_offsets[k]; ++i) info.push_back({k, i});
    }
    // the stage timer brackets the whole call's GPU work, its table upload
    // included (a bracket opened after the upload caught a varying share of it)
    Timed tm(this, "verify", st);
    VerifyArgs a{};
    if (count == 1) {
        a.seq0 = descs[0];    // rows, seqs and offs stay null: no table upload
        a.n0 = draft_offsets[1];
    } else {
        Tables tb;
        const size_t o_desc = tb.add(descs.data(), sizeof(SeqDesc) * descs.size());
        const size_t o_info = tb.add(info.data(), sizeof(RowInfo) * info.size());
        const size_t o_offs = tb.add(draft_offsets, sizeof(int32_t) * (size_t)(count + 1));
        HIP_OK(upload(tab, tb.blob.data(), tb.blob.size(), st));
        a.seqs = (const SeqDesc*)(tab + o_desc);
        a.rows = (const RowInfo*)(tab + o_info);
        a.offs = (const int32_t*)(tab + o_offs);
    }
    a.target = target;
    a.draft_ids = draft_ids;
    a.draft_probs = draft_probs;
    a.stats = stats;
    a.stats2 = stats2;
    a.accepted = accepted;
    a.nchunk = (c.vocab + kSampleChunk - 1) / kSampleChunk;
    a.next = next;
    a.V = c.vocab;
    a.Rt = Rt;
    a.nseq = count;
    a.chunk = kSampleChunk;
    a.round = p.round;
    a.temperature = p.temperature;
    HIP_OK(kern::verify(a, st));
    return 0;
}

int HipEngine::select(const std::vector<SessView>& sess, const int32_t* row_offsets, const float* logits,
                      const int32_t* current, const dflash_select_params& p, int32_t* tokens, int32_t* cand_ids,
                      float* cand_probs, float* dense, void* ws, int32_t ws_sessions, void* stream) {
    const dflash_config& c = m_.cfg;
    const WsLayout w = layout(ws_sessions);
    hipStream_t st = (hipStream_t)stream;
    char* base = (char*)ws;
    const int32_t count = (int32_t)sess.size();
    const int32_t R = row_offsets[count];
    if (R > w.r_blk) return fail(DFLASH_E_CAPACITY, "selected rows exceed the workspace");
    std::vector<SeqDesc> descs(count);
    for (int32_t k = 0; k < count; ++k) descs[k] = desc_of(sess[k]);
    Timed tm(this, "select", st);   // (the whole call, its table upload included)
    SelectArgs a{};
    if (count == 1) {
        a.seq0 = descs[0];            // seqs, offs and anchors stay null: no table upload
        a.seq0.current = current[0];
    } else {
        Tables tb;
        const size_t o_desc = tb.add(descs.data(), sizeof(SeqDesc) * descs.size());
        const size_t o_offs = tb.add(row_offsets, sizeof(int32_t) * (size_t)(count + 1));
        const size_t o_anch = tb.add(current, sizeof(int32_t) * (size_t)count);
        char* tab = base + w.tables;
        HIP_OK(upload(tab, tb.blob.data(), tb.blob.size(), st));
        a.seqs = (const SeqDesc*)(tab + o_desc);
        a.offs = (const int32_t*)(tab + o_offs);
        a.anchors = (const int32_t*)(tab + o_anch);
    }
    a.logits = logits;
    a.P = m_.sel_prev;
    a.Q = m_.sel_next;
    a.cand = (float*)(base + w.sel);
    a.prep = (float*)(base + w.sel_prep);
    a.tokens = tokens;
    a.cand_ids = cand_ids;
    a.cand_probs = cand_probs;
    a.dense = p.temperature > 0.f ? dense : nullptr;
    a.V = c.vocab;
    a.R = R;
    a.nseq = count;
    a.K = c.sel_candidates;
    a.Ds = c.sel_dim;
    a.chunk = kSampleChunk;
    a.nchunk = w.nchunk_max;
    a.round = p.round;
    a.w_bf16 = bf16();
    a.temperature = p.temperature;
    HIP_OK(kern::select(a, st));
    return 0;
}

int HipEngine::sample(const std::vector<SessView>& sess, const int32_t* row_offsets, const float* logits,
                      const dflash_sample_params& p, int32_t* ids, float* probs, void* ws, int32_t ws_sessions,
                      void* stream) {
    const dflash_config& c = m_.cfg;
    const WsLayout w = layout(ws_sessions);
    hipStream_t st = (hipStream_t)stream;
    char* base = (char*)ws;
    const int32_t count = (int32_t)sess.size();
    const int32_t R = row_offsets[count];
    if (R > w.r_blk) return fail(DFLASH_E_CAPACITY, "sampled rows exceed the workspace");
    std::vector<SeqDesc> descs(count);
    std::vector<RowInfo> info;
    bool any_hist = false;
    for (int32_t k = 0; k < count; ++k) {
        descs[k] = desc_of(sess[k]);
        descs[k].hist_n = std::min(std::min(sess[k].hist_count, kHistory), p.history);
        descs[k].hist_head = sess[k].hist_head;
        any_hist |= descs[k].hist_n > 0;
        for (int32_t r = row_offsets[k]; r < row_offsets[k + 1]; ++r) info.push_back({k, r - row_offsets[k]});
    }
    SampleArgs a{};
    if (count == 1) {
        a.seq0 = descs[0];    // rows and seqs stay null: no table upload
    } else {
        Tables tb;
        const size_t o_desc = tb.add(descs.data(), sizeof(SeqDesc) * descs.size());
        const size_t o_info = tb.add(info.data(), sizeof(RowInfo) * info.size());
        char* tab = base + w.tables;
        HIP_OK(upload(tab, tb.blob.data(), tb.blob.size(), st));
        a.seqs = (const SeqDesc*)(tab + o_desc);
        a.rows = (const RowInfo*)(tab + o_info);
    }
    a.logits = logits;
    a.bitmap = (uint32_t*)(base + w.bitmap);
    a.stats = (float*)(base + w.stats);
    a.ids = ids;
    a.probs = probs;
    a.V = c.vocab;
    a.R = R;
    a.nseq = count;
    a.words = (c.vocab + 31) / 32;
    a.chunk = kSampleChunk;
    a.nchunk = w.nchunk_max;
    a.round = p.round;
    a.use_penalty = (p.rep_penalty != 1.f && any_hist) ? 1 : 0;
    a.temperature = p.temperature;
    a.rho = p.rep_penalty;
    Timed tm(this, "sampler", st);
    HIP_OK(kern::sample(a, st));
    return 0;
}

}  // namespace

Engine* make_engine(const Model& m, std::string* err) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        *err = std::string("hipGetDevice: ") + hipGetErrorString(e);
        return nullptr;
    }
    int cus = 0;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess || cus <= 0) {
        *err = std::string("hipDeviceGetAttribute: ") + hipGetErrorString(e);
        return nullptr;
    }
    void* scratch_ptr = nullptr;
    e = scratch_address(dev, &scratch_ptr);
    if (e != hipSuccess) {
        *err = std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e);
        return nullptr;
    }
    return new HipEngine(m, cus, scratch_ptr);
}

}  // namespace dflash
