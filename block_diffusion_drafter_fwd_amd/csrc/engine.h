// Internal interface between the C-ABI state machine (api.cpp) and a compute
// backend.  The HIP backend (engine_hip.hip) runs every step on the GPU; the
// trace backend (engine_trace.cpp) records the calls so that the state machine
// can be tested on a host without a GPU.
#pragma once

#include <algorithm>
#include <cstddef>
#include <cstdint>
#include <string>
#include <vector>

#include "../../include/dflash.h"

namespace dflash {

constexpr int kMaxLayers = 16;
constexpr int kHistory = 512;      // committed tokens kept for penalties

struct LayerW {
    const void *in_ln, *post_ln;
    const void *q, *k, *v;          // row slices of qkv_proj when fused
    const void *q_norm, *k_norm, *g, *o;
    const void *gate, *up, *down;
};

struct Model {
    dflash_config cfg;
    const void *embed, *lm_head, *fc, *hidden_norm, *norm, *aux_norms;
    const void *sel_prev, *sel_next;     // DFlash2 selector tables [V, Ds] (sel_candidates > 0)
    LayerW layer[kMaxLayers];
    int qd, kd, fc_in;              // Hq*D, Hkv*D, taps*Ht
    size_t elem;                    // bytes per element of weights, cache and features
};

// Byte layout of a session arena: [K/V cache | pending rows | history ring].
struct ArenaLayout {
    size_t cache_off, cache_bytes, pending_off, pending_bytes, hist_off, total;
};
ArenaLayout arena_layout(const Model& m, int32_t capacity);

// What a backend needs to know about one session.
// One session's commit of a round: history tokens (host) into the ring at
// slot0 (wrapping), and `bytes` of feature rows from src to dst (device).
struct CommitItem {
    int32_t* hist;
    int32_t slot0;
    const int32_t* tokens;
    int32_t count;
    void* dst;
    const void* src;
    size_t bytes;
};

struct SessView {
    void* cache;        // arena base: [L][2][Hkv][cap][D]
    int32_t cap;
    int32_t ring;       // 1: slot = position mod cap
    int32_t* hist;      // device ring of kHistory committed tokens
    int32_t hist_count; // tokens ever written (clamped use: last min(count, kHistory))
    int32_t hist_head;  // next ring slot
    uint64_t seed, stream_id;
};

// A run of context rows of one session, contiguous in device memory.
struct CtxSeg {
    int32_t sess;       // index into the session list of the call
    const void* rows;   // first feature row [taps*Ht]
    int32_t nrows;
    int32_t pos0;       // absolute position of the first row
};

// One session's block in a block forward.
struct BlockSeq {
    int32_t sess;
    int32_t F;          // anchor position (frontier after taking pending rows)
    int32_t M;          // rows: anchor + n mask rows
    int32_t current;    // anchor token
};

class Engine {
public:
    virtual ~Engine() {}
    virtual size_t workspace_bytes(int32_t max_sessions) const = 0;
    virtual int copy_rows(void* dst, const void* src, size_t bytes, void* stream) = 0;
    virtual int write_history(const SessView& s, int32_t slot0, const int32_t* tokens,
                              int32_t count, void* stream) = 0;
    // write_history and then copy_rows, as one step where the backend can
    // (the history run must not wrap the ring)
    virtual int commit_rows(const SessView& s, int32_t slot0, const int32_t* tokens, int32_t count, void* dst,
                            const void* src, size_t bytes, void* stream) {
        if (int rc = write_history(s, slot0, tokens, count, stream)) return rc;
        return bytes ? copy_rows(dst, src, bytes, stream) : 0;
    }
    // commit_rows for several sessions, in as few launches as the backend can
    // (here: the history in at most two runs, as the ring wraps at most once
    // for count <= kHistory, then the rows)
    virtual int commit_many(const std::vector<CommitItem>& items, void* stream) {
        for (const CommitItem& c : items) {
            SessView v{};
            v.hist = c.hist;
            const int32_t first = std::min(c.count, kHistory - c.slot0);
            if (first > 0)
                if (int rc = write_history(v, c.slot0, c.tokens, first, stream)) return rc;
            if (c.count > first)
                if (int rc = write_history(v, 0, c.tokens + first, c.count - first, stream)) return rc;
            if (c.bytes)
                if (int rc = copy_rows(c.dst, c.src, c.bytes, stream)) return rc;
        }
        return 0;
    }
    // lane 0 or 1: which of the workspace's two sets of context-path buffers
    // the pass uses (the passes of one call may run on two streams at once)
    virtual int ctx_forward(const std::vector<SessView>& sess, const std::vector<CtxSeg>& segs,
                            void* ws, int32_t ws_sessions, void* stream, int lane) = 0;
    // A second stream for a session (lane 1 of its context passes): opened
    // with the session, closed with it; a call forks it from the session's
    // stream before its first lane-1 pass and joins it back before returning.
    // The default backend has none (every pass on lane 0).
    virtual int aux_open(void** aux) {
        *aux = nullptr;
        return 0;
    }
    virtual void aux_close(void*) {}
    virtual void* aux_stream(void*) { return nullptr; }
    virtual int aux_fork(void*, void*) { return 0; }
    virtual int aux_join(void*, void*) { return 0; }
    virtual int block_forward(const std::vector<SessView>& sess, const std::vector<BlockSeq>& seqs,
                              float* logits, float* hidden, void* ws, int32_t ws_sessions,
                              void* stream) = 0;
    virtual int sample(const std::vector<SessView>& sess, const int32_t* row_offsets,
                       const float* logits, const dflash_sample_params& p, int32_t* ids,
                       float* probs, void* ws, int32_t ws_sessions, void* stream) = 0;
    virtual int verify(const std::vector<SessView>& sess, const int32_t* draft_offsets, const float* target,
                       const int32_t* draft_ids, const float* draft_probs, const dflash_verify_params& p,
                       int32_t* accepted, int32_t* next, void* ws, int32_t ws_sessions, void* stream) = 0;
    virtual int select(const std::vector<SessView>& sess, const int32_t* row_offsets, const float* logits,
                       const int32_t* current, const dflash_select_params& p, int32_t* tokens, int32_t* cand_ids,
                       float* cand_probs, float* dense, void* ws, int32_t ws_sessions, void* stream) = 0;
    // verify with the backend's own static scratch instead of a workspace
    virtual int verify_scratch(const std::vector<SessView>& sess, const int32_t* draft_offsets,
                               const float* target, const int32_t* draft_ids, const float* draft_probs,
                               const dflash_verify_params& p, int32_t* accepted, int32_t* next, void* stream) = 0;
    virtual int cache_read(const SessView& s, int32_t layer, int32_t pos0, int32_t count,
                           float* k_out, float* v_out, void* stream) = 0;
    // event timing of one named stage (see dflash_profile_begin)
    virtual int profile_begin(const std::string& stage) = 0;
    virtual int profile_end(double* total_ms, int32_t* launches) = 0;
};

// Stages that can be timed.
inline bool known_stage(const std::string& s) {
    return s == "unembed" || s == "attention" || s == "attention_partial" || s == "flush_fc" || s == "flush_kv" || s == "sampler" ||
           s == "verify" || s == "layer_gemms" || s == "select";
}

// Defined by the backend translation unit that is linked in.
Engine* make_engine(const Model& m, std::string* err);

// Thread-local error text, read back by dflash_last_error().
int fail(int code, const std::string& msg);

}  // namespace dflash
