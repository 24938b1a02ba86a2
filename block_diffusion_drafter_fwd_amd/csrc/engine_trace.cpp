// Trace backend: records every device step the state machine asks for and
// performs none.  Linked into the host-only test library so that the C ABI's
// integer logic (offsets, pending rows, rewinds, window drop, chunking) can be
// checked on a machine without a GPU.  Pointers handed to it are never
// dereferenced.
#include <cstdio>
#include <mutex>
#include <string>
#include <vector>

#include "engine.h"

namespace dflash {
namespace {

std::mutex g_mu;
std::vector<std::string> g_log;
int g_fail_in = 0;     // > 0: the g_fail_in-th device step from now fails (E_HIP)

// a device step that the test asked to fail, as a refused HIP enqueue would
int injected() {
    std::lock_guard<std::mutex> lk(g_mu);
    if (g_fail_in > 0 && --g_fail_in == 0) return fail(DFLASH_E_HIP, "injected device failure");
    return 0;
}

void log_line(const std::string& s) {
    std::lock_guard<std::mutex> lk(g_mu);
    g_log.push_back(s);
}

class TraceEngine : public Engine {
public:
    explicit TraceEngine(const Model& m) : m_(m) {}
    size_t workspace_bytes(int32_t max_sessions) const override { return 256 * (size_t)max_sessions; }
    int copy_rows(void*, const void*, size_t bytes, void*) override {
        if (int rc = injected()) return rc;
        log_line("copy rows=" + std::to_string(bytes / ((size_t)m_.fc_in * m_.elem)));
        return 0;
    }
    int write_history(const SessView&, int32_t slot0, const int32_t* t, int32_t count, void*) override {
        if (int rc = injected()) return rc;
        std::string s = "hist slot=" + std::to_string(slot0) + " tokens=";
        for (int32_t i = 0; i < count; ++i) s += (i ? "," : "") + std::to_string(t[i]);
        log_line(s);
        return 0;
    }
    int ctx_forward(const std::vector<SessView>&, const std::vector<CtxSeg>& segs, void*, int32_t,
                    void*, int) override {
        if (int rc = injected()) return rc;
        for (const CtxSeg& g : segs)
            log_line("ctx sess=" + std::to_string(g.sess) + " pos0=" + std::to_string(g.pos0) +
                     " rows=" + std::to_string(g.nrows));
        return 0;
    }
    int block_forward(const std::vector<SessView>&, const std::vector<BlockSeq>& seqs, float*, float*,
                      void*, int32_t, void*) override {
        if (int rc = injected()) return rc;
        for (const BlockSeq& b : seqs)
            log_line("block sess=" + std::to_string(b.sess) + " F=" + std::to_string(b.F) +
                     " M=" + std::to_string(b.M) + " cur=" + std::to_string(b.current));
        return 0;
    }
    int verify(const std::vector<SessView>& sess, const int32_t* offs, const float*, const int32_t*, const float*,
               const dflash_verify_params& p, int32_t*, int32_t*, void*, int32_t, void*) override {
        if (int rc = injected()) return rc;
        log_line("verify drafts=" + std::to_string(offs[sess.size()]) + " sessions=" +
                 std::to_string(sess.size()) + " round=" + std::to_string(p.round));
        return 0;
    }
    int select(const std::vector<SessView>& sess, const int32_t* row_offsets, const float*, const int32_t* current,
               const dflash_select_params& p, int32_t*, int32_t*, float*, float* dense, void*, int32_t,
               void*) override {
        if (int rc = injected()) return rc;
        std::string s = "select rows=" + std::to_string(row_offsets[sess.size()]) +
                        " round=" + std::to_string(p.round) + " dense=" + std::to_string(dense != nullptr) + " anchors=";
        for (size_t k = 0; k < sess.size(); ++k) s += (k ? "," : "") + std::to_string(current[k]);
        log_line(s);
        return 0;
    }
    int verify_scratch(const std::vector<SessView>& sess, const int32_t* offs, const float*, const int32_t*,
                       const float*, const dflash_verify_params& p, int32_t*, int32_t*, void*) override {
        if (int rc = injected()) return rc;
        log_line("verify_noalloc drafts=" + std::to_string(offs[sess.size()]) + " sessions=" +
                 std::to_string(sess.size()) + " round=" + std::to_string(p.round));
        return 0;
    }
    int sample(const std::vector<SessView>& sess, const int32_t* row_offsets, const float*,
               const dflash_sample_params& p, int32_t*, float*, void*, int32_t, void*) override {
        if (int rc = injected()) return rc;
        std::string s = "sample rows=" + std::to_string(row_offsets[sess.size()]) +
                        " round=" + std::to_string(p.round) + " hist=";
        for (size_t k = 0; k < sess.size(); ++k)
            s += (k ? "," : "") + std::to_string(sess[k].hist_count) + "@" + std::to_string(sess[k].hist_head);
        log_line(s);
        return 0;
    }
    int cache_read(const SessView&, int32_t layer, int32_t pos0, int32_t count, float*, float*,
                   void*) override {
        log_line("read layer=" + std::to_string(layer) + " pos0=" + std::to_string(pos0) +
                 " count=" + std::to_string(count));
        return 0;
    }

    int profile_begin(const std::string& stage) override {
        log_line("profile " + stage);
        return 0;
    }
    int profile_end(double* ms, int32_t* n) override {
        *ms = 0.0;
        *n = 0;
        return 0;
    }

private:
    Model m_;
};

}  // namespace

Engine* make_engine(const Model& m, std::string*) { return new TraceEngine(m); }

}  // namespace dflash

extern "C" int dflash_trace_count(void) {
    std::lock_guard<std::mutex> lk(dflash::g_mu);
    return (int)dflash::g_log.size();
}

extern "C" int dflash_trace_line(int i, char* buf, int len) {
    std::lock_guard<std::mutex> lk(dflash::g_mu);
    if (i < 0 || i >= (int)dflash::g_log.size() || !buf || len <= 0) return -1;
    std::snprintf(buf, (size_t)len, "%s", dflash::g_log[i].c_str());
    return 0;
}

// the n-th device step from now returns DFLASH_E_HIP (0: none)
extern "C" void dflash_trace_fail_in(int n) {
    std::lock_guard<std::mutex> lk(dflash::g_mu);
    dflash::g_fail_in = n;
}

extern "C" void dflash_trace_clear(void) {
    std::lock_guard<std::mutex> lk(dflash::g_mu);
    dflash::g_log.clear();
}
