// api.cpp -- the extern "C" entry points of libdspark.so: argument
// validation, workspace layout, kernel sequencing and per-kernel profiling.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "dspark.h"
#include "internal.hpp"

namespace dspark {

// ------------------------------------------------------------------ profiling

namespace {

struct ProfEntry {
    std::string name;
    int64_t launches = 0;
    double total_ms = 0.0;
};

struct Pending {
    int entry;
    hipEvent_t start, stop;
};

struct Profiler {
    std::mutex mu;
    bool enabled = false;
    // read without the lock on every launch: with profiling off a launch
    // takes no lock
    std::atomic<bool> on{false};
    std::vector<ProfEntry> entries;
    std::vector<Pending> pending;
    std::vector<hipEvent_t> pool;

    int entry_for(const char *name) {
        for (size_t i = 0; i < entries.size(); ++i)
            if (entries[i].name == name) return int(i);
        entries.push_back(ProfEntry{name});
        return int(entries.size() - 1);
    }
    hipEvent_t take_event() {
        if (!pool.empty()) {
            hipEvent_t e = pool.back();
            pool.pop_back();
            return e;
        }
        hipEvent_t e = nullptr;
        if (hipEventCreate(&e) != hipSuccess) return nullptr;
        return e;
    }
};

Profiler &prof() {
    static Profiler p;
    return p;
}

}  // namespace

ProfEvents prof_events(const char *name) {
    Profiler &p = prof();
    if (!p.on.load(std::memory_order_acquire)) return {};
    std::lock_guard<std::mutex> g(p.mu);
    if (!p.enabled) return {};
    Pending pd{p.entry_for(name), p.take_event(), p.take_event()};
    if (!pd.start || !pd.stop) return {};
    p.pending.push_back(pd);
    return {pd.start, pd.stop};
}

}  // namespace dspark

using namespace dspark;

namespace {

bool rank_supported(int wdtype, int r) {
    if (wdtype == DSPARK_BF16) return r == 16 || r == 32 || r == 64 || r == 128 || r == 256;
    if (wdtype == DSPARK_F32) return r == 16 || r == 32 || r == 64 || r == 128;
    return false;
}

bool sizes_ok(int B, int gamma, int V, int r) {
    return B >= 1 && B <= DSPARK_MAX_BATCH && gamma >= 1 && gamma <= DSPARK_MAX_GAMMA && V >= 1 &&
           V <= DSPARK_MAX_VOCAB && r >= 1;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t draft_bytes(int B, int V) {
    const DraftPlan p = draft_plan(B, V);
    size_t bytes = 0;
    draft_carve(nullptr, B, p, &bytes);
    return bytes;
}

size_t accept_bytes(int B, int gamma, int V) {
    const AcceptPlan p = accept_plan(B, gamma, V);
    size_t bytes = 0;
    accept_carve(nullptr, B, gamma, p, &bytes);
    return bytes;
}

size_t verify_bytes(int B, int gamma, int V) {
    const VerifyPlan p = verify_plan(B, gamma, V);
    size_t bytes = 0;
    verify_carve(nullptr, B, gamma, V, p, &bytes);
    return bytes;
}

}  // namespace

extern "C" {

int dspark_version(void) { return 10000; }

const char *dspark_status_string(int status) {
    switch (status) {
        case DSPARK_OK: return "ok";
        case DSPARK_ERR_ARG: return "invalid argument";
        case DSPARK_ERR_UNSUPPORTED: return "unsupported size or type";
        case DSPARK_ERR_WORKSPACE: return "workspace missing or too small";
        case DSPARK_ERR_HIP: return "HIP runtime error";
        case DSPARK_ERR_DEVICE_INPUT: return "device-side input check failed";
        case DSPARK_ERR_SCRATCH: return "sizes exceed the allocation-free entry point's fixed scratch";
        default: return "unknown status";
    }
}

size_t dspark_draft_workspace_size(int B, int gamma, int V, int r) {
    if (!sizes_ok(B, gamma, V, r)) return 0;
    return draft_bytes(B, V);
}

}  // extern "C"

namespace {

// The host-side argument checks of the draft entry points.
int draft_args(const float *U, const void *W1, const void *W2, int wdtype, const int32_t *anchor,
               const float *temperature, int B, int gamma, int V, int r, const int32_t *x_out, const float *lse_out,
               const float *qx_out) {
    if (!U || !W1 || !W2 || !anchor || !temperature || !x_out || !lse_out || !qx_out) return DSPARK_ERR_ARG;
    if (!sizes_ok(B, gamma, V, r)) return DSPARK_ERR_ARG;
    if (wdtype != DSPARK_BF16 && wdtype != DSPARK_F32) return DSPARK_ERR_ARG;
    if (!rank_supported(wdtype, r)) return DSPARK_ERR_UNSUPPORTED;
    if (!aligned16(W1) || !aligned16(W2)) return DSPARK_ERR_ARG;
    return DSPARK_OK;
}

int draft_common(const float *U, const void *W1, const void *W2, int wdtype, const int32_t *anchor,
                 const float *temperature, int B, int gamma, int V, int r, uint64_t seed, uint64_t round_id,
                 const float *hidden, const float *conf_w, int d, const float *conf_tau, int32_t *x_out,
                 float *lse_out, float *qx_out, float *margin_out, float *conf_out, float *survival_out,
                 void *workspace, size_t workspace_bytes, void *stream) {
    const int st = draft_args(U, W1, W2, wdtype, anchor, temperature, B, gamma, V, r, x_out, lse_out, qx_out);
    if (st != DSPARK_OK) return st;
    const DraftPlan plan = draft_plan(B, V);
    size_t need = 0;
    draft_carve(nullptr, B, plan, &need);
    if (!workspace || workspace_bytes < need || !aligned16(workspace)) return DSPARK_ERR_WORKSPACE;
    const DraftWork w = draft_carve(workspace, B, plan, nullptr);
    DraftArgs a{};
    a.U = U;
    a.W1 = W1;
    a.W2 = W2;
    a.wdtype = wdtype;
    a.anchor = anchor;
    a.temperature = temperature;
    a.B = B;
    a.gamma = gamma;
    a.V = V;
    a.r = r;
    a.key0 = uint32_t(seed);
    a.key1 = uint32_t(seed >> 32);
    a.round32 = uint32_t(round_id);
    a.x_out = x_out;
    a.lse_out = lse_out;
    a.qx_out = qx_out;
    a.margin_out = margin_out;
    a.hidden = hidden;
    a.conf_w = conf_w;
    a.d = d;
    a.conf_tau = conf_tau;
    a.conf_out = conf_out;
    a.surv_out = survival_out;
    const hipError_t e = launch_draft(a, plan, w, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? DSPARK_OK : DSPARK_ERR_HIP;
}

}  // namespace

extern "C" {

int dspark_draft_sample(const float *U, const void *W1, const void *W2, int wdtype, const int32_t *anchor,
                        const float *temperature, int B, int gamma, int V, int r, uint64_t seed,
                        uint64_t round_id, int32_t *x_out, float *lse_out, float *qx_out, float *margin_out,
                        void *workspace, size_t workspace_bytes, void *stream) {
    return draft_common(U, W1, W2, wdtype, anchor, temperature, B, gamma, V, r, seed, round_id, nullptr, nullptr, 0,
                        nullptr, x_out, lse_out, qx_out, margin_out, nullptr, nullptr, workspace, workspace_bytes,
                        stream);
}

}  // extern "C"

namespace {

// The allocation-free entry point's scratch: a fixed array in the library's
// device code, so each device the library runs on holds its own copy from
// module load until the process ends.  Host code never uses the array's name
// as an address (it is a host-side stand-in); the device address comes from
// hipGetSymbolAddress, once per device with that device current, and is kept
// here.  The fast path is one atomic load; the first call on a device
// resolves the address under a lock.
static __device__ __align__(256) uint8_t scratch[DSPARK_NOALLOC_SCRATCH_BYTES];
constexpr int kScratchDevices = 256;
std::atomic<void *> scratch_addr[kScratchDevices];
std::mutex scratch_mu;

int scratch_for_current_device(void **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kScratchDevices) return DSPARK_ERR_HIP;
    void *p = scratch_addr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> g(scratch_mu);
        p = scratch_addr[dev].load(std::memory_order_relaxed);
        if (!p) {
            if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return DSPARK_ERR_HIP;
            scratch_addr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return DSPARK_OK;
}

}  // namespace

extern "C" {

int dspark_draft_sample_noalloc(const float *U, const void *W1, const void *W2, int wdtype, const int32_t *anchor,
                                const float *temperature, int B, int gamma, int V, int r, uint64_t seed,
                                uint64_t round_id, int32_t *x_out, float *lse_out, float *qx_out, float *margin_out,
                                void *stream) {
    const int st = draft_args(U, W1, W2, wdtype, anchor, temperature, B, gamma, V, r, x_out, lse_out, qx_out);
    if (st != DSPARK_OK) return st;
    if (draft_bytes(B, V) > DSPARK_NOALLOC_SCRATCH_BYTES) return DSPARK_ERR_SCRATCH;
    void *ws = nullptr;
    const int sc = scratch_for_current_device(&ws);
    if (sc != DSPARK_OK) return sc;
    // the draft's scratch needs no clearing: every partial is written before it is read
    return draft_common(U, W1, W2, wdtype, anchor, temperature, B, gamma, V, r, seed, round_id, nullptr, nullptr, 0,
                        nullptr, x_out, lse_out, qx_out, margin_out, nullptr, nullptr, ws,
                        DSPARK_NOALLOC_SCRATCH_BYTES, stream);
}

int dspark_draft_sample_confidence(const float *U, const void *W1, const void *W2, int wdtype,
                                   const int32_t *anchor, const float *temperature, int B, int gamma, int V, int r,
                                   uint64_t seed, uint64_t round_id, const float *hidden, const float *conf_w, int d,
                                   const float *conf_tau, int32_t *x_out, float *lse_out, float *qx_out,
                                   float *margin_out,
                                   float *conf_out, float *survival_out, void *workspace, size_t workspace_bytes,
                                   void *stream) {
    if (d < 0 || d > DSPARK_MAX_HIDDEN || (d > 0 && !hidden) || !conf_w || !conf_out || !survival_out)
        return DSPARK_ERR_ARG;
    return draft_common(U, W1, W2, wdtype, anchor, temperature, B, gamma, V, r, seed, round_id, hidden, conf_w, d,
                        conf_tau, x_out, lse_out, qx_out, margin_out, conf_out, survival_out, workspace,
                        workspace_bytes, stream);
}

size_t dspark_draft_rnn_workspace_size(int B, int gamma, int V, int r, int d) {
    if (!sizes_ok(B, gamma, V, r) || d < 0 || d > DSPARK_MAX_HIDDEN) return 0;
    const DraftPlan p = draft_plan(B, V);
    size_t bytes = 0;
    draft_carve(nullptr, B, p, &bytes, r, gamma, d);
    return bytes;
}

int dspark_draft_sample_rnn(const float *U, const void *W1, const void *W2, const void *Wgco, int wdtype,
                            const int32_t *anchor, const float *temperature, const float *hidden, int d, int B,
                            int gamma, int V, int r, uint64_t seed, uint64_t round_id, int32_t *x_out, float *lse_out,
                            float *qx_out, float *margin_out, void *e_out, float *state_out, void *workspace,
                            size_t workspace_bytes, void *stream) {
    if (!U || !W1 || !W2 || !Wgco || !anchor || !temperature || !x_out || !lse_out || !qx_out || !e_out)
        return DSPARK_ERR_ARG;
    if (!sizes_ok(B, gamma, V, r)) return DSPARK_ERR_ARG;
    if (wdtype != DSPARK_BF16 && wdtype != DSPARK_F32) return DSPARK_ERR_ARG;
    if (wdtype != DSPARK_BF16 || !rank_supported(wdtype, r)) return DSPARK_ERR_UNSUPPORTED;
    if (d < 0 || d > DSPARK_MAX_HIDDEN || (d > 0 && !hidden)) return DSPARK_ERR_ARG;
    if (d % 32 != 0) return DSPARK_ERR_UNSUPPORTED;
    if (!aligned16(W1) || !aligned16(W2) || !aligned16(Wgco) || !aligned16(e_out) || (d > 0 && !aligned16(hidden)))
        return DSPARK_ERR_ARG;
    const DraftPlan plan = draft_plan(B, V);
    size_t need = 0;
    draft_carve(nullptr, B, plan, &need, r, gamma, d);
    if (!workspace || workspace_bytes < need || !aligned16(workspace)) return DSPARK_ERR_WORKSPACE;
    const DraftWork w = draft_carve(workspace, B, plan, nullptr, r, gamma, d);
    DraftArgs a{};
    a.U = U;
    a.W1 = W1;
    a.W2 = W2;
    a.wdtype = wdtype;
    a.anchor = anchor;
    a.temperature = temperature;
    a.B = B;
    a.gamma = gamma;
    a.V = V;
    a.r = r;
    a.key0 = uint32_t(seed);
    a.key1 = uint32_t(seed >> 32);
    a.round32 = uint32_t(round_id);
    a.x_out = x_out;
    a.lse_out = lse_out;
    a.qx_out = qx_out;
    a.margin_out = margin_out;
    a.Wgco = Wgco;
    a.rnn_h = hidden;
    a.rnn_d = d;
    a.e_out = static_cast<uint16_t *>(e_out);
    a.state_out = state_out;
    const hipError_t e = launch_draft(a, plan, w, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? DSPARK_OK : DSPARK_ERR_HIP;
}

size_t dspark_sts_workspace_size(int N, int gamma, int G, int n_bins) {
    if (N < 1 || gamma < 1 || gamma > DSPARK_MAX_GAMMA || G < 1 || n_bins < 1 || G > DSPARK_MAX_STS_GRID ||
        G * n_bins > DSPARK_MAX_STS_CELLS)
        return 0;
    size_t bytes = 0;
    sts_carve(nullptr, N, gamma, G, n_bins, &bytes);
    return bytes;
}

int dspark_sts_fit(const float *c, const int32_t *n_accept, const int32_t *ell, int N, int gamma, const float *grid,
                   int G, int n_bins, float *tau_out, float *ece_out, float *ece_grid_out, void *workspace,
                   size_t workspace_bytes, void *stream) {
    if (!c || !n_accept || !grid || !tau_out || !ece_out) return DSPARK_ERR_ARG;
    if (N < 1 || N > DSPARK_MAX_STS_SAMPLES || gamma < 1 || gamma > DSPARK_MAX_GAMMA || G < 1 || n_bins < 1 ||
        G > DSPARK_MAX_STS_GRID || G * n_bins > DSPARK_MAX_STS_CELLS)
        return DSPARK_ERR_ARG;
    size_t need = 0;
    sts_carve(nullptr, N, gamma, G, n_bins, &need);
    if (!workspace || workspace_bytes < need || !aligned16(workspace)) return DSPARK_ERR_WORKSPACE;
    const StsWork w = sts_carve(workspace, N, gamma, G, n_bins, nullptr);
    StsArgs a{};
    a.c = c;
    a.n = n_accept;
    a.ell = ell;
    a.N = N;
    a.gamma = gamma;
    a.grid = grid;
    a.G = G;
    a.M = n_bins;
    a.tau_out = tau_out;
    a.ece_out = ece_out;
    a.ece_grid = ece_grid_out;
    const hipError_t e = launch_sts(a, sts_plan(N, gamma, G, n_bins), w, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? DSPARK_OK : DSPARK_ERR_HIP;
}

size_t dspark_verify_workspace_size(int B, int gamma, int V, int r) {
    if (!sizes_ok(B, gamma, V, r)) return 0;
    return verify_bytes(B, gamma, V);
}

static int verify_common(const float *target, int n_target_rows, const int32_t *ell, const int32_t *row_offsets,
                         const float *U, const void *W1, const void *W2, int wdtype, const int32_t *anchor,
                         const int32_t *x, const float *lse_q, const float *qx, const float *temperature, int B,
                         int gamma, int V, int r, uint64_t seed, uint64_t round_id, int32_t *n_accept_out,
                         int32_t *tokens_out, int32_t *out_offsets, float *diag_out, float *resid_out,
                         void *workspace, size_t workspace_bytes, void *stream, int erow_mode) {
    if (!target || !ell || !U || !W1 || !W2 || !anchor || !x || !lse_q || !qx || !temperature ||
        !n_accept_out || !tokens_out)
        return DSPARK_ERR_ARG;
    if (!sizes_ok(B, gamma, V, r) || n_target_rows < 1) return DSPARK_ERR_ARG;
    if (wdtype != DSPARK_BF16 && wdtype != DSPARK_F32) return DSPARK_ERR_ARG;
    if (!rank_supported(wdtype, r)) return DSPARK_ERR_UNSUPPORTED;
    if (!aligned16(W1) || !aligned16(W2)) return DSPARK_ERR_ARG;
    const VerifyPlan plan = verify_plan(B, gamma, V);
    size_t need = 0;
    verify_carve(nullptr, B, gamma, V, plan, &need);
    if (!workspace || workspace_bytes < need || !aligned16(workspace)) return DSPARK_ERR_WORKSPACE;
    const VerifyWork w = verify_carve(workspace, B, gamma, V, plan, nullptr);
    VerifyArgs a{};
    a.target = target;
    a.n_target_rows = n_target_rows;
    a.ell = ell;
    a.row_offsets = row_offsets;
    a.U = U;
    a.W1 = W1;
    a.W2 = W2;
    a.wdtype = wdtype;
    a.anchor = anchor;
    a.x = x;
    a.lse_q = lse_q;
    a.qx = qx;
    a.temperature = temperature;
    a.B = B;
    a.gamma = gamma;
    a.V = V;
    a.r = r;
    a.key0 = uint32_t(seed);
    a.key1 = uint32_t(seed >> 32);
    a.round32 = uint32_t(round_id);
    a.n_accept_out = n_accept_out;
    a.tokens_out = tokens_out;
    a.out_offsets = out_offsets;
    a.diag_out = diag_out;
    a.resid_out = resid_out;
    a.erow_mode = erow_mode;
    const hipError_t e = launch_verify(a, plan, w, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? DSPARK_OK : DSPARK_ERR_HIP;
}

int dspark_verify(const float *target, int n_target_rows, const int32_t *ell, const int32_t *row_offsets,
                  const float *U, const void *W1, const void *W2, int wdtype, const int32_t *anchor,
                  const int32_t *x, const float *lse_q, const float *qx, const float *temperature, int B,
                  int gamma, int V, int r, uint64_t seed, uint64_t round_id, int32_t *n_accept_out,
                  int32_t *tokens_out, int32_t *out_offsets, float *diag_out, float *resid_out,
                  void *workspace, size_t workspace_bytes, void *stream) {
    return verify_common(target, n_target_rows, ell, row_offsets, U, W1, W2, wdtype, anchor, x, lse_q, qx,
                         temperature, B, gamma, V, r, seed, round_id, n_accept_out, tokens_out, out_offsets, diag_out,
                         resid_out, workspace, workspace_bytes, stream, 0);
}

int dspark_verify_rnn(const float *target, int n_target_rows, const int32_t *ell, const int32_t *row_offsets,
                      const float *U, const void *head_rows, const void *W2, int wdtype, const int32_t *anchor,
                      const int32_t *x, const float *lse_q, const float *qx, const float *temperature, int B,
                      int gamma, int V, int r, uint64_t seed, uint64_t round_id, int32_t *n_accept_out,
                      int32_t *tokens_out, int32_t *out_offsets, float *diag_out, float *resid_out,
                      void *workspace, size_t workspace_bytes, void *stream) {
    return verify_common(target, n_target_rows, ell, row_offsets, U, head_rows, W2, wdtype, anchor, x, lse_q, qx,
                         temperature, B, gamma, V, r, seed, round_id, n_accept_out, tokens_out, out_offsets, diag_out,
                         resid_out, workspace, workspace_bytes, stream, 1);
}

size_t dspark_acceptance_workspace_size(int B, int gamma, int V, int r) {
    if (!sizes_ok(B, gamma, V, r)) return 0;
    return accept_bytes(B, gamma, V);
}

static int acceptance_common(const float *target, int n_target_rows, const int32_t *ell, const int32_t *row_offsets,
                             const float *U, const void *W1, const void *W2, int wdtype, const int32_t *anchor,
                             const int32_t *x, const float *lse_q, const float *temperature, int B, int gamma,
                             int V, int r, float *alpha_out, void *workspace, size_t workspace_bytes, void *stream,
                             int erow_mode) {
    if (!target || !ell || !U || !W1 || !W2 || !anchor || !x || !lse_q || !temperature || !alpha_out)
        return DSPARK_ERR_ARG;
    if (!sizes_ok(B, gamma, V, r) || n_target_rows < 1) return DSPARK_ERR_ARG;
    if (wdtype != DSPARK_BF16 && wdtype != DSPARK_F32) return DSPARK_ERR_ARG;
    if (!rank_supported(wdtype, r)) return DSPARK_ERR_UNSUPPORTED;
    if (!aligned16(W1) || !aligned16(W2)) return DSPARK_ERR_ARG;
    const AcceptPlan plan = accept_plan(B, gamma, V);
    size_t need = 0;
    accept_carve(nullptr, B, gamma, plan, &need);
    if (!workspace || workspace_bytes < need || !aligned16(workspace)) return DSPARK_ERR_WORKSPACE;
    const AcceptWork w = accept_carve(workspace, B, gamma, plan, nullptr);
    AcceptArgs a{};
    a.target = target;
    a.n_target_rows = n_target_rows;
    a.ell = ell;
    a.row_offsets = row_offsets;
    a.U = U;
    a.W1 = W1;
    a.W2 = W2;
    a.wdtype = wdtype;
    a.anchor = anchor;
    a.x = x;
    a.lse_q = lse_q;
    a.temperature = temperature;
    a.B = B;
    a.gamma = gamma;
    a.V = V;
    a.r = r;
    a.alpha_out = alpha_out;
    a.erow_mode = erow_mode;
    const hipError_t e = launch_accept(a, plan, w, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? DSPARK_OK : DSPARK_ERR_HIP;
}

int dspark_acceptance(const float *target, int n_target_rows, const int32_t *ell, const int32_t *row_offsets,
                      const float *U, const void *W1, const void *W2, int wdtype, const int32_t *anchor,
                      const int32_t *x, const float *lse_q, const float *temperature, int B, int gamma, int V,
                      int r, float *alpha_out, void *workspace, size_t workspace_bytes, void *stream) {
    return acceptance_common(target, n_target_rows, ell, row_offsets, U, W1, W2, wdtype, anchor, x, lse_q,
                             temperature, B, gamma, V, r, alpha_out, workspace, workspace_bytes, stream, 0);
}

int dspark_acceptance_rnn(const float *target, int n_target_rows, const int32_t *ell, const int32_t *row_offsets,
                          const float *U, const void *head_rows, const void *W2, int wdtype, const int32_t *anchor,
                          const int32_t *x, const float *lse_q, const float *temperature, int B, int gamma, int V,
                          int r, float *alpha_out, void *workspace, size_t workspace_bytes, void *stream) {
    return acceptance_common(target, n_target_rows, ell, row_offsets, U, head_rows, W2, wdtype, anchor, x, lse_q,
                             temperature, B, gamma, V, r, alpha_out, workspace, workspace_bytes, stream, 1);
}

int dspark_verify_check(const void *workspace, void *stream) {
    if (!workspace) return DSPARK_ERR_ARG;
    if (hipStreamSynchronize(static_cast<hipStream_t>(stream)) != hipSuccess) return DSPARK_ERR_HIP;
    int32_t st = 0;
    // the status word is the first region of the verify workspace
    if (hipMemcpy(&st, workspace, sizeof(st), hipMemcpyDeviceToHost) != hipSuccess) return DSPARK_ERR_HIP;
    return st == 0 ? DSPARK_OK : DSPARK_ERR_DEVICE_INPUT;
}

int dspark_debug_random_words(uint64_t seed, uint64_t round_id, int stream_id, int k, int req, int v0, int n,
                              uint32_t *out, void *stream) {
    if (!out || n < 0 || stream_id < 0 || stream_id > 4 || k < 0 || k >= (1 << 24) || v0 < 0) return DSPARK_ERR_ARG;
    const hipError_t e = launch_debug_words(uint32_t(seed), uint32_t(seed >> 32), uint32_t(round_id), stream_id,
                                            k, req, v0, n, out, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? DSPARK_OK : DSPARK_ERR_HIP;
}

int dspark_debug_bias_gemm(const void *W1, const void *W2, int wdtype, const int32_t *idx, int B, int V, int r,
                           float *rowmax_out, void *workspace, size_t workspace_bytes, void *stream) {
    if (!W1 || !W2 || !idx || !rowmax_out) return DSPARK_ERR_ARG;
    if (!sizes_ok(B, 1, V, r)) return DSPARK_ERR_ARG;
    if (wdtype != DSPARK_BF16 && wdtype != DSPARK_F32) return DSPARK_ERR_ARG;
    if (!rank_supported(wdtype, r)) return DSPARK_ERR_UNSUPPORTED;
    if (!aligned16(W1) || !aligned16(W2)) return DSPARK_ERR_ARG;
    const DraftPlan plan = draft_plan(B, V);
    size_t need = 0;
    draft_carve(nullptr, B, plan, &need);
    if (!workspace || workspace_bytes < need || !aligned16(workspace)) return DSPARK_ERR_WORKSPACE;
    const DraftWork w = draft_carve(workspace, B, plan, nullptr);
    const hipError_t e =
        launch_bias_gemm(W1, W2, wdtype, idx, B, V, r, plan, w, rowmax_out, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? DSPARK_OK : DSPARK_ERR_HIP;
}

int dspark_debug_gumbel(const uint32_t *words, int n, float *out, void *stream) {
    if (!words || !out || n < 0) return DSPARK_ERR_ARG;
    const hipError_t e = launch_debug_gumbel(words, n, out, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? DSPARK_OK : DSPARK_ERR_HIP;
}

int dspark_profile_enable(int enable) {
    Profiler &p = prof();
    std::lock_guard<std::mutex> g(p.mu);
    p.enabled = enable != 0;
    p.on.store(p.enabled, std::memory_order_release);
    return DSPARK_OK;
}

int dspark_profile_collect(void) {
    Profiler &p = prof();
    std::lock_guard<std::mutex> g(p.mu);
    int status = DSPARK_OK;
    for (const Pending &pd : p.pending) {
        float ms = 0.f;
        if (hipEventSynchronize(pd.stop) != hipSuccess || hipEventElapsedTime(&ms, pd.start, pd.stop) != hipSuccess) {
            status = DSPARK_ERR_HIP;
        } else {
            p.entries[size_t(pd.entry)].launches += 1;
            p.entries[size_t(pd.entry)].total_ms += ms;
        }
        p.pool.push_back(pd.start);
        p.pool.push_back(pd.stop);
    }
    p.pending.clear();
    return status;
}

int dspark_profile_count(void) {
    Profiler &p = prof();
    std::lock_guard<std::mutex> g(p.mu);
    return int(p.entries.size());
}

int dspark_profile_get(int i, const char **name, int64_t *launches, double *total_ms) {
    Profiler &p = prof();
    std::lock_guard<std::mutex> g(p.mu);
    if (i < 0 || i >= int(p.entries.size())) return DSPARK_ERR_ARG;
    if (name) *name = p.entries[size_t(i)].name.c_str();
    if (launches) *launches = p.entries[size_t(i)].launches;
    if (total_ms) *total_ms = p.entries[size_t(i)].total_ms;
    return DSPARK_OK;
}

int dspark_profile_reset(void) {
    Profiler &p = prof();
    std::lock_guard<std::mutex> g(p.mu);
    for (ProfEntry &e : p.entries) {
        e.launches = 0;
        e.total_ms = 0.0;
    }
    return DSPARK_OK;
}

}  // extern "C"
