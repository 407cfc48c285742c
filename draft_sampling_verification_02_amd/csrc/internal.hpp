// internal.hpp -- declarations shared by the host entry points (api.cpp) and
// the kernel translation units (draft.hip, verify.hip, debug.hip).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace dspark {

// Per-launch profiling (api.cpp): while profiling is on, prof_events hands out
// a start / stop event pair filed under `name`, which the launch below passes
// to hipExtLaunchKernel so that the events carry the kernel's own start and
// end; while it is off both are null.
struct ProfEvents {
    hipEvent_t start = nullptr, stop = nullptr;
};
ProfEvents prof_events(const char *name);

// Launches kernel<<<grid, block, 0, s>>>(args...) (timed when profiling is on).
template <typename F, typename... Args>
inline void launch_kernel(const char *name, F kernel, dim3 grid, dim3 block, hipStream_t s, Args... args) {
    const ProfEvents ev = prof_events(name);
    hipExtLaunchKernelGGL(kernel, grid, block, 0, s, ev.start, ev.stop, 0, args...);
}

// Bump allocator over the caller's workspace: every region 256-byte aligned.
struct Carve {
    char *base;
    size_t off = 0;
    explicit Carve(void *p) : base(static_cast<char *>(p)) {}
    template <typename T>
    T *take(size_t n) {
        off = (off + 255) & ~size_t(255);
        T *p = reinterpret_cast<T *>(base ? base + off : nullptr);
        off += n * sizeof(T);
        return p;
    }
};

// ---- draft -----------------------------------------------------------

// Vocabulary walk of the MFMA tile kernels: a workgroup of `nw` waves (one
// 32-row block of requests each) streams the W2 tiles of one vocabulary chunk
// through LDS; `nbg` workgroups cover the request blocks of a chunk.
struct DraftPlan {
    int nbb;              // request blocks of 32 rows
    int nw;               // waves per workgroup
    int nbg;              // workgroups per vocabulary chunk = ceil(nbb / nw)
    int ntiles;           // 32-entry vocabulary tiles
    int tiles_per_chunk;  // tiles one workgroup walks
    int nchunk;           // vocabulary chunks = ceil(ntiles / tiles_per_chunk)
    int blocks;           // workgroups = nchunk * nbg
};
DraftPlan draft_plan(int B, int V);
// Walk of up to nw_max waves per workgroup, sized for about target_blocks
// workgroups; tiles_per_chunk is a multiple of `align`.
DraftPlan tile_walk_plan(int B, int V, int nw_max, long long target_blocks, int align);

struct DraftWork {
    float *pm, *ps, *pb, *p2;  // [B, nchunk] partial max, sum, best score, second score
    int32_t *pi;               // [B, nchunk] partial best index
    float *rnn_s[2];           // RNN head: [B, r] states of alternate positions
    int32_t *rnn_idx;          // RNN head: [B] the draft step's row of e_out for request b (b * gamma)
    float *rnn_yh;             // RNN head: precomputed h part of the gate product (RnnProjPlan)
    uint4 *ep;                 // [nbb, 32 rows of at most 512 bytes] packed E rows for the next position's step
};
// rnn_r > 0 also carves the RNN head's buffers for rank rnn_r, block gamma
// and width rnn_d.
DraftWork draft_carve(void *ws, int B, const DraftPlan &p, size_t *bytes, int rnn_r = 0, int rnn_gamma = 0,
                      int rnn_d = 0);

struct DraftArgs {
    const float *U;
    const void *W1, *W2;
    int wdtype;
    const int32_t *anchor;
    const float *temperature;
    int B, gamma, V, r;
    uint32_t key0, key1, round32;
    int32_t *x_out;
    float *lse_out, *qx_out, *margin_out;
    // confidence head; conf_out == nullptr: not evaluated
    const float *hidden;  // [B, gamma, d]
    const float *conf_w;  // [d + r]
    int d;
    const float *conf_tau;       // [gamma] temperatures of the head's logits, or nullptr (1)
    float *conf_out, *surv_out;  // [B, gamma] c_k and a_k
    // RNN head (bf16 weights only); Wgco == nullptr: the Markov head
    const void *Wgco;      // [3r, 2r + rnn_d]
    const float *rnn_h;    // [B, gamma, rnn_d]
    int rnn_d;
    uint16_t *e_out;       // [B, gamma, r] the rows e_k fed to the W2 product
    float *state_out;      // [B, r] s_gamma, or nullptr
};

// One position of the RNN head: s_out, e_out from s_in (nullptr: s_0 = 0),
// x_{k-1}, h_k, W1 and Wgco.
struct RnnGateArgs {
    const float *s_in;
    float *s_out;
    const int32_t *xprev;
    int xprev_stride;
    const float *h;
    size_t h_stride;
    const uint16_t *W1, *Wgco;
    uint16_t *e_out;
    size_t e_stride;
    int32_t *idx_out;
    int gamma, B, V, r, d;
    const float *yh;  // precomputed h part [yS, B * gamma, 3r], or nullptr
    size_t yh_split;
    int yS, kpos;     // its splits; k - 1
};
hipError_t launch_rnn_gate(const RnnGateArgs &a, hipStream_t s);

// The h part of the RNN head's gate product for every position at once;
// S == 0: not used (d == 0, or the partials would exceed 512 MiB).
struct RnnProjPlan {
    int S, kchunk, blocks;
    size_t floats;  // S * B * gamma * 3r
};
RnnProjPlan rnn_proj_plan(int B, int gamma, int r, int d);
hipError_t launch_rnn_hproj(const float *h, const uint16_t *Wgco, float *y, int B, int gamma, int r, int d,
                            const RnnProjPlan &p, hipStream_t s);
hipError_t launch_draft(const DraftArgs &a, const DraftPlan &p, const DraftWork &w, hipStream_t s);
// The bias product alone: rowmax[b] = max_v W1[idx[b]] . W2[v] (diagnostic).
hipError_t launch_bias_gemm(const void *W1, const void *W2, int wdtype, const int32_t *idx, int B, int V, int r,
                            const DraftPlan &p, const DraftWork &w, float *rowmax, hipStream_t s);

// ---- verify ----------------------------------------------------------

struct VerifyPlan {
    bool walk;                      // a workgroup a request walks its rows (else the position passes)
    int tail_from;                  // walk: rows from this one on read by the tail kernel (0: none)
    int nseg_first, seg_len_first;  // passes: segments of a target row in the first pass, entries each
    int nseg, seg_len;              // the same for the later passes (entries a multiple of 4)
    int nseg_max;                   // partials kept per request (at most 64 / rows a pass)
    int nbb;          // ceil(B / 32)
    DraftPlan tile;   // vocabulary walk of the resample / bonus draw
    int draw_nw;      // waves per workgroup of the draw
    int draw_nbg;     // workgroups per chunk of the draw (room for both lists)
    int draw_blocks;  // workgroups of the draw kernel
};
VerifyPlan verify_plan(int B, int gamma, int V);

struct VerifyWork {
    int32_t *status;     // [4] word 0: OR of the requests' input flags
    int32_t *req_flags;  // [B] the status flags each request's inputs raise
    int32_t *off;        // [B + 1] packed row offsets in use
    // position passes only, double buffered by pass parity (pass p reads the
    // half pass p - 1 wrote), one slot per row a pass reduces
    int32_t *act;        // [2, B] 1: the request's rows of that pass were reduced
    float *seg_m, *seg_s, *seg_v;  // [2, rows, B, nseg] per-segment max, sum of 2^(z - max), best value
    int32_t *seg_i;      // [2, rows, B, nseg] per-segment lowest-index argmax
    float *seg_tx;       // [2, rows, B] t(x_j) / T in log2 units for the accept test
    // walk tail only: the requests it takes, its row statistics
    int32_t *tail_flag, *tail_cnt;  // [B] 1: in the tail; rows reduced so far
    float *tail_lse2, *tail_tx;     // [B, gamma + 2 - tail_from] row logsumexp, t(x_j) / T (log2 units)
    int32_t *tail_amax;             // [B, gamma + 2 - tail_from] row argmax
    float *fin_lse2;     // [B] logsumexp (log2 units) of the row the draw uses
    int32_t *prev;       // [B] x_{j-1} of a residual draw at position j (the anchor for j = 1)
    float *lse2q;        // [B] log2-unit logsumexp of q_j for a residual draw
    int32_t *mode;       // [B] 0 done, 1 residual draw, 2 bonus draw, -1 invalid
    int32_t *jpos;       // [B] position of the emitted non-draft token
    // draw partials per (request, vocabulary chunk)
    float *dw_sum;       // residual mass
    float *dw_bl;        // best tile score of the level-1 race
    int32_t *dw_bt;      // its tile
};
VerifyWork verify_carve(void *ws, int B, int gamma, int V, const VerifyPlan &p, size_t *bytes);

struct VerifyArgs {
    const float *target;
    int n_target_rows;
    const int32_t *ell, *row_offsets;
    const float *U;
    const void *W1, *W2;
    int wdtype;
    const int32_t *anchor, *x;
    const float *lse_q, *qx, *temperature;
    int B, gamma, V, r;
    uint32_t key0, key1, round32;
    int32_t *n_accept_out, *tokens_out, *out_offsets;
    float *diag_out, *resid_out;
    int erow_mode;  // 0: q_k from W1[x_{k-1}]; 1: W1 holds the head's rows [B, gamma, r]
};
hipError_t launch_verify(const VerifyArgs &a, const VerifyPlan &p, const VerifyWork &w, hipStream_t s);

// ---- acceptance probability ------------------------------------------

struct AcceptPlan {
    int maxent;         // listed rows at most: B * gamma
    int nseg, seg_len;  // segments of a target row in the row statistics, entries each
    DraftPlan tile;     // vocabulary walk of the accepted-mass kernel
};
AcceptPlan accept_plan(int B, int gamma, int V);

struct AcceptWork {
    int32_t *count;                        // [4] sampled rows, greedy rows
    int32_t *ent_rho, *ent_trow, *ent_prev;  // [maxent] listed rows: b * gamma + k - 1, target row, x_{k-1}
    float *rs_m, *rs_s, *rs_v;             // [maxent, nseg] row statistics per segment
    int32_t *rs_i;
    float *mass;                           // [maxent, nchunk] sum of min(p, q) per chunk
};
AcceptWork accept_carve(void *ws, int B, int gamma, const AcceptPlan &p, size_t *bytes);

struct AcceptArgs {
    const float *target;
    int n_target_rows;
    const int32_t *ell, *row_offsets;
    const float *U;
    const void *W1, *W2;
    int wdtype;
    const int32_t *anchor, *x;
    const float *lse_q, *temperature;
    int B, gamma, V, r;
    float *alpha_out;
    int erow_mode;  // as for VerifyArgs
};
hipError_t launch_accept(const AcceptArgs &a, const AcceptPlan &p, const AcceptWork &w, hipStream_t s);

// ---- sequential temperature scaling ------------------------------------

struct StsPlan {
    int blocks;   // histogram workgroups: one per 256 samples
    size_t lds;   // dynamic LDS of a histogram workgroup
};
StsPlan sts_plan(int N, int gamma, int G, int M);

struct StsWork {
    float *a;                   // [N] calibrated prefix survival of each sample
    unsigned long long *acc_p;  // [gamma, G, M] sum of a' in 2^-32 fixed point
    uint32_t *acc_y;            // [gamma, G, M] outcome counts
    uint32_t *acc_n;            // [gamma] samples that verified each position
};
StsWork sts_carve(void *ws, int N, int gamma, int G, int M, size_t *bytes);

struct StsArgs {
    const float *c;
    const int32_t *n, *ell;
    int N, gamma;
    const float *grid;
    int G, M;
    float *tau_out, *ece_out, *ece_grid;
};
hipError_t launch_sts(const StsArgs &a, const StsPlan &p, const StsWork &w, hipStream_t s);

// ---- diagnostics -----------------------------------------------------

hipError_t launch_debug_words(uint32_t key0, uint32_t key1, uint32_t round32, int stream_id, int k,
                              int req, int v0, int n, uint32_t *out, hipStream_t s);
hipError_t launch_debug_gumbel(const uint32_t *words, int n, float *out, hipStream_t s);

}  // namespace dspark
