// schedule.cpp -- host-side confidence-scheduled prefix scheduler.
//
// Method (page "DSpark：DeepSeek 线上跑的投机解码..." (marsggbo.github.io),
// section 4.3 Hardware-Aware Prefix Scheduler; "DeepSeek DSpark explained"
// (share.concentrate1.com), section 04): the prefix survival
// a_{r,j} = c_{r,1} ... c_{r,j} of every (request, position) candidate, the
// candidates visited in descending a, each one extending its request's
// verify length when it is the next position of that request; B counts the
// target positions sum_r (1 + ell_r), tau the expected emitted tokens
// sum_r (1 + sum_{j<=ell_r} a_{r,j}), and the visit stops at the first
// candidate that does not raise Theta = tau * SPS(B).
//
// Because every a_{r,.} is non-increasing in j (c in [0, 1]), each request's
// candidates already come sorted, so the descending order is a k-way merge of
// R sorted lists: a binary heap holding each request's next candidate yields
// the same sequence as sorting all R * gamma candidates by (-a, r, j), in
// O(steps * log R) instead of O(R gamma log(R gamma)), and stops as soon as
// Theta stops improving.
#include <cmath>
#include <cstdint>
#include <queue>
#include <vector>

#include "dspark.h"

namespace {

struct Head {
    double a;
    int r;
};

struct HeadLess {  // priority: larger a first, then lower request index
    bool operator()(const Head &x, const Head &y) const {
        if (x.a != y.a) return x.a < y.a;
        return x.r > y.r;
    }
};

inline double sps_at(const double *sps, int sps_len, long long B) {
    return (B >= 0 && B < sps_len) ? sps[B] : 0.0;
}

}  // namespace

extern "C" int dspark_schedule(const double *c, int R, int gamma, const double *sps, int sps_len,
                               int32_t *ell_out, double *theta_out, double *tau_out, int32_t *B_out) {
    if (R < 0 || R > DSPARK_MAX_BATCH || gamma < 1 || gamma > DSPARK_MAX_GAMMA) return DSPARK_ERR_ARG;
    if (R > 0 && (!c || !ell_out)) return DSPARK_ERR_ARG;
    if (!sps || sps_len <= R) return DSPARK_ERR_ARG;
    const size_t n = size_t(R) * size_t(gamma);
    for (size_t i = 0; i < n; ++i)
        if (!(c[i] >= 0.0 && c[i] <= 1.0)) return DSPARK_ERR_ARG;  // also rejects NaN

    // prefix survival products, left to right
    std::vector<double> a(n);
    for (int r = 0; r < R; ++r) {
        double p = 1.0;
        for (int j = 0; j < gamma; ++j) {
            p *= c[size_t(r) * gamma + j];
            a[size_t(r) * gamma + j] = p;
        }
    }
    std::vector<int32_t> len(size_t(R), 0);
    std::priority_queue<Head, std::vector<Head>, HeadLess> heap;
    for (int r = 0; r < R; ++r)
        if (a[size_t(r) * gamma] > 0.0) heap.push(Head{a[size_t(r) * gamma], r});

    long long B = R;
    double tau = double(R);
    double best_theta = tau * sps_at(sps, sps_len, B);
    while (!heap.empty()) {
        const Head h = heap.top();
        const long long B1 = B + 1;
        const double tau1 = tau + h.a;
        const double theta = tau1 * sps_at(sps, sps_len, B1);
        if (!(theta > best_theta)) break;  // first non-improving step ends the search
        heap.pop();
        best_theta = theta;
        B = B1;
        tau = tau1;
        const int j = ++len[size_t(h.r)];
        if (j < gamma) {
            const double an = a[size_t(h.r) * gamma + j];
            if (an > 0.0) heap.push(Head{an, h.r});
        }
    }
    for (int r = 0; r < R; ++r) ell_out[r] = len[size_t(r)];
    if (theta_out) *theta_out = best_theta;
    if (tau_out) *tau_out = tau;
    if (B_out) *B_out = int32_t(B);
    return DSPARK_OK;
}

// Production-style scheduling ("DeepSeek DSpark explained", section 04, the
// strict implementation): the step's capacity comes from the previous two
// steps' predictions, and the current candidates only fill it, in the same
// descending-a order as above, with no early stop on the current step.
extern "C" int dspark_history_capacity(const int32_t *B_hist, const int32_t *R_hist, int n_hist, int R, int gamma,
                                       int64_t *capacity_out) {
    if (R < 0 || R > DSPARK_MAX_BATCH || gamma < 1 || gamma > DSPARK_MAX_GAMMA || n_hist < 0 || !capacity_out)
        return DSPARK_ERR_ARG;
    if (n_hist > 0 && (!B_hist || !R_hist)) return DSPARK_ERR_ARG;
    double sum = 0.0;
    int used = 0;
    for (int i = 0; i < n_hist && i < 2; ++i) {
        if (R_hist[i] <= 0) continue;
        sum += double(B_hist[i]) / double(R_hist[i]);
        ++used;
    }
    const int64_t hi = int64_t(R) * (1 + gamma);
    int64_t cap = hi;
    if (used > 0) {
        cap = int64_t(std::floor(double(R) * (sum / used) + 0.5));
        cap = cap < R ? R : (cap > hi ? hi : cap);
    }
    *capacity_out = cap;
    return DSPARK_OK;
}

extern "C" int dspark_schedule_capacity(const double *c, int R, int gamma, int64_t capacity, int32_t *ell_out,
                                        double *tau_out, int32_t *B_out) {
    if (R < 0 || R > DSPARK_MAX_BATCH || gamma < 1 || gamma > DSPARK_MAX_GAMMA) return DSPARK_ERR_ARG;
    if (R > 0 && (!c || !ell_out)) return DSPARK_ERR_ARG;
    const size_t n = size_t(R) * size_t(gamma);
    for (size_t i = 0; i < n; ++i)
        if (!(c[i] >= 0.0 && c[i] <= 1.0)) return DSPARK_ERR_ARG;
    std::vector<double> a(n);
    for (int r = 0; r < R; ++r) {
        double p = 1.0;
        for (int j = 0; j < gamma; ++j) {
            p *= c[size_t(r) * gamma + j];
            a[size_t(r) * gamma + j] = p;
        }
    }
    std::vector<int32_t> len(size_t(R), 0);
    std::priority_queue<Head, std::vector<Head>, HeadLess> heap;
    for (int r = 0; r < R; ++r)
        if (a[size_t(r) * gamma] > 0.0) heap.push(Head{a[size_t(r) * gamma], r});
    long long B = R;
    double tau = double(R);
    while (!heap.empty() && B < capacity) {
        const Head h = heap.top();
        heap.pop();
        B += 1;
        tau += h.a;
        const int j = ++len[size_t(h.r)];
        if (j < gamma) {
            const double an = a[size_t(h.r) * gamma + j];
            if (an > 0.0) heap.push(Head{an, h.r});
        }
    }
    for (int r = 0; r < R; ++r) ell_out[r] = len[size_t(r)];
    if (tau_out) *tau_out = tau;
    if (B_out) *B_out = int32_t(B);
    return DSPARK_OK;
}
