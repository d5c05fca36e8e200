// Exact attention, plain fp64 CPU definition: the ORACLE.
//
// TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
// load this file: only the tests, the smoke check and the CPU-baseline leg
// of the benchmark use it.  It shares no code, header or constant with the
// HIP path.
//
// What it computes follows the FlashAttention-2 overview page
// (lshu.cn/news/55956), section 2.1 ("standard attention", first hardware
// anti-pattern): form the score row q_i . k_j, take the softmax of each row,
// then the weighted sum of the V rows.  The page states (section 1) that the
// tiled method reaches exactly this result, so the oracle is that definition
// written out, in double precision, from the same 16-bit input values the GPU
// sees (converted exactly to double by the caller).  Masking is exact: keys
// that are not visible are left out of the row (causal upper-triangular mask,
// same page, section 4.2 question 4; sliding window "window_size", install
// guide page yfxerp.com/news/195771, section 1).
//
// The backward uses the textbook gradient of softmax attention; the pages
// only say that the scores are recomputed (install guide page, section 1).
// For one row i with probabilities P_ij and upstream gradient dO_i:
//   dV_j += P_ij dO_i
//   dP_ij = dO_i . v_j
//   dS_ij = P_ij (dP_ij - sum_k P_ik dP_ik)          (softmax Jacobian)
//   dQ_i  = scale * sum_j dS_ij k_j
//   dK_j += scale * dS_ij q_i
//
// Dropout (the dropout_p argument of the attention call, overview page section
// 3.3; every call on the pages passes 0): each probability P_ij is kept with
// probability T/256 and scaled by 256/T, or dropped (set to 0), after the
// softmax and before the weighted sum; LSE stays that of the softmax.  The
// keep decision of element (sequence b, query head h, query row i, key j) is
// an 8-bit draw from the counter-based generator Philox4x32-10 (Salmon, Moraes,
// Dror, Shaw, "Parallel random numbers: as easy as 1, 2, 3", SC 2011):
//   counter = (j / 4, i / 4, h, b), key = (seed low 32 bits, seed high 32 bits),
//   u = byte (j mod 4) of output word (i mod 4), kept iff u < T,
//   T = floor((1 - dropout_p) * 256 + 1/2).
// With M_ij = kept / dropped (1 / 0) and s = 256 / T (0 when T = 0):
//   O_i = sum_j P_ij M_ij s v_j
//   dV_j += P_ij M_ij s dO_i,  dP_ij = dO_i . v_j,
//   dS_ij = P_ij (M_ij s dP_ij - D_i),  D_i = sum_k P_ik M_ik s dP_ik = dO_i . O_i
// (the gradient of O = (P o M s) V with P the softmax of the score row).
//
// Readings where the pages are silent (each also listed in the design notes):
//   * visible set of query row i in a sequence with Lq queries and Lk keys:
//     with p = i + (Lk - Lq) (bottom-right alignment), key j is visible iff
//     0 <= j < Lk, (not causal or j <= p), (left < 0 or j >= p - left) and
//     (right < 0 or j <= p + right);
//   * LSE_i = natural log of sum over visible j of exp(scale * q_i . k_j);
//   * a row with no visible key gets O_i = 0, LSE_i = -inf, dQ_i = 0;
//   * GQA: query head h reads kv head h / (heads / kv_heads).
//
// Layout: q, o, dout, dq are (batch, seqlen_q, heads, d) or, with cu_seqlens,
// packed (total_q, heads, d); k, v, dk, dv likewise with kv_heads.  LSE is
// (batch, heads, seqlen_q), or (heads, total_q) when packed.  All row-major
// with the head dimension contiguous.
//
// Parallel over rows (forward, phase 1 of the backward) and over key rows
// (phase 2 of the backward).  Every output element is written by exactly one
// task and every sum runs in a fixed order, so results are deterministic.

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <functional>
#include <limits>
#include <thread>
#include <vector>

namespace {

// Philox4x32-10 as published: ten rounds of
//   (c0, c1, c2, c3) -> (hi(M1 c2) ^ c1 ^ k0, lo(M1 c2), hi(M0 c0) ^ c3 ^ k1, lo(M0 c0))
// with the key bumped by the Weyl constants between rounds.
void philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2], uint32_t out[4]) {
    const uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u, W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
    uint32_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
    uint32_t k0 = key_in[0], k1 = key_in[1];
    for (int r = 0; r < 10; ++r) {
        if (r > 0) { k0 += W0; k1 += W1; }
        const uint64_t p0 = (uint64_t)M0 * c0, p1 = (uint64_t)M1 * c2;
        const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0, n1 = (uint32_t)p1;
        const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1, n3 = (uint32_t)p0;
        c0 = n0; c1 = n1; c2 = n2; c3 = n3;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

// The same construction on 64-bit words (Philox4x64-10), used only to check the
// round structure against an independent library implementation.
void philox4x64_10(const uint64_t ctr_in[4], const uint64_t key_in[2], uint64_t out[4]) {
    const uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
    const uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
    uint64_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
    uint64_t k0 = key_in[0], k1 = key_in[1];
    for (int r = 0; r < 10; ++r) {
        if (r > 0) { k0 += W0; k1 += W1; }
        const unsigned __int128 p0 = (unsigned __int128)M0 * c0, p1 = (unsigned __int128)M1 * c2;
        const uint64_t n0 = (uint64_t)(p1 >> 64) ^ c1 ^ k0, n1 = (uint64_t)p1;
        const uint64_t n2 = (uint64_t)(p0 >> 64) ^ c3 ^ k1, n3 = (uint64_t)p0;
        c0 = n0; c1 = n1; c2 = n2; c3 = n3;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

// Keep threshold T for a dropout probability p.
int dropout_threshold(double p) {
    double t = std::floor((1.0 - p) * 256.0 + 0.5);
    if (t < 0.0) t = 0.0;
    if (t > 256.0) t = 256.0;
    return (int)t;
}

struct Geometry {
    int batch, heads, kv_heads, seqlen_q, seqlen_k, d;
    int causal, left, right;
    double scale;
    const int32_t* cu_q;  // host pointers or null
    const int32_t* cu_k;
    int drop_t = 256;        // keep threshold (256: no dropout)
    uint64_t seed = 0;
    double drop_scale() const { return drop_t > 0 ? 256.0 / drop_t : 0.0; }
    // M_ij times the kept-value scale: s when kept, 0 when dropped
    double keep(int b, int h, int i, int j) const {
        if (drop_t >= 256) return 1.0;
        const uint32_t ctr[4] = {(uint32_t)j >> 2, (uint32_t)i >> 2, (uint32_t)h, (uint32_t)b};
        const uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
        uint32_t w[4];
        philox4x32_10(ctr, key, w);
        const uint32_t u = (w[i & 3] >> (8 * (j & 3))) & 0xffu;
        return (int)u < drop_t ? drop_scale() : 0.0;
    }
    bool packed() const { return cu_q != nullptr; }
    int64_t q_start(int b) const { return packed() ? cu_q[b] : (int64_t)b * seqlen_q; }
    int64_t k_start(int b) const { return packed() ? cu_k[b] : (int64_t)b * seqlen_k; }
    int len_q(int b) const { return packed() ? cu_q[b + 1] - cu_q[b] : seqlen_q; }
    int len_k(int b) const { return packed() ? cu_k[b + 1] - cu_k[b] : seqlen_k; }
    int64_t total_q() const { return packed() ? cu_q[batch] : (int64_t)batch * seqlen_q; }
    int group() const { return heads / kv_heads; }
    // element offsets
    int64_t qoff(int b, int i, int h) const { return ((q_start(b) + i) * heads + h) * (int64_t)d; }
    int64_t koff(int b, int j, int hk) const { return ((k_start(b) + j) * kv_heads + hk) * (int64_t)d; }
    int64_t lse_off(int b, int h, int i) const {
        return packed() ? (int64_t)h * total_q() + q_start(b) + i
                        : ((int64_t)b * heads + h) * seqlen_q + i;
    }
    bool visible(int b, int i, int j) const {
        const int lq = len_q(b), lk = len_k(b);
        if (j < 0 || j >= lk) return false;
        const long p = (long)i + (lk - lq);
        if (causal && j > p) return false;
        if (left >= 0 && j < p - left) return false;
        if (right >= 0 && j > p + right) return false;
        return true;
    }
};

double dot(const double* a, const double* b, int n) {
    double s = 0.0;
    for (int c = 0; c < n; ++c) s += a[c] * b[c];
    return s;
}

void run_tasks(int64_t ntasks, int nthreads, const std::function<void(int64_t)>& fn) {
    if (nthreads <= 0) nthreads = (int)std::thread::hardware_concurrency();
    if (nthreads <= 0) nthreads = 1;
    if (nthreads > ntasks) nthreads = (int)(ntasks > 0 ? ntasks : 1);
    std::atomic<int64_t> next{0};
    auto worker = [&]() {
        for (;;) {
            const int64_t t = next.fetch_add(1);
            if (t >= ntasks) return;
            fn(t);
        }
    };
    std::vector<std::thread> pool;
    for (int t = 1; t < nthreads; ++t) pool.emplace_back(worker);
    worker();
    for (auto& th : pool) th.join();
}

// One query row: the score row over visible keys, its softmax, O_i, LSE_i and,
// when dout is given, dQ_i and the row term D_i = sum_j P_ij dP_ij.
struct RowResult {
    double lse;
    double dsum;  // sum_j P_ij dP_ij (only with dout)
};

RowResult attend_row(const Geometry& g, const double* q, const double* k, const double* v,
                     const double* dout, int b, int h, int i,
                     double* o_row, double* dq_row, std::vector<double>& s,
                     std::vector<double>& dp) {
    const int d = g.d, lk = g.len_k(b), hk = h / g.group();
    const double* qi = q + g.qoff(b, i, h);
    s.assign(lk, 0.0);
    thread_local std::vector<double> km;  // M_ij s of the row (dropout)
    km.assign(lk, 1.0);
    std::vector<char> vis(lk, 0);
    // materialise the score row
    double m = -std::numeric_limits<double>::infinity();
    int nvis = 0;
    for (int j = 0; j < lk; ++j) {
        if (!g.visible(b, i, j)) continue;
        vis[j] = 1;
        ++nvis;
        km[j] = g.keep(b, h, i, j);
        s[j] = g.scale * dot(qi, k + g.koff(b, j, hk), d);
        if (s[j] > m) m = s[j];
    }
    RowResult r{-std::numeric_limits<double>::infinity(), 0.0};
    if (o_row) for (int c = 0; c < d; ++c) o_row[c] = 0.0;
    if (dq_row) for (int c = 0; c < d; ++c) dq_row[c] = 0.0;
    if (nvis == 0) return r;
    // softmax of the row: exp(s - max), normalised by the row sum
    double l = 0.0;
    for (int j = 0; j < lk; ++j) if (vis[j]) { s[j] = std::exp(s[j] - m); l += s[j]; }
    for (int j = 0; j < lk; ++j) if (vis[j]) s[j] /= l;  // s now holds P_ij
    r.lse = m + std::log(l);
    if (o_row) {
        for (int j = 0; j < lk; ++j) {
            if (!vis[j]) continue;
            const double* vj = v + g.koff(b, j, hk);
            for (int c = 0; c < d; ++c) o_row[c] += s[j] * km[j] * vj[c];
        }
    }
    if (dout) {
        const double* doi = dout + g.qoff(b, i, h);
        dp.assign(lk, 0.0);
        double dsum = 0.0;
        for (int j = 0; j < lk; ++j) {
            if (!vis[j]) continue;
            dp[j] = dot(doi, v + g.koff(b, j, hk), d);
            dsum += s[j] * km[j] * dp[j];
        }
        r.dsum = dsum;
        if (dq_row) {
            for (int j = 0; j < lk; ++j) {
                if (!vis[j]) continue;
                const double ds = s[j] * (km[j] * dp[j] - dsum);
                const double* kj = k + g.koff(b, j, hk);
                for (int c = 0; c < d; ++c) dq_row[c] += g.scale * ds * kj[c];
            }
        }
    }
    return r;
}

int check_args(const Geometry& g) {
    if (g.batch < 0 || g.heads <= 0 || g.kv_heads <= 0 || g.d <= 0) return 1;
    if (g.heads % g.kv_heads != 0) return 1;
    if (g.seqlen_q < 0 || g.seqlen_k < 0) return 1;
    if ((g.cu_q == nullptr) != (g.cu_k == nullptr)) return 1;
    return 0;
}

std::vector<char> selection(const int32_t* sel, int nsel, int n) {
    std::vector<char> on(n > 0 ? n : 0, sel ? 0 : 1);
    if (sel)
        for (int t = 0; t < nsel; ++t)
            if (sel[t] >= 0 && sel[t] < n) on[sel[t]] = 1;
    return on;
}

}  // namespace

extern "C" {

// Forward.  Writes O and LSE for the selected rows (row_sel: query row
// positions within each sequence, null = all) of the selected query heads
// (head_sel, null = all); other entries are left untouched.  Returns 0, or 1
// on bad arguments.
int oracle_attention_fwd(const double* q, const double* k, const double* v,
                         double* o, double* lse,
                         const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                         int batch, int heads, int kv_heads, int seqlen_q, int seqlen_k,
                         int head_dim, int causal, int window_left, int window_right,
                         double softmax_scale,
                         const int32_t* row_sel, int n_row_sel,
                         const int32_t* head_sel, int n_head_sel, int n_threads,
                         double dropout_p, uint64_t seed) {
    Geometry g{batch, heads, kv_heads, seqlen_q, seqlen_k, head_dim,
               causal, window_left, window_right, softmax_scale,
               cu_seqlens_q, cu_seqlens_k};
    if (!(dropout_p >= 0.0 && dropout_p < 1.0)) return 1;
    g.drop_t = dropout_threshold(dropout_p);
    g.seed = seed;
    if (check_args(g)) return 1;
    int maxq = 0;
    for (int b = 0; b < batch; ++b) maxq = std::max(maxq, g.len_q(b));
    const std::vector<char> rows_on = selection(row_sel, n_row_sel, maxq);
    const std::vector<char> heads_on = selection(head_sel, n_head_sel, heads);
    const int64_t ntasks = (int64_t)batch * heads * maxq;
    run_tasks(ntasks, n_threads, [&](int64_t t) {
        const int i = (int)(t % (maxq ? maxq : 1));
        const int h = (int)((t / (maxq ? maxq : 1)) % heads);
        const int b = (int)(t / ((int64_t)(maxq ? maxq : 1) * heads));
        if (!heads_on[h] || !rows_on[i] || i >= g.len_q(b)) return;
        thread_local std::vector<double> s, dp;
        const RowResult r = attend_row(g, q, k, v, nullptr, b, h, i,
                                       o + g.qoff(b, i, h), nullptr, s, dp);
        lse[g.lse_off(b, h, i)] = r.lse;
    });
    return 0;
}

// Backward.  Computes, from the same definition, dQ on the selected query
// rows (q_row_sel; null = all) and dK/dV on the selected key rows (k_row_sel;
// null = all), for the query heads of the selected kv heads (kv_head_sel;
// null = all).  o and lse (optional, may be null) receive the oracle's own
// forward outputs for every row the computation needed.  Entries outside the
// selection are left untouched.  Returns 0, or 1 on bad arguments.
int oracle_attention_bwd(const double* q, const double* k, const double* v,
                         const double* dout, double* dq, double* dk, double* dv,
                         double* o, double* lse,
                         const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                         int batch, int heads, int kv_heads, int seqlen_q, int seqlen_k,
                         int head_dim, int causal, int window_left, int window_right,
                         double softmax_scale,
                         const int32_t* q_row_sel, int n_q_row_sel,
                         const int32_t* k_row_sel, int n_k_row_sel,
                         const int32_t* kv_head_sel, int n_kv_head_sel, int n_threads,
                         double dropout_p, uint64_t seed) {
    Geometry g{batch, heads, kv_heads, seqlen_q, seqlen_k, head_dim,
               causal, window_left, window_right, softmax_scale,
               cu_seqlens_q, cu_seqlens_k};
    if (!(dropout_p >= 0.0 && dropout_p < 1.0)) return 1;
    g.drop_t = dropout_threshold(dropout_p);
    g.seed = seed;
    if (check_args(g)) return 1;
    const int d = head_dim, grp = g.group();
    int maxq = 0, maxk = 0;
    for (int b = 0; b < batch; ++b) {
        maxq = std::max(maxq, g.len_q(b));
        maxk = std::max(maxk, g.len_k(b));
    }
    const std::vector<char> qsel = selection(q_row_sel, n_q_row_sel, maxq);
    const std::vector<char> ksel = selection(k_row_sel, n_k_row_sel, maxk);
    const std::vector<char> kvh_on = selection(kv_head_sel, n_kv_head_sel, kv_heads);

    // Rows whose statistics are needed: selected dQ rows, and every row that
    // sees a selected key row.
    const int64_t nrows_all = (int64_t)batch * maxq;
    std::vector<int> klist;
    for (int j = 0; j < maxk; ++j) if (ksel[j]) klist.push_back(j);
    std::vector<char> need(nrows_all, 0);
    run_tasks(batch, n_threads, [&](int64_t b) {
        const int lq = g.len_q((int)b);
        for (int i = 0; i < lq; ++i) {
            bool n = qsel[i] != 0;
            for (size_t t = 0; t < klist.size() && !n; ++t) n = g.visible((int)b, i, klist[t]);
            need[b * maxq + i] = n;
        }
    });

    // Phase 1, row by row: LSE_i and D_i = sum_j P_ij dP_ij, plus dQ_i.
    std::vector<double> row_lse((size_t)batch * heads * maxq, 0.0);
    std::vector<double> row_dsum((size_t)batch * heads * maxq, 0.0);
    const int64_t n1 = (int64_t)batch * heads * maxq;
    run_tasks(n1, n_threads, [&](int64_t t) {
        const int i = (int)(t % maxq);
        const int h = (int)((t / maxq) % heads);
        const int b = (int)(t / ((int64_t)maxq * heads));
        if (!kvh_on[h / grp] || i >= g.len_q(b) || !need[(int64_t)b * maxq + i]) return;
        thread_local std::vector<double> s, dp, orow;
        orow.assign(d, 0.0);
        double* dq_row = qsel[i] ? dq + g.qoff(b, i, h) : nullptr;
        const RowResult r = attend_row(g, q, k, v, dout, b, h, i, orow.data(), dq_row, s, dp);
        row_lse[t] = r.lse;
        row_dsum[t] = r.dsum;
        if (o) std::memcpy(o + g.qoff(b, i, h), orow.data(), sizeof(double) * d);
        if (lse) lse[g.lse_off(b, h, i)] = r.lse;
    });

    // Phase 2, key row by key row: dK_j and dV_j summed over every query row
    // of every query head in the kv head's group that sees key j.
    const int64_t n2 = (int64_t)batch * kv_heads * maxk;
    run_tasks(n2, n_threads, [&](int64_t t) {
        const int j = (int)(t % maxk);
        const int hk = (int)((t / maxk) % kv_heads);
        const int b = (int)(t / ((int64_t)maxk * kv_heads));
        if (!kvh_on[hk] || !ksel[j] || j >= g.len_k(b)) return;
        double* dkj = dk + g.koff(b, j, hk);
        double* dvj = dv + g.koff(b, j, hk);
        for (int c = 0; c < d; ++c) dkj[c] = dvj[c] = 0.0;
        const double* kj = k + g.koff(b, j, hk);
        const double* vj = v + g.koff(b, j, hk);
        for (int h = hk * grp; h < (hk + 1) * grp; ++h) {
            for (int i = 0; i < g.len_q(b); ++i) {
                if (!g.visible(b, i, j)) continue;
                const int64_t ri = ((int64_t)b * heads + h) * maxq + i;
                const double* qi = q + g.qoff(b, i, h);
                const double* doi = dout + g.qoff(b, i, h);
                const double p = std::exp(g.scale * dot(qi, kj, d) - row_lse[ri]);
                const double dpij = dot(doi, vj, d);
                const double km = g.keep(b, h, i, j);
                const double ds = p * (km * dpij - row_dsum[ri]);
                for (int c = 0; c < d; ++c) {
                    dvj[c] += p * km * doi[c];
                    dkj[c] += g.scale * ds * qi[c];
                }
            }
        }
    });
    return 0;
}

// The generators and the dropout decision, exposed for their pins.
void oracle_philox4x32_10(const uint32_t* ctr, const uint32_t* key, uint32_t* out) {
    philox4x32_10(ctr, key, out);
}
void oracle_philox4x64_10(const uint64_t* ctr, const uint64_t* key, uint64_t* out) {
    philox4x64_10(ctr, key, out);
}
int oracle_dropout_threshold(double p) { return dropout_threshold(p); }

// keep[((b * heads + h) * lq + i) * lk + j] = 1 if element (b, h, i, j) is kept.
void oracle_dropout_mask(int batch, int heads, int lq, int lk, double dropout_p, uint64_t seed,
                         uint8_t* keep) {
    Geometry g{batch, heads, heads, lq, lk, 1, 0, -1, -1, 1.0, nullptr, nullptr};
    g.drop_t = dropout_threshold(dropout_p);
    g.seed = seed;
    for (int b = 0; b < batch; ++b)
        for (int h = 0; h < heads; ++h)
            for (int i = 0; i < lq; ++i)
                for (int j = 0; j < lk; ++j)
                    keep[(((int64_t)b * heads + h) * lq + i) * lk + j] = g.keep(b, h, i, j) != 0.0;
}

}  // extern "C"
