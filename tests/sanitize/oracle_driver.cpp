// Runs the fp64 oracle's entry points on small problems with exactly sized
// heap buffers, under ASan/UBSan: fixed and packed layouts (empty sequences
// included), masks, GQA, dropout, and row / head selections.  Checks that
// every finite output is finite and that selections leave the rest untouched.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <random>
#include <vector>

extern "C" {
int oracle_attention_fwd(const double*, const double*, const double*, double*, double*, const int32_t*,
                         const int32_t*, int, int, int, int, int, int, int, int, int, double, const int32_t*, int,
                         const int32_t*, int, int, double, uint64_t);
int oracle_attention_bwd(const double*, const double*, const double*, const double*, double*, double*, double*,
                         double*, double*, const int32_t*, const int32_t*, int, int, int, int, int, int, int, int,
                         int, double, const int32_t*, int, const int32_t*, int, const int32_t*, int, int, double,
                         uint64_t);
void oracle_dropout_mask(int, int, int, int, double, uint64_t, uint8_t*);
int oracle_dropout_threshold(double);
}

static int fails = 0;
static void check(bool ok, const char* what, int cfg) {
    if (!ok) {
        std::printf("FAIL config %d: %s\n", cfg, what);
        ++fails;
    }
}

int main() {
    std::mt19937_64 rng(12345);
    std::normal_distribution<double> nd(0.0, 1.0);
    struct Cfg { int batch, heads, kv, lq, lk, d, causal, left, right; double p; bool varlen; };
    const Cfg cfgs[] = {
        {2, 4, 2, 17, 17, 8, 1, -1, -1, 0.0, false}, {1, 2, 1, 5, 9, 16, 1, 3, 0, 0.0, false},
        {3, 3, 3, 9, 4, 8, 0, 2, 1, 0.3, false},     {0, 2, 2, 0, 0, 8, 1, -1, -1, 0.0, true},
        {4, 6, 2, 0, 0, 24, 1, 5, 0, 0.5, true},      {2, 2, 1, 1, 1, 8, 0, -1, -1, 0.0, false},
    };
    int ci = 0;
    for (const Cfg& c : cfgs) {
        ++ci;
        std::vector<int32_t> cu{0};
        int batch = c.batch, lq = c.lq, lk = c.lk;
        if (c.varlen) {  // packed: lengths 0, 1, 7, 12 ... (an empty sequence included)
            const int lens[] = {0, 7, 1, 12};
            batch = 4;
            for (int b = 0; b < batch; ++b) cu.push_back(cu.back() + lens[b]);
            lq = lk = 12;
        }
        const int64_t tq = c.varlen ? cu.back() : (int64_t)batch * lq;
        const int64_t tk = c.varlen ? cu.back() : (int64_t)batch * lk;
        std::vector<double> q(tq * c.heads * c.d), k(tk * c.kv * c.d), v(k.size()), dout(q.size());
        for (auto* t : {&q, &k, &v, &dout})
            for (double& x : *t) x = nd(rng);
        const double nan = std::nan("");
        std::vector<double> o(q.size(), nan), lse(tq * c.heads, nan);
        const int32_t* cup = c.varlen ? cu.data() : nullptr;
        check(oracle_attention_fwd(q.data(), k.data(), v.data(), o.data(), lse.data(), cup, cup, batch, c.heads,
                                   c.kv, lq, lk, c.d, c.causal, c.left, c.right, 0.35, nullptr, 0, nullptr, 0, 2,
                                   c.p, 99) == 0, "fwd status", ci);
        for (double x : o) check(std::isfinite(x), "O finite", ci);
        std::vector<double> dq(q.size(), nan), dk(k.size(), nan), dv(v.size(), nan), o2(q.size(), nan),
            lse2(lse.size(), nan);
        check(oracle_attention_bwd(q.data(), k.data(), v.data(), dout.data(), dq.data(), dk.data(), dv.data(),
                                   o2.data(), lse2.data(), cup, cup, batch, c.heads, c.kv, lq, lk, c.d, c.causal,
                                   c.left, c.right, 0.35, nullptr, 0, nullptr, 0, nullptr, 0, 3, c.p, 99) == 0,
              "bwd status", ci);
        for (double x : dq) check(std::isfinite(x), "dQ finite", ci);
        for (double x : dk) check(std::isfinite(x), "dK finite", ci);
        // selections: one row, one head, one kv head; the rest stays NaN
        if (lq > 1 && c.heads > 1) {
            const int32_t row = 1, head = c.heads - 1, kvh = 0;
            std::vector<double> os(q.size(), nan), ls(lse.size(), nan);
            check(oracle_attention_fwd(q.data(), k.data(), v.data(), os.data(), ls.data(), cup, cup, batch, c.heads,
                                       c.kv, lq, lk, c.d, c.causal, c.left, c.right, 0.35, &row, 1, &head, 1, 1, c.p,
                                       99) == 0, "fwd selection status", ci);
            size_t untouched = 0;
            for (double x : os) untouched += std::isnan(x);
            check(untouched > 0 && untouched < os.size() + 1, "fwd selection leaves the rest", ci);
            std::vector<double> dqs(q.size(), nan), dks(k.size(), nan), dvs(v.size(), nan);
            check(oracle_attention_bwd(q.data(), k.data(), v.data(), dout.data(), dqs.data(), dks.data(), dvs.data(),
                                       nullptr, nullptr, cup, cup, batch, c.heads, c.kv, lq, lk, c.d, c.causal,
                                       c.left, c.right, 0.35, &row, 1, &row, 1, &kvh, 1, 1, c.p, 99) == 0,
                  "bwd selection status", ci);
        }
        // bad arguments are refused, not read
        check(oracle_attention_fwd(q.data(), k.data(), v.data(), o.data(), lse.data(), cup, cup, batch, 3, 2, lq, lk,
                                   c.d, 0, -1, -1, 0.35, nullptr, 0, nullptr, 0, 1, 0.0, 0) == 1, "heads % kv", ci);
        check(oracle_attention_fwd(q.data(), k.data(), v.data(), o.data(), lse.data(), cup, cup, batch, c.heads, c.kv,
                                   lq, lk, c.d, 0, -1, -1, 0.35, nullptr, 0, nullptr, 0, 1, 1.0, 0) == 1, "p = 1", ci);
    }
    std::vector<uint8_t> m(2 * 3 * 33 * 47);
    oracle_dropout_mask(2, 3, 33, 47, 0.25, 0xDEADBEEFull, m.data());
    size_t kept = 0;
    for (uint8_t x : m) kept += x;
    check(kept > m.size() / 2 && kept < m.size(), "dropout mask kept fraction", 0);
    check(oracle_dropout_threshold(0.0) == 256 && oracle_dropout_threshold(0.999) == 0, "thresholds", 0);
    std::printf("%s\n", fails ? "FAILED" : "oracle: all checks passed");
    return fails ? 1 : 0;
}
