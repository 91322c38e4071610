// pcp_plan_splits: host-side choice of per-virtual-row key-range counts (split KV) and of the
// order in which the dense kernels take the virtual rows.
//
// Split KV spreads one row's keys over several workgroups whose partials the LSE merge
// combines ("[DeepSeekV4][PCP] Enable context-parallel prefill for hybrid KV and MegaMoE",
// "Purpose"). It pays only where a few long work items would otherwise leave compute units
// idle at the end of the launch -- decode rows over long contexts (replicated on every rank,
// "[Core] Add MRV2 virtual-batch PCP for MLA", "PCP algorithm"), or a batch whose longest
// tiles are a large share of a compute unit's work -- and costs a fixed amount per extra
// workgroup everywhere else. The planner therefore models the launch: every (row tile, key
// range) item costs its key count plus a fixed per-workgroup cost, items are dealt to the
// compute units in launch order, each to the first unit that falls idle, and the plan with the
// shortest modelled finish time among a few candidate families wins; a split plan must beat
// the unsplit one by 2 %.
#include <algorithm>
#include <cmath>
#include <functional>
#include <queue>
#include <vector>

#include "internal.h"

namespace mla {
namespace {

constexpr double kItemCost = 640.0;  // fixed cost of one workgroup, in keys of one row tile
constexpr double kMinGain = 0.98;    // a split plan must finish within 98 % of the unsplit one

struct VRow {
    int T;       // tokens
    int64_t p0;  // position of the first token
    int64_t L;   // last position + 1
};

// Keys of range s of ns over a row whose last position is L - 1, inside [0, K).
int64_t range_keys(int64_t L, int64_t K, int s, int ns) {
    const int64_t n = (L + 63) / 64;
    const int64_t lo = 64 * (s * n / ns), hi = 64 * ((s + 1) * n / ns);
    return std::max<int64_t>(0, std::min(K, hi) - lo);
}

struct RankModel {
    std::vector<VRow> rows;
    int H = 1, R = 128;

    int tiles(const VRow& v) const { return v.T > 0 ? (int)(((int64_t)v.T * H + R - 1) / R) : 0; }
    // Key count (last position + 1) of row tile j.
    int64_t tile_keys(const VRow& v, int j) const {
        const int64_t last = std::min<int64_t>(((int64_t)(j + 1) * R - 1) / H, v.T - 1);
        return v.p0 + last + 1;
    }
    int64_t longest(const VRow& v) const { return v.T > 0 ? tile_keys(v, tiles(v) - 1) : 0; }

    // Total modelled work of a plan (keys plus the fixed cost of every item).
    double work(const std::vector<int>& ns) const {
        double w = 0;
        for (size_t i = 0; i < rows.size(); ++i) {
            const VRow& v = rows[i];
            for (int j = 0; j < tiles(v); ++j) w += (double)tile_keys(v, j) + kItemCost * ns[i];
        }
        return w;
    }

    // Modelled finish time: items in launch order, each to the compute unit that idles first.
    double finish(const std::vector<int>& ns, const std::vector<int>& order, int workers) const {
        std::priority_queue<double, std::vector<double>, std::greater<double>> idle;
        for (int i = 0; i < workers; ++i) idle.push(0.0);
        double end = 0.0;
        for (int v : order) {
            const VRow& r = rows[v];
            for (int j = tiles(r) - 1; j >= 0; --j) {
                const int64_t K = tile_keys(r, j);
                for (int s = 0; s < ns[v]; ++s) {
                    const double keys = ns[v] > 1 ? (double)range_keys(r.L, K, s, ns[v]) : (double)K;
                    const double t = idle.top() + keys + kItemCost;
                    idle.pop();
                    idle.push(t);
                    end = std::max(end, t);
                }
            }
        }
        return end;
    }
};

}  // namespace
}  // namespace mla

using namespace mla;

extern "C" mla_status pcp_plan_splits(const int32_t* q_lens, const int32_t* kv_lens, int32_t n_req, int32_t P,
                                      int32_t H, int32_t D_latent, int32_t max_splits, int32_t n_workers,
                                      int32_t* vrow_splits, int32_t* vrow_order) {
    int32_t T_loc[64], n_vrows = 0;
    int64_t T_glob = 0;
    const mla_status st = pcp_plan_sizes(q_lens, kv_lens, n_req, P, T_loc, &n_vrows, &T_glob);
    if (st != MLA_OK) return st;  // lengths, P and totals checked there
    if (H < 1 || H > 128) return fail(MLA_ERR_INVALID_ARG, "pcp_plan_splits: H=%d outside 1..128", H);
    if (D_latent != 512 && D_latent != 64)
        return fail(MLA_ERR_UNSUPPORTED, "pcp_plan_splits: D_latent=%d (512 or 64)", D_latent);
    if (max_splits < 1 || max_splits > 64)
        return fail(MLA_ERR_INVALID_ARG, "pcp_plan_splits: max_splits=%d outside 1..64", max_splits);
    if (n_workers < 1) return fail(MLA_ERR_INVALID_ARG, "pcp_plan_splits: n_workers=%d < 1", n_workers);
    if (n_vrows > 0 && (!vrow_splits || !vrow_order))
        return fail(MLA_ERR_INVALID_ARG, "pcp_plan_splits: null output");

    for (int r = 0; r < P; ++r) {
        // This rank's virtual rows, as pcp_partition lays them out.
        RankModel m;
        m.H = H;
        m.R = D_latent == 512 ? 128 : 64;  // rows of a dense workgroup for the shape
        for (int32_t b = 0; b < n_req; ++b) {
            const int64_t q = q_lens[b], kv = kv_lens[b], past = kv - q;
            if (q >= 2 * (int64_t)P) {
                const int64_t n = 2 * (int64_t)P, base = q / n, extra = q % n;
                for (const int64_t c : {(int64_t)r, n - 1 - r}) {
                    const int64_t start = c * base + std::min(c, extra), size = base + (c < extra);
                    m.rows.push_back({(int)size, past + start, past + start + size});
                }
            } else {
                m.rows.push_back({(int)q, past, kv});
            }
        }
        const int nv = (int)m.rows.size();
        int32_t* splits_out = vrow_splits + (int64_t)r * n_vrows;
        int32_t* order_out = vrow_order + (int64_t)r * n_vrows;

        std::vector<int> ns(nv, 1), order(nv);
        for (int k = 0; k < nv; ++k) order[k] = nv - 1 - k;  // the kernels' default: last row first
        const double base = m.finish(ns, order, n_workers);
        double best = base * kMinGain;
        std::vector<int> best_ns = ns, best_order = order;
        // Tries a plan in the default order and with rows taken longest range first; returns
        // false once the plan's work alone exceeds the best finish (more ranges only add work).
        auto consider = [&](const std::vector<int>& cand) {
            if (m.work(cand) / n_workers >= best) return false;
            std::vector<int> ord = order;
            std::stable_sort(ord.begin(), ord.end(), [&](int a, int b) {
                return (double)m.longest(m.rows[a]) / cand[a] > (double)m.longest(m.rows[b]) / cand[b];
            });
            for (const std::vector<int>* o : {&order, &ord}) {
                const double f = m.finish(cand, *o, n_workers);
                if (f < best) {
                    best = f;
                    best_ns = cand;
                    best_order = *o;
                }
            }
            return true;
        };
        int64_t longest = 1;
        for (const VRow& v : m.rows) longest = std::max(longest, m.longest(v));
        auto ranges = [&](const VRow& v, double piece, int cap) {
            return (int)std::min<int64_t>(cap, std::max<int64_t>(1, (int64_t)std::ceil((double)m.longest(v) / piece)));
        };
        // (a) rows split so that no range of their longest tile exceeds tau keys, tau halving
        // from half the longest tile: long rows first.
        std::vector<int> prev = ns;
        for (double tau = (double)longest / 2; tau >= 4 * kItemCost && max_splits > 1; tau /= 2) {
            std::vector<int> cand(nv);
            for (int i = 0; i < nv; ++i) cand[i] = ranges(m.rows[i], tau, max_splits);
            if (cand == prev) continue;
            prev = cand;
            if (!consider(cand)) break;
        }
        // (b) every row k ranges (k = 2, 4, ...), no range under 4 fixed costs of keys: a finer
        // grain where many rows are of similar length.
        prev = ns;
        std::vector<int> ks;
        for (int k = 2; k < max_splits; k *= 2) ks.push_back(k);
        if (max_splits > 1) ks.push_back(max_splits);
        for (const int k : ks) {
            std::vector<int> cand(nv);
            for (int i = 0; i < nv; ++i) cand[i] = ranges(m.rows[i], 4 * kItemCost, k);
            if (cand == prev) break;
            prev = cand;
            if (!consider(cand)) break;
        }
        for (int k = 0; k < nv; ++k) {
            splits_out[k] = best_ns[k];
            order_out[k] = best_order[k];
        }
    }
    return MLA_OK;
}
