// Top-k selection of index scores: for every query row, the k keys of its causal prefix
// with the largest index scores, the selected-index input of the sparse partial attention
// (the indexer's top-k ahead of sparse MLA: "DeepSeek-V4.1: Prefill support CP with
// multistream forward prepare (4/N)", "Modifications" -- indexer work before the MQA
// logits -- and its commit list, "Indexer ... uses topk_v2").
//
// Order: a larger score first; equal scores (-0 equals +0) by the smaller key index. The
// selected indices are written in increasing order.
//
// One workgroup per row; the row streams from HBM:
//   1. a threshold estimate t0 from 2048 sampled scores (32 blocks of 64 consecutive ones),
//      the sample rank chosen so that about (k + CAND) / 2 scores of a row lie at or above it;
//   2. one pass gathers every score >= t0 (key and index) into LDS, at most CAND of them;
//   3. an exact radix select (four 8-bit digits, LDS histograms) over the gathered keys gives
//      the k-th largest key thr and how many keys equal to thr are taken;
//   4. one ordered pass writes the indices of keys > thr, and of the first `need` keys == thr,
//      at their rank among the selected ones (a workgroup prefix sum per 2048 scores).
// When fewer than k or more than CAND scores reach t0 (rows far from i.i.d., e.g. sorted or
// heavily tied), step 3 runs over the row in memory instead (four passes). Rows of at most
// CAND scores are loaded into LDS whole and never re-read.
#include "internal.h"

namespace mla {
namespace {

constexpr int NT = 512;        // threads per workgroup (8 waves)
constexpr int NW = NT / 64;
constexpr int CAND = 6144;     // LDS candidates (4-byte key + 4-byte index each)
constexpr int NSAMP = 2048;    // sampled scores for the threshold estimate
constexpr int TILE = NT * 4;   // scores per ordered-pass step (4 consecutive per thread)

// Monotone map of a finite (or infinite) fp32 score to uint32: a larger score gives a larger
// key; -0 and +0 give the same key.
__device__ __forceinline__ uint32_t order_key(float x) {
    uint32_t u = __float_as_uint(x);
    if ((u << 1) == 0) u = 0;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

struct Shared {
    uint32_t key[CAND];
    int32_t idx[CAND];
    uint32_t hist[256];
    uint32_t wsum[NW];
    uint32_t sel[2];
    uint32_t count;
};

// Exclusive prefix sum of v over the workgroup; `total` gets the sum. Two barriers.
__device__ __forceinline__ uint32_t wg_exclusive_scan(uint32_t v, Shared& sh, uint32_t& total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t inc = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = __shfl_up(inc, o, 64);
        if (lane >= o) inc += y;
    }
    if (lane == 63) sh.wsum[wave] = inc;
    __syncthreads();
    uint32_t before = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        const uint32_t s = sh.wsum[w];
        before += w < wave ? s : 0;
        tot += s;
    }
    __syncthreads();
    total = tot;
    return before + inc - v;
}

// The rank-th largest key (1-based) among count keys produced by key_at(i), by four 8-bit
// radix digits from the top. On return `rank` holds how many keys equal to the result are
// among the rank largest. Every thread returns the same values.
template <class KeyAt>
__device__ uint32_t select_rank(KeyAt key_at, int64_t count, uint32_t& rank, Shared& sh) {
    const int tid = threadIdx.x;
    uint32_t prefix = 0, mask = 0;
    for (int shift = 24; shift >= 0; shift -= 8) {
        for (int b = tid; b < 256; b += NT) sh.hist[b] = 0;
        __syncthreads();
        for (int64_t i = tid; i < count; i += NT) {
            const uint32_t key = key_at(i);
            if ((key & mask) == prefix) atomicAdd(&sh.hist[(key >> shift) & 255u], 1u);
        }
        __syncthreads();
        if (tid < 64) {
            // lane l owns bins 255-4l .. 252-4l, scanned from the top bin down
            uint32_t c[4], s = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                c[e] = sh.hist[255 - 4 * tid - e];
                s += c[e];
            }
            uint32_t inc = s;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const uint32_t y = __shfl_up(inc, o, 64);
                if (tid >= o) inc += y;
            }
            uint32_t above = inc - s;
            if (above < rank && rank <= inc) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if (rank <= above + c[e]) {
                        sh.sel[0] = 255u - 4u * tid - e;
                        sh.sel[1] = rank - above;
                        break;
                    }
                    above += c[e];
                }
            }
        }
        __syncthreads();
        prefix |= sh.sel[0] << shift;
        mask |= 255u << shift;
        rank = sh.sel[1];
    }
    return prefix;
}

__global__ __launch_bounds__(NT) void topk_select_kernel(const float* __restrict__ scores, int64_t ld,
                                                         const int32_t* __restrict__ positions, int k,
                                                         int32_t* __restrict__ out) {
    __shared__ Shared sh;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int64_t row = blockIdx.x;
    const int64_t n = min(max((int64_t)positions[row] + 1, (int64_t)0), ld);
    int32_t* __restrict__ orow = out + row * k;
    const float* __restrict__ srow = scores + row * ld;

    if (n <= k) {  // the whole prefix, then pads
        for (int i = tid; i < k; i += NT) orow[i] = i < n ? i : -1;
        return;
    }

    uint32_t thr, need;
    const bool whole = n <= CAND;
    if (whole) {
        for (int64_t i = tid; i < n; i += NT) sh.key[i] = order_key(srow[i]);
        __syncthreads();
        need = (uint32_t)k;
        thr = select_rank([&](int64_t i) { return sh.key[i]; }, n, need, sh);
    } else {
        // 1. threshold estimate: sample block b starts at floor(b * n / 32) rounded down to 4
        for (int i = tid; i < NSAMP; i += NT) {
            const int64_t s0 = (((int64_t)(i >> 6) * n) >> 5) & ~(int64_t)3;
            sh.key[i] = order_key(srow[s0 + (i & 63)]);
        }
        if (tid == 0) sh.count = 0;
        __syncthreads();
        uint32_t j = (uint32_t)min((int64_t)NSAMP, max((int64_t)1, (int64_t)(k + CAND) / 2 * NSAMP / n));
        const uint32_t t0 = select_rank([&](int64_t i) { return sh.key[i]; }, NSAMP, j, sh);
        // 2. gather keys >= t0 (slots by a wave-aggregated counter)
        for (int64_t base = (int64_t)tid * 4; base < n; base += TILE) {
            float4 v;
            if (base + 4 <= n) {
                v = *reinterpret_cast<const float4*>(srow + base);
            } else {
                v.x = srow[base];
                v.y = base + 1 < n ? srow[base + 1] : -INFINITY;
                v.z = base + 2 < n ? srow[base + 2] : -INFINITY;
                v.w = -INFINITY;
            }
            const float e4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t key = order_key(e4[e]);
                const bool take = base + e < n && key >= t0;
                const uint64_t bal = __ballot(take);
                if (bal == 0) continue;  // wave-uniform
                uint32_t slot0 = 0;
                if (lane == 0) slot0 = atomicAdd(&sh.count, (uint32_t)__popcll(bal));
                slot0 = __shfl(slot0, 0, 64);
                const uint32_t slot = slot0 + (uint32_t)__popcll(bal & ((1ull << lane) - 1));
                if (take && slot < CAND) {
                    sh.key[slot] = key;
                    sh.idx[slot] = (int32_t)(base + e);
                }
            }
        }
        __syncthreads();
        const uint32_t c = sh.count;
        need = (uint32_t)k;
        if (c >= (uint32_t)k && c <= (uint32_t)CAND) {
            thr = select_rank([&](int64_t i) { return sh.key[i]; }, c, need, sh);
        } else {
            thr = select_rank([&](int64_t i) { return order_key(srow[i]); }, n, need, sh);
        }
    }

    // 4. ordered pass: keys > thr, and the first `need` keys == thr, in index order
    const uint32_t gt_total = (uint32_t)k - need;
    uint32_t g_run = 0, e_run = 0;
    for (int64_t t0 = 0; t0 < n; t0 += TILE) {
        const int64_t base = t0 + (int64_t)tid * 4;
        uint32_t key[4];
        if (whole) {
#pragma unroll
            for (int e = 0; e < 4; ++e) key[e] = base + e < n ? sh.key[base + e] : 0u;
        } else if (base + 4 <= n) {
            const float4 v = *reinterpret_cast<const float4*>(srow + base);
            key[0] = order_key(v.x);
            key[1] = order_key(v.y);
            key[2] = order_key(v.z);
            key[3] = order_key(v.w);
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) key[e] = base + e < n ? order_key(srow[base + e]) : 0u;
        }
        uint32_t gt = 0, eq = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const bool in = base + e < n;
            gt += (in && key[e] > thr) ? 1u : 0u;
            eq += (in && key[e] == thr) ? 1u : 0u;
        }
        uint32_t total;
        const uint32_t ex = wg_exclusive_scan(gt | (eq << 16), sh, total);  // per-tile sums <= 2048
        uint32_t g_before = g_run + (ex & 0xFFFFu);
        uint32_t e_before = e_run + (ex >> 16);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const bool in = base + e < n;
            const bool is_gt = in && key[e] > thr;
            const bool is_eq = in && key[e] == thr;
            if (is_gt || (is_eq && e_before < need)) orow[g_before + min(e_before, need)] = (int32_t)(base + e);
            g_before += is_gt ? 1u : 0u;
            e_before += is_eq ? 1u : 0u;
        }
        g_run += total & 0xFFFFu;
        e_run += total >> 16;
        if (g_run >= gt_total && e_run >= need) break;  // workgroup-uniform: all k written
    }
}

}  // namespace

hipError_t launch_topk_select(const float* scores, int64_t ld, const int32_t* positions, int32_t T, int32_t k,
                              int32_t* topk_idx, hipStream_t stream) {
    hipLaunchKernelGGL(topk_select_kernel, dim3((unsigned)T), dim3(NT), 0, stream, scores, ld, positions, k,
                       topk_idx);
    return hipGetLastError();
}

}  // namespace mla
