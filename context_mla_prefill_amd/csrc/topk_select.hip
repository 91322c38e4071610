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
//      the k-th largest key thr and how many keys equal to thr are taken; when more keys equal
//      thr than are taken, a second select over their indices finds the cut;
//   4. the k selected indices are marked in an LDS bitmap over the row and written in order
//      (a workgroup prefix sum of the words' popcounts).
// So the row is read once. When fewer than k or more than CAND scores reach t0 (rows far from
// i.i.d., e.g. sorted or heavily tied), step 3 runs over the row in memory instead (four
// passes) and an ordered pass over the row writes the indices of keys > thr and of the first
// `need` keys == thr at their rank (a workgroup prefix sum per 2048 scores). Rows of at most
// CAND scores are loaded into LDS whole and take the ordered pass from LDS.
#include "internal.h"

namespace mla {
namespace {

constexpr int NT = 512;        // threads per workgroup (8 waves)
constexpr int NW = NT / 64;
constexpr int CAND = 6144;     // LDS candidates (4-byte key + 4-byte index each)
constexpr int PER_THREAD = CAND / NT;
constexpr int UNROLL = 4;      // float4 loads per thread and gather step (two steps in flight)
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
    uint32_t sel[3];
    uint32_t count;
    uint32_t orbits;
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
// among the rank largest and `equal` how many keys equal it. Every thread returns the same
// values.
// With SKIP (keys in LDS) the digits above the highest bit in which two keys differ are
// taken from the first key without a histogram: that spares passes in which every key would
// fall in one bin and every atomic would hit one address.
template <bool SKIP, class KeyAt>
__device__ uint32_t select_rank(KeyAt key_at, int64_t count, uint32_t& rank, uint32_t& equal, Shared& sh) {
    const int tid = threadIdx.x;
    uint32_t prefix = 0, mask = 0;
    int top_shift = 24;
    if constexpr (SKIP) {
        const uint32_t k0 = key_at(0);
        uint32_t x = 0;
        for (int64_t i = tid; i < count; i += NT) x |= key_at(i) ^ k0;
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) x |= __shfl_xor(x, o, 64);
        if (tid == 0) sh.orbits = 0;
        __syncthreads();
        if ((tid & 63) == 0 && x) atomicOr(&sh.orbits, x);
        __syncthreads();
        x = sh.orbits;
        if (x == 0) {  // every key equals k0
            equal = (uint32_t)count;
            return k0;
        }
        top_shift = ((31 - __builtin_clz(x)) >> 3) << 3;
        if (top_shift < 24) {
            mask = ~((1u << (top_shift + 8)) - 1u);
            prefix = k0 & mask;
        }
    }
    for (int shift = top_shift; shift >= 0; shift -= 8) {
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
                        sh.sel[2] = c[e];
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
        equal = sh.sel[2];
    }
    return prefix;
}

// Six waves per SIMD (three workgroups per CU, as many as the LDS allows): the register cap
// this sets (80 VGPRs) costs a few values parked in scratch between the prologue and the output
// phase, outside the streaming loop, and hides far more memory latency than it costs.
__global__ __launch_bounds__(NT, 6) void topk_select_kernel(const float* __restrict__ scores, int64_t ld,
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

    uint32_t thr, need, equal;
    const bool whole = n <= CAND;
    if (whole) {
        // all of a thread's loads issued before any is used (one memory latency, not one per score)
        constexpr int WPER = (CAND + NT - 1) / NT;
        float x[WPER];
#pragma unroll
        for (int j = 0; j < WPER; ++j) {
            const int64_t i = tid + (int64_t)j * NT;
            x[j] = srow[min(i, n - 1)];  // n > k >= 1 here; past the row end re-reads its last score
        }
#pragma unroll
        for (int j = 0; j < WPER; ++j) {
            const int64_t i = tid + (int64_t)j * NT;
            if (i < n) sh.key[i] = order_key(x[j]);
        }
        __syncthreads();
        need = (uint32_t)k;
        thr = select_rank<true>([&](int64_t i) { return sh.key[i]; }, n, need, equal, sh);
    } else {
        // 1. threshold estimate: sample block b starts at floor(b * n / 32) rounded down to 4
        //    (all of a thread's sample loads issued before any is used)
        static_assert(NSAMP % NT == 0, "sample split evenly over the threads");
        float xs[NSAMP / NT];
#pragma unroll
        for (int j = 0; j < NSAMP / NT; ++j) {
            const int i = tid + j * NT;
            const int64_t s0 = (((int64_t)(i >> 6) * n) >> 5) & ~(int64_t)3;
            xs[j] = srow[s0 + (i & 63)];
        }
#pragma unroll
        for (int j = 0; j < NSAMP / NT; ++j) sh.key[tid + j * NT] = order_key(xs[j]);
        if (tid == 0) sh.count = 0;
        __syncthreads();
        uint32_t j = (uint32_t)min((int64_t)NSAMP, max((int64_t)1, (int64_t)(k + CAND) / 2 * NSAMP / n));
        const uint32_t t0 = select_rank<true>([&](int64_t i) { return sh.key[i]; }, NSAMP, j, equal, sh);
        // the score whose key is t0: for any score x (NaN aside), x >= f0 exactly when
        // order_key(x) >= t0 (-0 >= +0 holds, as their keys are equal)
        const float f0 = __uint_as_float((t0 & 0x80000000u) ? (t0 & 0x7FFFFFFFu) : ~t0);
        // 2. gather keys >= t0 (slots by a wave-aggregated counter). The steps whose every score
        //    lies in the row for every thread load unconditionally, the next step's loads issued
        //    before the current step is processed: a static count in flight, so only the current
        //    step's loads are waited for. The last, partial step follows them.
        constexpr int64_t SU = UNROLL * TILE;
        auto take = [&](const float4 (&v)[UNROLL], int64_t b0, bool full) {
            // this lane's takes among its 4 * UNROLL scores, then one slot range per wave: the
            // lane's offset is a wave prefix sum of the take counts, bit plane by bit plane
            uint32_t tm = 0;
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) {
                const int64_t base = b0 + u * TILE;
                const float e4[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if ((full || base + e < n) && e4[e] >= f0) tm |= 1u << (4 * u + e);
            }
            const uint32_t cnt = (uint32_t)__popc(tm);  // <= 32: six bit planes
            uint32_t pre = 0, tot = 0;
#pragma unroll
            for (int bb = 0; bb < 6; ++bb) {
                const uint64_t m = __ballot((cnt >> bb) & 1u);
                pre += __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u)) << bb;
                tot += (uint32_t)__popcll(m) << bb;
            }
            if (tot) {  // wave-uniform
                uint32_t slot0 = 0;
                if (lane == 0) slot0 = atomicAdd(&sh.count, tot);  // lane 0 is active whenever any lane is
                uint32_t slot = (uint32_t)__builtin_amdgcn_readfirstlane((int)slot0) + pre;
#pragma unroll
                for (int q = 0; q < 4 * UNROLL; ++q) {
                    if ((tm >> q) & 1u) {
                        if (slot < CAND) {
                            const float4 vq = v[q >> 2];
                            sh.key[slot] = order_key((q & 3) == 0 ? vq.x : (q & 3) == 1 ? vq.y : (q & 3) == 2 ? vq.z : vq.w);
                            sh.idx[slot] = (int32_t)(b0 + (q >> 2) * TILE + (q & 3));
                        }
                        ++slot;
                    }
                }
            }
        };
        const int64_t n_full = n / SU;
        auto load_full = [&](float4 (&d)[UNROLL], int64_t s) {
#pragma unroll
            for (int u = 0; u < UNROLL; ++u)
                d[u] = *reinterpret_cast<const float4*>(srow + s * SU + u * TILE + (int64_t)tid * 4);
        };
        float4 v[UNROLL], vn[UNROLL];
        if (n_full > 0) load_full(v, 0);
        for (int64_t s = 0; s < n_full; ++s) {
            load_full(vn, min(s + 1, n_full - 1));  // after the last full step: a repeat, unused
            take(v, s * SU + (int64_t)tid * 4, true);
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) v[u] = vn[u];
        }
        if (n_full * SU < n) {  // the partial step
            const int64_t b0 = n_full * SU + (int64_t)tid * 4;
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) {
                const int64_t base = b0 + u * TILE;
                if (base + 4 <= n) {
                    v[u] = *reinterpret_cast<const float4*>(srow + base);
                } else {
                    v[u].x = base < n ? srow[base] : -INFINITY;
                    v[u].y = base + 1 < n ? srow[base + 1] : -INFINITY;
                    v[u].z = base + 2 < n ? srow[base + 2] : -INFINITY;
                    v[u].w = -INFINITY;
                }
            }
            take(v, b0, false);
        }
        __syncthreads();
        const uint32_t c = sh.count;
        need = (uint32_t)k;
        if (c >= (uint32_t)k && c <= (uint32_t)CAND) {
            // 3. every selected key is a candidate (t0 <= thr): select among them in LDS
            thr = select_rank<true>([&](int64_t i) { return sh.key[i]; }, c, need, equal, sh);
            const int nwords = (int)((n + 31) >> 5);
            if (nwords <= CAND) {  // else the ordered pass below
                int32_t cut = INT32_MAX;  // keys == thr are taken up to this index
                if (equal > need) {
                    uint32_t r = need, e2;
                    cut = (int32_t)~select_rank<true>(
                        [&](int64_t i) { return sh.key[i] == thr ? ~(uint32_t)sh.idx[i] : 0u; }, c, r, e2, sh);
                }
                // 4. mark the k selected indices in a bitmap over the row (it overwrites the keys,
                //    so every thread first takes its candidates' verdicts into registers)
                int32_t mine[PER_THREAD];
#pragma unroll
                for (int q = 0; q < PER_THREAD; ++q) {
                    const uint32_t i = (uint32_t)(tid + q * NT);
                    mine[q] = -1;
                    if (i < c && (sh.key[i] > thr || (sh.key[i] == thr && sh.idx[i] <= cut))) mine[q] = sh.idx[i];
                }
                __syncthreads();
                uint32_t* bits = sh.key;
                for (int i = tid; i < nwords; i += NT) bits[i] = 0;
                __syncthreads();
#pragma unroll
                for (int q = 0; q < PER_THREAD; ++q)
                    if (mine[q] >= 0) atomicOr(&bits[mine[q] >> 5], 1u << (mine[q] & 31));
                __syncthreads();
                // thread t owns words [t * W, t * W + W): their set bits, in order, after the
                // set bits of all lower words
                const int W = (nwords + NT - 1) / NT;
                uint32_t cnt = 0;
                for (int q = 0; q < W; ++q) {
                    const int wi = tid * W + q;
                    cnt += wi < nwords ? (uint32_t)__popc(bits[wi]) : 0u;
                }
                uint32_t total;
                uint32_t pos = wg_exclusive_scan(cnt, sh, total);
                for (int q = 0; q < W; ++q) {
                    const int wi = tid * W + q;
                    uint32_t b = wi < nwords ? bits[wi] : 0u;
                    while (b) {
                        orow[pos++] = wi * 32 + (__builtin_ffs((int)b) - 1);
                        b &= b - 1;
                    }
                }
                return;
            }
        } else {
            thr = select_rank<false>([&](int64_t i) { return order_key(srow[i]); }, n, need, equal, sh);
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
