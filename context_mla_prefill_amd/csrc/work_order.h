// Which part of a rank's attention a workgroup computes, shared by the partial-attention kernels.
//
// Split KV ("[DeepSeekV4][PCP] Enable context-parallel prefill for hybrid KV and MegaMoE",
// "Purpose": local partials whose LSE and output are merged globally, here applied to key
// ranges of one row as to ranks): virtual row v's keys are cut into s_v ranges by position,
// s_v = vrow_splits[v] clamped into [1, kv_splits] (every row kv_splits when vrow_splits is
// NULL). With L = vrow_kv_len[v] and n = ceil(L / 64), range s holds request-relative keys
// [64 floor(s n / s_v), 64 floor((s + 1) n / s_v)) and is written to split slice s; slices
// s_v .. kv_splits-1 of the row hold no keys and get LSE = -inf from the range-0 workgroup
// (their O is not written: the merge reads no output whose weight is zero).
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

namespace mla {
namespace sched {

template <int NTH>
__device__ __forceinline__ int block_scan_incl(int v, int* sh) {
    const int t = threadIdx.x;
    sh[t] = v;
    __syncthreads();
    for (int off = 1; off < NTH; off <<= 1) {
        const int add = t >= off ? sh[t - off] : 0;
        __syncthreads();
        sh[t] += add;
        __syncthreads();
    }
    const int r = sh[t];
    __syncthreads();
    return r;
}

// Key ranges of virtual row v.
__device__ __forceinline__ int row_splits(const int32_t* __restrict__ vrow_splits, int v, int kv_splits) {
    return vrow_splits ? min(max(vrow_splits[v], 1), kv_splits) : kv_splits;
}

// First key and end of range `split` of `nsplit` over a row whose last position is L - 1:
// whole 64-key blocks (n <= 2^25 blocks and nsplit <= 64, so the products fit 32 bits).
__device__ __forceinline__ void split_range(int L, int split, int nsplit, int& key_lo, int& key_hi) {
    const unsigned n = (unsigned)(L + 63) / 64;
    key_lo = 64 * (int)((unsigned)split * n / (unsigned)nsplit);
    key_hi = 64 * (int)((unsigned)(split + 1) * n / (unsigned)nsplit);
}

struct DenseWork {
    int v;       // virtual row (-1: no work, the launch's grid is an upper bound)
    int tile;    // row tile inside the virtual row
    int split;   // key range
    int nsplit;  // key ranges of the row
};

// Work item wg of a dense launch. Virtual rows are taken in the order vrow_order[0], [1], ...
// (entries clamped into [0, n_vrows)), else from the last row to the first; a row contributes
// ceil(rows * H / ROWS) row tiles times its split count items, its tiles from the last (the
// longest key range under the causal mask) to the first, the ranges of one tile adjacent.
template <int ROWS, int NTH>
__device__ __forceinline__ DenseWork find_work(int wg, const int32_t* __restrict__ cu, int n_vrows, int H,
                                               const int32_t* __restrict__ vrow_splits,
                                               const int32_t* __restrict__ vrow_order, int kv_splits, int* sh) {
    __shared__ int s_v, s_tile, s_split, s_ns, s_carry;
    if (threadIdx.x == 0) {
        s_v = -1;
        s_tile = s_split = 0;
        s_ns = 1;
        s_carry = 0;
    }
    __syncthreads();
    for (int base = 0; base < n_vrows; base += NTH) {
        const int k = base + threadIdx.x;
        int v = 0, cnt = 0, tiles = 0, ns = 1;
        if (k < n_vrows) {
            v = vrow_order ? min(max(vrow_order[k], 0), n_vrows - 1) : n_vrows - 1 - k;
            const int len = cu[v + 1] - cu[v];
            tiles = len > 0 ? (int)(((int64_t)len * H + ROWS - 1) / ROWS) : 0;
            ns = row_splits(vrow_splits, v, kv_splits);
            cnt = tiles * ns;
        }
        const int incl = block_scan_incl<NTH>(cnt, sh);
        const int lo = s_carry + incl - cnt;
        if (k < n_vrows && wg >= lo && wg < lo + cnt) {
            const int i = wg - lo;
            s_v = v;
            s_tile = tiles - 1 - i / ns;
            s_split = i - (i / ns) * ns;
            s_ns = ns;
        }
        __syncthreads();
        if (threadIdx.x == NTH - 1) s_carry += incl;
        __syncthreads();
        if (s_v >= 0) break;
    }
    DenseWork w;
    w.v = __builtin_amdgcn_readfirstlane(s_v);  // workgroup-uniform: kept in SGPRs
    w.tile = __builtin_amdgcn_readfirstlane(s_tile);
    w.split = __builtin_amdgcn_readfirstlane(s_split);
    w.nsplit = __builtin_amdgcn_readfirstlane(s_ns);
    return w;
}

// LSE = -inf in the slices a row with nsplit ranges leaves empty; lse0 is split slice 0.
__device__ __forceinline__ void mark_empty_slices(float* __restrict__ lse0, int64_t grow, bool writer, int split,
                                                  int nsplit, int kv_splits, int64_t split_stride, int H) {
    if (writer && split == 0)
        for (int s = nsplit; s < kv_splits; ++s) lse0[(int64_t)s * split_stride * H + grow] = -INFINITY;
}

}  // namespace sched
}  // namespace mla
