// Key sets and work items of the sparse partial attention.
//
// Key set of a query at position p (request-relative): the selected indices that lie in
// [0, p] and outside the window, plus every window key [max(0, p-window+1), p]; a selected
// index inside the window is counted once (the window supplies it). Selected indices must be
// distinct; -1 (or anything outside [0, p]) is a pad. With split KV only keys in the split's
// range [key_lo, key_hi) count. ("[DeepSeekV4][PCP] Enable context-parallel prefill for hybrid
// KV and MegaMoE", "Purpose": sparse prefill attention under PCP.)
//
// A workgroup owns one token, a group of up to 64 heads (a head count that is not a multiple
// of 64 leaves the last group's rows past H idle: nothing of theirs is stored) and one key
// range of its row.
#pragma once

#include "attn_core.h"
#include "work_order.h"

namespace mla {
namespace attn {

constexpr int MAX_TOPK = 2048;

// The workgroup's token, head group and key split, its virtual row, the row's number of key
// ranges and the split's key range.
struct SparseWork {
    int tok, hg, split, nsplit, lo_v, p, key_lo, key_hi;
    int64_t kv0;
};

// Grid: (token, head group, split < kv_splits); a workgroup whose split is not below its row's
// range count (nsplit) has no work.
__device__ __forceinline__ SparseWork sparse_work(int H, int kv_splits, const int32_t* __restrict__ cu, int n_vrows,
                                                 const int32_t* __restrict__ vrow_kv_start,
                                                 const int32_t* __restrict__ positions,
                                                 const int32_t* __restrict__ vrow_kv_len,
                                                 const int32_t* __restrict__ vrow_splits) {
    SparseWork w;
    // workgroup = (token, group of up to 64 heads, key split); splits of one row are adjacent
    const int hg_count = (H + BM - 1) / BM;
    const int ridx = (int)blockIdx.x / kv_splits;
    w.split = (int)blockIdx.x - ridx * kv_splits;
    w.tok = ridx / hg_count;
    w.hg = ridx - w.tok * hg_count;
    // virtual row of this token: last v with cu[v] <= tok
    int lo_v = 0, hi_v = n_vrows;
    while (hi_v - lo_v > 1) {
        const int mid = (lo_v + hi_v) >> 1;
        if (cu[mid] <= w.tok) lo_v = mid; else hi_v = mid;
    }
    w.lo_v = lo_v;
    w.kv0 = vrow_kv_start[lo_v];
    w.p = positions[w.tok];
    // Key range of this split: whole 64-key tiles [key_lo, key_hi) of the request's KV.
    w.nsplit = sched::row_splits(vrow_splits, lo_v, kv_splits);
    w.key_lo = 0;
    w.key_hi = INT32_MAX;
    if (w.nsplit > 1) sched::split_range(vrow_kv_len[lo_v], w.split, w.nsplit, w.key_lo, w.key_hi);
    return w;
}

// Q rows of a workgroup are copied whole into LDS (a token's Q rows are contiguous, so
// direct-to-LDS loads move whole cache lines) and read back as MFMA fragments: 16-byte chunk c
// of row r sits at chunk r * 72 + (c ^ q_swizzle(r)), so the fragment reads (row r = lane % 32,
// one chunk per lane) meet distinct bank slots both for 8 consecutive lanes over 128 bytes and
// for 16 over 256.
constexpr int Q_CHUNKS = 72;  // 16-byte chunks of a 576-element bf16 row
__device__ __forceinline__ int q_swizzle(int r) { return (r ^ (r >> 3)) & 7; }

}  // namespace attn
}  // namespace mla
