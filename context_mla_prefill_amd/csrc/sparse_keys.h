// Key sets of the sparse partial attention, shared by its fp8 and bf16 kernels.
//
// Key set of a query at position p (request-relative): the selected indices that lie in
// [0, p] and outside the window, plus every window key [max(0, p-window+1), p]; a selected
// index inside the window is counted once (the window supplies it). Selected indices must be
// distinct; -1 (or anything outside [0, p]) is a pad. With split KV only keys in the split's
// range [key_lo, key_hi) count. ("[DeepSeekV4][PCP] Enable context-parallel prefill for hybrid
// KV and MegaMoE", "Purpose": sparse prefill attention under PCP.)
//
// A workgroup owns one token and a group of up to 64 heads (a head count that is not a multiple
// of 64 leaves the last group's rows past H idle: their Q is zero and nothing is stored); its
// keys are visited in tiles of 64 slots: first the selected indices in groups of 64, then the
// window.
#pragma once

#include "attn_core.h"
#include "work_order.h"

namespace mla {
namespace attn {

constexpr int MAX_TOPK = 2048;
constexpr int MAX_WINDOW = 4096;

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

// Q rows of a workgroup through LDS. A token's Q rows are contiguous (H rows of 1152 bytes),
// so direct-to-LDS loads move them in whole cache lines, where per-lane fragment loads would
// touch 32 bytes of a row per instruction. The WAVES waves that share 32 rows copy them into
// `region` (36 KB of a tile buffer not yet in use) with 36 loads of 64 x 16 bytes between them,
// wave `first` taking loads first, first + WAVES, ... 16-byte chunk c of row r goes to chunk
// r * 72 + (c ^ f(r)), f(r) = (r ^ (r >> 3)) % 8: the fragment reads (row r = lane % 32, one
// chunk per lane) then meet distinct bank slots both for 8 consecutive lanes over 128 bytes and
// for 16 over 256. Rows past the head count read row H - 1 (their results are never stored).
constexpr int Q_CHUNKS = 72;                      // 16-byte chunks of a 576-element bf16 row
constexpr int Q_REGION_BYTES = 32 * Q_CHUNKS * 16;  // 32 rows
__device__ __forceinline__ int q_swizzle(int r) { return (r ^ (r >> 3)) & 7; }
// q_rsrc: the token's Q rows; row0: head of the first of the 32 rows.
template <int WAVES>
__device__ __forceinline__ void dma_q_rows(__amdgpu_buffer_rsrc_t q_rsrc, int row0, int H, char* region, int first,
                                           int lane) {
    static_assert(Q_CHUNKS * 32 % (64 * WAVES) == 0, "loads split evenly over the waves");
#pragma unroll
    for (int j = 0; j < Q_CHUNKS * 32 / 64 / WAVES; ++j) {
        const int i = WAVES * j + first;  // load i fills LDS chunks 64 i .. 64 i + 63
        const int L = 64 * i + lane;
        const int r = L / Q_CHUNKS;
        const int c = (L - r * Q_CHUNKS) ^ q_swizzle(r);
        const int row = min(row0 + r, H - 1);
        lds_dma16(q_rsrc, (uint32_t)(row * (Q_CHUNKS * 16) + c * 16), region + 1024 * i);
    }
}
// Q K^T operand fragments of row lane % 32 of the pair from `region`: elements
// [16 kb + 8 (lane / 32), +8) of the row.
template <int KB>
__device__ __forceinline__ void read_q_frags(const char* region, int lane, bf16x8 (&qf)[KB]) {
    const int r = lane & 31, half = lane >> 5;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
        const int c = (2 * kb + half) ^ q_swizzle(r);
        qf[kb] = *reinterpret_cast<const bf16x8*>(region + 16 * (r * Q_CHUNKS + c));
    }
}

// Epilogue of a sparse workgroup: the normalised O rows go through LDS so that every global
// store writes one whole 1 KB row (the MFMA layout leaves a lane 8 bytes of each of 32 rows per
// store otherwise); LSE as in the dense epilogue. `region` is a free 64 KB tile buffer (the
// caller has waited for its own loads into LDS). 8-byte chunk q of row r sits at chunk
// q ^ (r % 32), so the row-per-lane writes (32 rows at one chunk) meet distinct bank slots for
// both 16 lanes over 128 bytes and 32 over 256, and each row stays inside its own 1 KB.
// grow: this lane's global row; valid: it is below the head count (the valid rows of a
// workgroup are a prefix). The workgroup's first row and valid-row count are derived here from
// these two, so nothing more stays live through the key loop.
template <class S, int DL>
__device__ __forceinline__ void write_rows_staged(const f32x16 (&acc_o)[S::NB / 2], float m_ref, float l_run,
                                                  bool valid, int64_t grow, int wave, int side, int lane,
                                                  Exchange& ex, char* region, __bf16* __restrict__ o_out,
                                                  float* __restrict__ lse_out) {
    static_assert(DL * 2 == 1024 && BM * DL * 2 <= S::ROPE_OFF, "64 rows of 1 KB fit a tile buffer");
    constexpr int NB0 = S::NB / 2;
    const int half = lane >> 5;
    const int r = (wave >> 1) * 32 + (lane & 31);  // this lane's row of the workgroup
    const float l_w = l_run + __shfl_xor(l_run, 32);
    const int n_mine = __popcll(__ballot(valid)) / 2;  // valid rows of this wave's pair
    __syncthreads();  // every wave is past its last tile: the tile buffers are free
    ex.mx[wave][lane] = l_w;
    if (lane == 0) ex.flag[wave] = n_mine;
    __syncthreads();
    const float l_tot = l_w + ex.mx[wave ^ 1][lane];
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    const int n_valid = __builtin_amdgcn_readfirstlane(n_mine + ex.flag[wave ^ 2]);
    char* const lrow = region + r * (DL * 2);
#pragma unroll
    for (int d = 0; d < NB0; ++d) {
        const int db = side * NB0 + d;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            bf16x4 y;
#pragma unroll
            for (int e = 0; e < 4; ++e) y[e] = (__bf16)(acc_o[d][4 * g + e] * inv);
            const int q = (db * 32 + 8 * g + 4 * half) / 4;
            *reinterpret_cast<bf16x4*>(lrow + 8 * (q ^ (r & 31))) = y;
        }
    }
    if (valid && side == 0 && half == 0) lse_out[grow] = (m_ref + __builtin_amdgcn_logf(l_tot)) * kLn2;
    __syncthreads();
    // wave w stores rows 16w .. 16w+15; lane l the row's bytes [16 l, 16 l + 16): stored chunks
    // 2l ^ s and 2l+1 ^ s (s = row % 32) share the 16-byte slot l ^ (s / 2), swapped when s is odd
    __bf16* const o_wg = o_out + (grow - r) * DL + 8 * lane;  // the workgroup's first row
    constexpr int ROWS = BM / (NT / 64);
#pragma unroll
    for (int i = 0; i < ROWS; ++i) {
        const int row = ROWS * wave + i;
        if (row >= n_valid) break;  // wave-uniform
        const int s = row & 31;
        uint4 v = *reinterpret_cast<const uint4*>(region + row * (DL * 2) + 16 * (lane ^ (s >> 1)));
        if (s & 1) v = uint4{v.z, v.w, v.x, v.y};
        *reinterpret_cast<uint4*>(o_wg + row * DL) = v;
    }
}

// Rows of the keys: relative to the request's first row for packed KV (row = key position),
// absolute for paged KV (row = block_table entry * 64 + position % 64).
template <bool PAGED>
struct SparseKeys {
    const int* sel;      // LDS [MAX_TOPK]: row of each selected key of the set, -1 otherwise
    const int* win_blk;  // LDS: paged cache blocks the window spans
    int n_sel_tiles, n_tiles, window, win_lo, p, key_lo, key_hi, pad_row;

    // Row of the key in slot j of tile t and whether the slot holds a key of the set; empty
    // slots and tiles past the last one read pad_row (the row of key 0: a written key whose
    // value meets a zero probability, so it must be finite).
    __device__ __forceinline__ int slot_key(int t, int j, bool& ok) const {
        if (t < n_sel_tiles) {
            const int e = sel[t * BN + j];
            ok = e >= 0;
            return ok ? e : pad_row;
        }
        const int w = (t - n_sel_tiles) * BN + j;
        const int k = win_lo + w;
        ok = window > 0 && w < window && k <= p && k >= key_lo && k < key_hi;
        if (!ok) return pad_row;
        return PAGED ? win_blk[(k >> 6) - (win_lo >> 6)] * BN + (k & (BN - 1)) : k;
    }
    // Next tile index >= t that holds at least one key (n_tiles if none); workgroup-uniform.
    __device__ __forceinline__ int next_live(int t, int lane) const {
        for (; t < n_tiles; ++t) {
            bool ok = false;
            if (lane < BN) slot_key(t, lane, ok);
            if (__ballot(ok)) break;  // every wave evaluates the same slots
        }
        return t;
    }
};

// Fills the workgroup's selected-row list and window blocks (all threads take part; a barrier
// must follow before slot_key is used). The selected indices are filtered once: an entry
// outside [0, p], outside the split's key range or inside the window becomes -1, a kept one
// its row.
template <bool PAGED>
__device__ __forceinline__ SparseKeys<PAGED> sparse_keys(int* sel, int* win_blk, const int32_t* __restrict__ topk_idx,
                                                         int topk, int window, const SparseWork& w,
                                                         const int32_t* __restrict__ bt_row, int bt_stride) {
    // paged: table columns past bt_stride read its last entry; the kernels clamp every row
    // into the cache before they form an offset from it (a block id outside the cache reads
    // wrong rows of the cache, never memory outside it)
    auto blk = [&](int col) { return bt_row[min(col, bt_stride - 1)]; };
    SparseKeys<PAGED> ks;
    ks.sel = sel;
    ks.win_blk = win_blk;
    ks.window = window;
    ks.p = w.p;
    ks.key_lo = w.key_lo;
    ks.key_hi = w.key_hi;
    ks.win_lo = max(0, w.p - window + 1);  // first window key (window > 0)
    ks.pad_row = PAGED ? blk(0) * BN : 0;
    ks.n_sel_tiles = (topk + BN - 1) / BN;
    ks.n_tiles = ks.n_sel_tiles + (window + BN - 1) / BN;
    // Every thread's PER entries: all index loads issued before the first is used (and, paged,
    // all block-table loads, at clamped columns so they need no branch), so the list costs one
    // or two memory latencies instead of one per entry.
    constexpr int PER = MAX_TOPK / NT;
    static_assert(MAX_TOPK % NT == 0, "selected-row list split evenly over the threads");
    int e[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        const int i = (int)threadIdx.x + j * NT;
        e[j] = i < topk ? topk_idx[(int64_t)w.tok * topk + i] : -1;
    }
    int r[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        if constexpr (PAGED)
            r[j] = blk(max(e[j], 0) >> 6) * BN + (e[j] & (BN - 1));
        else
            r[j] = e[j];
    }
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        const bool ok = e[j] >= w.key_lo && e[j] < w.key_hi && e[j] <= w.p && (window == 0 || e[j] < ks.win_lo);
        sel[(int)threadIdx.x + j * NT] = ok ? r[j] : -1;
    }
    if constexpr (PAGED) {
        const int nwb = window > 0 ? (w.p >> 6) - (ks.win_lo >> 6) + 1 : 0;  // <= MAX_WINDOW / BN + 1
        for (int i = threadIdx.x; i < nwb; i += NT) win_blk[i] = blk((ks.win_lo >> 6) + i);
    }
    return ks;
}

}  // namespace attn
}  // namespace mla
