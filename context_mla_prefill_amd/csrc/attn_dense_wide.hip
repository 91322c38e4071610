// Rank-local causal MLA partial attention (dense) for the 512 + 64 shape, bf16 MFMA on gfx950.
//
// Absorbed MLA is multi-query attention with one latent KV head: key = latent || rope,
// value = latent. Every rank attends its local rows against the full all-gathered latent KV
// ("[Core] Add MRV2 virtual-batch PCP for MLA", "DualChunkSwap partitioning") and returns the
// normalised partial output and its natural-log LSE without the sink, which the merge applies
// once ("[DeepSeekV4][PCP] Enable context-parallel prefill for hybrid KV and MegaMoE",
// "Purpose").
//
// Work decomposition
//  * A workgroup (4 waves, one per SIMD) owns BM = 128 rows of one virtual row, a row being a
//    (token, head) pair: all heads share the KV, so token x head is the M dimension. Each wave
//    owns 32 rows outright: their Q (144 VGPRs, the B operand of Q K^T) and their whole output
//    (512 columns, 256 fp32 accumulators in AGPRs) stay in its registers for the KV loop, so
//    the softmax is wave-local and no scores or probabilities cross waves.
//  * KV tiles of 32 keys move HBM -> LDS with direct-to-LDS buffer loads into three buffers and
//    are read by all 128 rows (37 KB of tile per 8.9 MFLOP: twice the rows per byte of a
//    64-row workgroup). During tile t a wave reads tile t (Q K^T), reads tile t-1 (P V) and
//    issues its share of tile t+1's loads among its Q K^T MFMAs; one barrier per tile.
//  * Scores transposed, S^T = K Q^T (v_mfma_f32_32x32x16_bf16, A = K from LDS, B = Q^T). Each
//    lane then holds 16 scores of ONE row; the row max is one half-wave swap.
//  * Output transposed, O^T += V^T P^T, V^T from transposing LDS reads (ds_read_b64_tr_b16),
//    P^T the score accumulator re-packed to bf16 in place.
//  * Software pipeline: the P V MFMAs of tile t-1 run beside the softmax of tile t (row max,
//    reference, probabilities), so the VALU work hides under the matrix core and only one
//    tile's scores are live.
//  * Softmax against a fixed per-row reference: a row's reference is the max of its first tile
//    with a visible key, and later probabilities 2^(s - ref) are taken against it as long as
//    every later score stays within 2^kRefSlack of it (fp32 O and bf16 P stay far from
//    overflow), so O is never rescaled. Each row also tracks its exact max; a workgroup in
//    which some row passes the slack redoes its pass with every row's exact max as reference
//    (no score can pass it then). Causal masks only on tiles a diagonal crosses (a separate
//    copy of the step, chosen once per tile).
//  * The P V MFMAs are issued as inline asm so that O can live in AGPRs while the scores use
//    the MFMA's VGPR form (the compiler picks one accumulator form per function).
//  * Work order (work_order.h): virtual rows in the caller's order, else last row first; inside
//    a row its tiles from the last (longest key range) to the first, the key ranges of one
//    tile adjacent when the row's keys are split.
#include <type_traits>

#include "attn_core.h"
#include "wide_tile.h"
#include "work_order.h"

namespace mla {
namespace {

using namespace attn;
using wide::kRefSlack;
using wide::NBO;
using wide::o_read_fence;
using wide::o_zero;
using wide::p_fence;
using wide::pv_mfma;
using wide::Softmax;

constexpr int WBM = 128;   // rows per workgroup
constexpr int TK = 32;     // keys per KV tile
constexpr int DL = 512, DR = 64;
constexpr int DQK = DL + DR;
constexpr int KB = DQK / 16;             // 36 k-blocks of Q K^T
constexpr int KBL = DL / 16;             // 32 of them latent
constexpr int LAT_STRIDE = DL * 2 + 16;  // 1040: an odd number of 16-byte bank slots
constexpr int ROPE_OFF = TK * LAT_STRIDE;
constexpr int TILE_BYTES = ROPE_OFF + TK * DR * 2;
constexpr int LAT_PER_WAVE = TK / 4;  // 8 latent row loads per wave and tile
constexpr int QK_AHEAD = 4;           // Q K^T operand reads in flight
constexpr int PV_AHEAD_W = 2;         // P V MFMAs' worth of V^T reads in flight
static_assert(NBO == DL / 32, "16 output column blocks of 32");

// Where the keys of one tile live: KV row of its first key and how many keys it has.
struct TileRows {
    int64_t row0;
    int rows;  // 1..TK
};

// Buffer views of one tile's rows: the base is the tile's first row, the range its valid
// rows, so a load can only touch rows of this tile. Rows past the extent repeat the last
// valid row (finite values; their scores are masked).
struct TileSrc {
    __amdgpu_buffer_rsrc_t lat_rsrc, rope_rsrc;
    int rows;
    __device__ __forceinline__ TileSrc(const char* lat, const char* rope, TileRows tr) : rows(tr.rows) {
        lat_rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)(lat + tr.row0 * (DL * 2)), 0, rows * (DL * 2), kBufferFlags);
        rope_rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)(rope + tr.row0 * (DR * 2)), 0, rows * (DR * 2), kBufferFlags);
    }
    // Latent load i (0..7) of this wave: tile row n = 4 i + wave, one 1024-byte row per load
    // (row offset in an SGPR, lane offset constant).
    __device__ __forceinline__ void lat_load(char* dst, int wave, int lane, int i) const {
        const int n = i * 4 + wave;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(lat_rsrc, (lds_void*)(dst + n * LAT_STRIDE), 16, lane * 16,
                                                 min(n, rows - 1) * (DL * 2), 0, 0);
    }
    // Rope load of this wave: rows 8 wave .. 8 wave + 7, packed at 128 bytes; lane l fills LDS
    // chunk l % 8 of row 8 wave + l / 8 from source chunk (l % 8) ^ ((row / 2) % 8), a swizzle
    // that keeps the Q K^T rope reads conflict-free.
    __device__ __forceinline__ void rope_load(char* dst, int wave, int lane) const {
        const int r = wave * 8 + (lane >> 3);
        const int c = (lane & 7) ^ ((r >> 1) & 7);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rope_rsrc, (lds_void*)(dst + ROPE_OFF + wave * 1024), 16,
                                                 min(r, rows - 1) * (DR * 2) + c * 16, 0, 0, 0);
    }
};

// Masks the scores of keys past this lane's row position: score s[i] is tile key
// 16 (i / 8) + 4 (i % 4) + 2 ((i / 4) % 2) + half, visible when <= rel_h + half (the row's
// position minus the tile's first key; a negative value masks the whole tile).
__device__ __forceinline__ void causal_mask(f32x16& s, int rel_h) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int off = 16 * (i >> 3) + 4 * (i & 3) + 2 * ((i >> 2) & 1);
        s[i] = off <= rel_h ? s[i] : -INFINITY;
    }
}

template <bool PAGED>
__global__ __launch_bounds__(NT, 1) void dense_wide_kernel(
    const __bf16* __restrict__ q, const char* __restrict__ lat, const char* __restrict__ rope,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ vrow_kv_start, const int32_t* __restrict__ positions,
    int n_vrows, int H, int64_t N_kv, float scale_log2, __bf16* __restrict__ o_out, float* __restrict__ lse_out,
    int kv_splits, int64_t split_stride, const int32_t* __restrict__ vrow_kv_len,
    const int32_t* __restrict__ block_table, int bt_stride, const int32_t* __restrict__ vrow_req,
    const int32_t* __restrict__ vrow_splits, const int32_t* __restrict__ vrow_order) {
    // KV tile buffers: three separate LDS objects, so the compiler can tell that loads streaming
    // into one never touch the others and does not wait for them before reading a tile.
    __shared__ __attribute__((aligned(1024))) char kv0[TILE_BYTES];
    __shared__ __attribute__((aligned(1024))) char kv1[TILE_BYTES];
    __shared__ __attribute__((aligned(1024))) char kv2[TILE_BYTES];
    __shared__ int sh[NT];
    __shared__ int s_maxpos[NT / 64];
    __shared__ int s_redo[NT / 64];

    // workgroup = (virtual row, row tile, key range)
    const sched::DenseWork wk =
        sched::find_work<WBM, NT>((int)blockIdx.x, cu, n_vrows, H, vrow_splits, vrow_order, kv_splits, sh);
    const int v = wk.v, tile = wk.tile, split = wk.split;
    if (v < 0) return;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int half = lane >> 5;
    const int l32 = lane & 31;

    const int tok0 = cu[v];
    const int nrows = (cu[v + 1] - tok0) * H;
    const int rloc = tile * WBM + wave * 32 + l32;  // row inside the virtual row
    const bool valid = rloc < nrows;
    const int64_t grow = (int64_t)tok0 * H + rloc;
    const int pos = valid ? positions[tok0 + rloc / H] : -1;
    const int64_t kv0r = __builtin_amdgcn_readfirstlane(vrow_kv_start[v]);

    int mp = pos;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) mp = max(mp, __shfl_xor(mp, off));
    if (lane == 0) s_maxpos[wave] = mp;

    // Q^T fragments: lane holds row l32, elements [16 kb + 8 half, +8) of every k-block.
    bf16x8 qf[KB];
    {
        const __bf16* qrow = q + grow * DQK + 8 * half;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) qf[kb] = valid ? *reinterpret_cast<const bf16x8*>(qrow + kb * 16) : bf16x8{};
    }
    __syncthreads();
    int kv_hi = s_maxpos[0];
#pragma unroll
    for (int w = 1; w < NT / 64; ++w) kv_hi = max(kv_hi, s_maxpos[w]);
    kv_hi = kv_hi + 1;
    // Key range of this split: whole 64-key blocks of the request's KV (the split rule does not
    // depend on the kernel's tile size).
    int key_lo = 0;
    if (wk.nsplit > 1) {
        int key_hi;
        sched::split_range(vrow_kv_len[v], split, wk.nsplit, key_lo, key_hi);
        kv_hi = min(kv_hi, key_hi);
    }
    float* const lse0 = lse_out;
    if (kv_splits > 1) {
        o_out += split * split_stride * H * DL;
        lse_out += split * split_stride * H;
    }
    kv_hi = __builtin_amdgcn_readfirstlane(kv_hi);
    const int kt0 = __builtin_amdgcn_readfirstlane(key_lo / TK);
    // smallest position among this wave's rows: tiles at or below it need no mask
    int pmin = valid ? pos : INT32_MAX;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) pmin = min(pmin, __shfl_xor(pmin, off));
    pmin = __builtin_amdgcn_readfirstlane(pmin);
    // last key (request-relative) a load may touch
    const int64_t last = PAGED ? (int64_t)kv_hi - 1 : min((int64_t)kv_hi - 1, N_kv - 1 - kv0r);
    // Paged KV: ids of 64 consecutive 64-row blocks [bw_base, bw_base + 64), one per lane, read
    // by v_readlane; the next 64 are fetched once the window's last block has been used. Ids are
    // clamped into the cache as they load (an id outside it reads wrong rows of the cache); the
    // cache holds whole blocks, so every tile -- half a block, or the last key alone -- stays
    // inside it.
    const int32_t* bt_row = PAGED ? block_table + (int64_t)vrow_req[v] * bt_stride : nullptr;
    const int nblk = (int)(last >> 6) + 1;
    const int blk_max = (int)(N_kv >> 6) - 1;
    int bw_base = 0, bw_v = 0;
    auto bw_load = [&](int base) __attribute__((always_inline)) {
        bw_base = base;
        bw_v = min(max(bt_row[min(base + lane, min(nblk, bt_stride) - 1)], 0), blk_max);
    };
    auto tile_rows = [&](int kt) __attribute__((always_inline)) -> TileRows {
        const int64_t tb = min((int64_t)kt * TK, last);
        TileRows tr;
        tr.rows = (int)min((int64_t)TK, last - tb + 1);
        if constexpr (PAGED) {
            const int t = (int)(tb >> 6);
            tr.row0 = (int64_t)__builtin_amdgcn_readlane(bw_v, t - bw_base) * 64 + (tb & 63);
            if (t == bw_base + 63 && (tb & 32)) bw_load(bw_base + 64);
        } else {
            tr.row0 = kv0r + tb;
        }
        return tr;
    };

    f32x16 acc_o[NBO];
    float m_ref = -INFINITY;   // reference max (log2 domain) of this lane's row
    float m_true = -INFINITY;  // exact max of the row's scores so far (log2 domain)
    float l_run = 0.0f;        // running sum over this lane's share of the keys
    bool over = false;         // a score of this row passed the reference's slack

    // Per-lane LDS offsets inside a tile: Q K^T reads of score row l32 (8 elements at 8 half of
    // each k-block; rope rows swizzled as they were loaded); V^T reads (first of the two per
    // MFMA) at LDS row kperm(4 half + (lane % 16) / 4) of a 16-key half, dims
    // 16 ((lane / 16) % 2) + 4 (lane % 4); the second read is 2 rows further.
    const int krow = 16 * (l32 >> 4) + kperm(l32 & 15);
    const int k_lat_off = krow * LAT_STRIDE + 16 * half;
    int k_rope_off[KB - KBL];
#pragma unroll
    for (int kb = 0; kb < KB - KBL; ++kb)
        k_rope_off[kb] = ROPE_OFF + krow * (DR * 2) + 16 * ((2 * kb + half) ^ ((krow >> 1) & 7));
    const int v_off = kperm(4 * half + ((lane & 15) >> 2)) * LAT_STRIDE + 2 * (16 * ((lane >> 4) & 1) + 4 * (lane & 3));

    const int n_tiles = (kv_hi + TK - 1) / TK;

    // Lane offsets re-derived every tile (laundered through an empty asm), so the compiler forms
    // a handful of base addresses per tile and reaches the rest through the 16-bit immediate
    // offset, instead of hoisting one address register per read and buffer out of the loop.
    struct LaneOffs {
        int lat, v, rope[KB - KBL];
    };
    auto lane_offs = [&]() __attribute__((always_inline)) {
        LaneOffs o;
        o.lat = k_lat_off;
        o.v = v_off;
#pragma unroll
        for (int kb = 0; kb < KB - KBL; ++kb) o.rope[kb] = k_rope_off[kb];
        asm volatile("" : "+v"(o.lat), "+v"(o.v), "+v"(o.rope[0]), "+v"(o.rope[1]), "+v"(o.rope[2]), "+v"(o.rope[3]));
        return o;
    };

    // V^T operands of the P V MFMAs, PV_AHEAD_W MFMAs ahead: MFMA m (16 column blocks x two
    // 16-key halves) reads two transposing 4-key slices of column block m % 16.
    constexpr int NVB = PV_AHEAD_W + 1;
    struct VOps {
        bf16x8 v[NVB];
    };
    auto vread = [&](VOps& vo, const char* kvp, const LaneOffs& lo, int m) __attribute__((always_inline)) {
        const int h = m / NBO, d = m % NBO;
        const char* vb = kvp + lo.v;
        const int o0 = 16 * h * LAT_STRIDE + d * 64;
        const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vb + o0));
        const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vb + (o0 + 2 * LAT_STRIDE)));
        vo.v[m % NVB] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
    };

    // Q K^T of tile kvt: S^T[key, row] for key score_key(0, half, i) of the tile, row l32, with
    // the next tile's loads (8 latent rows and 1 rope load per wave) among the MFMAs and, when
    // a P V follows (PRE), its first V^T reads among the last MFMAs, which have no Q K^T reads
    // left to overlap.
    auto qk_tile = [&](const char* kvt, const LaneOffs& lo, const TileSrc& src, char* nxt, const char* kvp, VOps& vo,
                       auto pre_tag) __attribute__((always_inline)) {
        constexpr bool PRE = decltype(pre_tag)::value;
        bf16x8 qa[KB];
        auto rd = [&](int kb) __attribute__((always_inline)) {
            const char* ap = kb < KBL ? kvt + lo.lat + kb * 32 : kvt + lo.rope[kb - KBL];
            qa[kb] = *reinterpret_cast<const bf16x8*>(ap);
        };
        f32x16 s = f32x16{};
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < LAT_PER_WAVE; ++i) src.lat_load(nxt, wave, lane, i);
        src.rope_load(nxt, wave, lane);
#pragma unroll
        for (int kb = 0; kb < QK_AHEAD; ++kb) rd(kb);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            if (kb + QK_AHEAD < KB) rd(kb + QK_AHEAD);
            s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[kb], qf[kb], s, 0, 0, 0);
        }
        if constexpr (PRE) {
#pragma unroll
            for (int m = 0; m < PV_AHEAD_W; ++m) vread(vo, kvp, lo, m);
        }
        // QK_AHEAD operand reads first, then per MFMA one read, and a load of the next tile
        // after every fourth MFMA, so the vector memory pipe drains them under the matrix core;
        // the V^T reads (two per P V MFMA) go among the last MFMAs.
        __builtin_amdgcn_sched_group_barrier(0x100, QK_AHEAD, 0);
#pragma unroll
        for (int k = 0; k < KB; ++k) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            if (k + QK_AHEAD < KB)
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            else if (PRE && k + QK_AHEAD - KB < PV_AHEAD_W)
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            if (k % 4 == 0 && k / 4 < LAT_PER_WAVE + 1) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        return s;
    };

    // P V of the previous tile (kvp, probabilities pp) beside the softmax of this tile's scores
    // s: 32 MFMAs (16 column blocks x two 16-key halves), V^T reads PV_AHEAD_W MFMAs ahead, and
    // one piece of the softmax per MFMA, each chunk fenced so the interleave holds.
    auto pv_softmax = [&](const char* kvp, const LaneOffs& lo, VOps& vo, bf16x8 (&pp)[2], const f32x16& s,
                          Softmax& sm, bf16x8 (&pn)[2], auto do_pv, auto do_soft, auto pre_tag)
        __attribute__((always_inline)) {
        constexpr bool PV = decltype(do_pv)::value, SOFT = decltype(do_soft)::value;
        constexpr bool PRE = decltype(pre_tag)::value;  // the first V^T reads were issued already
        constexpr int NM = 2 * NBO;
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (PV) {
            p_fence(pp);
            if constexpr (!PRE) {
#pragma unroll
                for (int m = 0; m < PV_AHEAD_W; ++m) vread(vo, kvp, lo, m);
            }
        }
#pragma unroll
        for (int m = 0; m < NM; ++m) {
            if constexpr (PV) {
                if (m + PV_AHEAD_W < NM) vread(vo, kvp, lo, m + PV_AHEAD_W);
                pv_mfma(acc_o[m % NBO], vo.v[m % NVB], pp[m / NBO]);
            }
            if constexpr (SOFT) sm.piece(m, s, m_ref, scale_log2, pn);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // One tile step: wait for tile kt (buffer cur), issue tile kt+1 into nxt, Q K^T on cur;
    // then P V of tile kt-1 (buffer prv, probabilities pprev) beside this tile's softmax. The
    // step's only branch (the causal mask) touches the scores alone, so O keeps one home in
    // AGPRs; a tile past the row's last one (kt >= n_tiles) is masked whole.
    bf16x8 pprev[2];
    auto step = [&](const char* cur, const char* prv, char* nxt, int kt, auto has_prev) __attribute__((always_inline)) {
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's loads of tile kt landed
        __syncthreads();                     // ... and every wave's; buffer nxt is free
        const TileSrc src(lat, rope, tile_rows(kt + 1));  // clamped past the last tile
        const LaneOffs lo = lane_offs();
        VOps vo;
        f32x16 s = qk_tile(cur, lo, src, nxt, prv, vo, has_prev);
        // wave-uniform: a causal diagonal crosses this tile, or it is past the last one (the
        // branch touches only the scores, never O)
        if (kt * TK + TK - 1 > pmin || kt >= n_tiles) causal_mask(s, (kt < n_tiles ? pos - kt * TK : -1) - half);
        Softmax sm;
        bf16x8 pn[2];
        pv_softmax(prv, lo, vo, pprev, s, sm, pn, has_prev, std::true_type{}, has_prev);
        m_ref = sm.mn;
        m_true = fmaxf(m_true, sm.mloc);
        over = over || sm.over;
        l_run += sm.l;
        pprev[0] = pn[0];
        pprev[1] = pn[1];
    };
    // P V of the last tile.
    auto last_pv = [&](const char* kvp) __attribute__((always_inline)) {
        const LaneOffs lo = lane_offs();
        Softmax sm;
        bf16x8 pn[2];
        const f32x16 s{};
        VOps vo;
        pv_softmax(kvp, lo, vo, pprev, s, sm, pn, std::true_type{}, std::false_type{}, std::false_type{});
    };

    // Pass 0 against first-tile references; pass 1 only if some row of the workgroup passed
    // its reference's slack, against every row's exact max.
    for (int pass = 0;; ++pass) {
#pragma unroll
        for (int d = 0; d < NBO; ++d) o_zero(acc_o[d]);
        l_run = 0.0f;
        m_ref = pass == 0 ? -INFINITY : m_true;
        pprev[0] = pprev[1] = bf16x8{};
        if (kt0 < n_tiles) {  // workgroup-uniform; an empty key range leaves O = 0, LSE = -inf
            if constexpr (PAGED) bw_load(min(kt0 >> 1, nblk - 1) & ~63);
            {
                const TileSrc first(lat, rope, tile_rows(kt0));
#pragma unroll
                for (int i = 0; i < LAT_PER_WAVE; ++i) first.lat_load(kv0, wave, lane, i);
                first.rope_load(kv0, wave, lane);
            }
            // tile i (from kt0) sits in buffer i % 3: the first step has no P V before it, then
            // groups of three steps (the count padded up with fully masked tiles), so the loop
            // body has no internal exit and the last tile is in kv0
            step(kv0, kv2, kv1, kt0, std::false_type{});
            const int n_iter = (n_tiles - kt0 - 1 + 2) / 3;
            int kt = kt0 + 1;
            for (int it = 0; it < n_iter; ++it, kt += 3) {
                step(kv1, kv0, kv2, kt, std::true_type{});
                step(kv2, kv1, kv0, kt + 1, std::true_type{});
                step(kv0, kv2, kv1, kt + 2, std::true_type{});
            }
            last_pv(kv0);
        }
        __builtin_amdgcn_s_waitcnt(0x0F70);  // loads issued after the last tile landed before LDS is reused
        if (pass > 0) break;
        if (lane == 0) s_redo[wave] = __ballot(over) != 0;
        __syncthreads();
        int redo = 0;
#pragma unroll
        for (int w = 0; w < NT / 64; ++w) redo |= s_redo[w];
        __syncthreads();
        if (!redo) break;  // workgroup-uniform
    }
    o_read_fence(acc_o);

    // Row sum: this lane's share + the other half-wave's.
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    if (valid) {
        __bf16* orow = o_out + grow * DL;
#pragma unroll
        for (int d = 0; d < NBO; ++d) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                bf16x4 y;
#pragma unroll
                for (int e = 0; e < 4; ++e) y[e] = (__bf16)(acc_o[d][4 * g + e] * inv);
                *reinterpret_cast<bf16x4*>(orow + d * 32 + 8 * g + 4 * half) = y;
            }
        }
        if (half == 0) lse_out[grow] = (m_ref + __builtin_amdgcn_logf(l_tot)) * kLn2;
    }
    sched::mark_empty_slices(lse0, grow, valid && half == 0, split, wk.nsplit, kv_splits, split_stride, H);
}

template <bool PAGED>
hipError_t launch_wide(const mla_partial_args& a, hipStream_t stream) {
    const int64_t grid = (((int64_t)a.T_loc * a.H + WBM - 1) / WBM + a.n_vrows) * a.kv_splits;
    hipLaunchKernelGGL((dense_wide_kernel<PAGED>), dim3((unsigned)grid), dim3(NT), 0, stream, (const __bf16*)a.q,
                       (const char*)a.latent_kv, (const char*)a.rope_k, a.cu_seqlens_q, a.vrow_kv_start, a.positions,
                       a.n_vrows, a.H, a.N_kv, a.scale * kLog2e, (__bf16*)a.o_partial, a.lse, a.kv_splits,
                       a.split_stride, a.vrow_kv_len, a.block_table, a.bt_stride, a.vrow_req,
                       a.kv_splits > 1 ? a.vrow_splits : nullptr, a.vrow_order);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_dense_wide_partial(const mla_partial_args& a, hipStream_t stream) {
    return a.block_table ? launch_wide<true>(a, stream) : launch_wide<false>(a, stream);
}

}  // namespace mla
