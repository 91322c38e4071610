// Rank-local sparse MLA partial attention over bf16 latent rows -- a bf16 cache, or the
// workspace that pcp_kv_dequant_fp8 fills from an fp8 cache once per step (sparse BF16 CP prefill
// on a dequantised workspace: "DeepSeek-V4.1: Prefill support CP with multistream forward
// prepare (4/N)", commit list, "Reuse shared compressed KV dequantization in V4.1 CP prefill";
// the partial itself: "[DeepSeekV4][PCP] Enable context-parallel prefill for hybrid KV and
// MegaMoE", "Purpose"). The key set of a query is that of sparse_keys.h: its selected indices in
// [0, p] outside the window, plus the window, inside the key range of its split.
//
// Work decomposition
//  * A workgroup of two waves owns one token and a group of up to 64 heads (and one key range
//    when the keys are split); each wave owns 32 heads outright with the per-wave tile compute of
//    wide_tile.h: Q^T in VGPRs, the whole O^T in AGPRs, a wave-local softmax, so no scores or
//    probabilities cross waves. Two workgroups share a CU (74 KB of LDS each), one wave per
//    SIMD, each stalling on its own tiles only.
//  * Key tiles of 32 slots: the selected indices in groups of 32, then the window. A tile with no
//    key of the set is skipped: a 64-bit mask of the selected-index tiles is built once from the
//    whole index row, and the live window tiles are one contiguous range.
//  * A key's 1 KB latent row moves HBM -> LDS with one wave-wide direct-to-LDS load (row offset
//    in an SGPR), its rope row with an eighth of one; the next tile's 32 rows stream into the
//    second buffer among this tile's Q K^T MFMAs, so a gather has a whole tile of compute to land.
//    The rows come from a pipeline of small loads one tile apart: the tile's selected indices,
//    then (paged) the block-table entries of their keys, then the rows themselves.
//  * Per tile: S^T = K Q^T (36 MFMAs), the key mask, the softmax against the fixed reference,
//    O^T += V^T P^T (32 MFMAs); one barrier per tile.
#include "sparse_keys.h"
#include "wide_tile.h"

namespace mla {
namespace {

using namespace attn;
using wide::NBO;

constexpr int TK = 32;    // key slots per tile
constexpr int NTW = 128;  // threads per workgroup: two waves of 32 rows
constexpr int DL = 512, DR = 64;
constexpr int DQK = DL + DR;
constexpr int KB = DQK / 16;             // 36 k-blocks of Q K^T
constexpr int KBL = DL / 16;             // 32 of them latent
constexpr int LAT_STRIDE = DL * 2 + 16;  // 1040: an odd number of 16-byte bank slots
constexpr int ROPE_OFF = TK * LAT_STRIDE;
constexpr int TILE_BYTES = ROPE_OFF + TK * DR * 2;
constexpr int LAT_PER_WAVE = TK / 2;  // latent row loads per wave and tile
constexpr int ROPE_PER_WAVE = 2;      // rope loads (8 rows of 128 bytes each) per wave and tile
constexpr int QK_AHEAD = 4;           // Q K^T operand reads in flight
constexpr int PV_AHEAD = 2;           // P V MFMAs' worth of V^T reads in flight
constexpr int SEL_TILES = MAX_TOPK / TK;
static_assert(SEL_TILES == 64, "one bit per selected-index tile in a 64-bit mask");
static_assert(TILE_BYTES >= Q_REGION_BYTES && TILE_BYTES >= 32 * DL * 2,
              "a wave's Q rows and O rows fit a tile buffer");
static_assert(2 * TILE_BYTES + 1024 <= 160 * 1024 / 2, "two workgroups per CU");
static_assert(2 * (LAT_PER_WAVE + ROPE_PER_WAVE) == KB, "one load after every second Q K^T MFMA");

template <bool PAGED>
__global__ __launch_bounds__(NTW, 1) void sparse_wide_kernel(
    const __bf16* __restrict__ q, const char* __restrict__ lat, const char* __restrict__ rope,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ vrow_kv_start, const int32_t* __restrict__ positions,
    const int32_t* __restrict__ topk_idx, int topk, int window, int n_vrows, int H, int64_t N_kv, float scale_log2,
    __bf16* __restrict__ o_out, float* __restrict__ lse_out, int kv_splits, int64_t split_stride,
    const int32_t* __restrict__ vrow_kv_len, const int32_t* __restrict__ block_table, int bt_stride,
    const int32_t* __restrict__ vrow_req, const int32_t* __restrict__ vrow_splits) {
    // Tile buffers: two separate LDS objects, so the compiler can tell that loads streaming into
    // one never touch the other. Each first holds one wave's Q rows, last its O rows.
    __shared__ __attribute__((aligned(1024))) char kv0[TILE_BYTES];
    __shared__ __attribute__((aligned(1024))) char kv1[TILE_BYTES];
    __shared__ uint64_t s_live[2];
    __shared__ int s_redo[2];

    const SparseWork wk =
        sparse_work(H, kv_splits, cu, n_vrows, vrow_kv_start, positions, vrow_kv_len, vrow_splits);
    if (wk.split >= wk.nsplit) return;  // a range past the row's count: no keys, nothing to write
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int half = lane >> 5;
    const int l32 = lane & 31;
    float* const lse0 = lse_out;
    if (kv_splits > 1) {
        o_out += wk.split * split_stride * H * DL;
        lse_out += wk.split * split_stride * H;
    }
    const int head = wk.hg * BM + wave * 32 + l32;
    const bool valid = head < H;  // rows past H (a last head group under 64) stay idle
    const int64_t grow = (int64_t)wk.tok * H + head;
    // Buffer views of the latent and rope rows from row_base (the request's first row when
    // packed, the cache's first row when paged); the caller keeps N_kv * DL * 2 below 2^32.
    // Every row is clamped into the cache before an offset is formed from it (a paged block id
    // outside the cache reads a wrong row of the cache, never memory outside it).
    const int64_t row_base = PAGED ? 0 : wk.kv0;
    const int last_row = (int)(N_kv - 1 - row_base);
    const __amdgpu_buffer_rsrc_t lat_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(lat + row_base * (DL * 2)), 0, (int)(uint32_t)((N_kv - row_base) * (DL * 2)), kBufferFlags);
    const __amdgpu_buffer_rsrc_t rope_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(rope + row_base * (DR * 2)), 0, (int)(uint32_t)((N_kv - row_base) * (DR * 2)), kBufferFlags);
    const int32_t* bt_row = PAGED ? block_table + (int64_t)vrow_req[wk.lo_v] * bt_stride : nullptr;

    // Q rows of this wave into its tile buffer; in flight while the live-tile mask is built.
    char* const q_region = wave == 0 ? kv0 : kv1;
    dma_q_rows<1>(__builtin_amdgcn_make_buffer_rsrc((void*)(q + (int64_t)wk.tok * H * DQK), 0, H * DQK * 2,
                                                    kBufferFlags),
                  wk.hg * BM + wave * 32, H, q_region, 0, lane);

    // The key set in this key range. A selected index counts when it lies in [key_lo, key_hi),
    // in [0, p] and before the window (the window supplies its own keys).
    const int p = wk.p, key_lo = wk.key_lo, key_hi = wk.key_hi;
    const int win_lo = max(0, p - window + 1);  // first window key (window > 0)
    auto sel_ok = [&](int e) { return e >= key_lo && e < key_hi && e <= p && (window == 0 || e < win_lo); };
    const int n_sel = (topk + TK - 1) / TK;
    const int32_t* const idx_row = topk_idx + (int64_t)wk.tok * topk;
    {
        // Live selected-index tiles: thread t holds entries t + 128 j, which lie in tile
        // 4 j + 2 wave (lanes 0-31) or 4 j + 2 wave + 1 (lanes 32-63). All loads go out first.
        constexpr int PER = MAX_TOPK / NTW;
        int e[PER];
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int i = tid + j * NTW;
            e[j] = i < topk ? idx_row[i] : -1;
        }
        uint64_t live = 0;
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const uint64_t b = __ballot(sel_ok(e[j]));
            const int t = 4 * j + 2 * wave;
            live |= ((uint64_t)((uint32_t)b != 0u) << t) | ((uint64_t)((uint32_t)(b >> 32) != 0u) << (t + 1));
        }
        if (lane == 0) s_live[wave] = live;
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's Q rows landed
    __syncthreads();                     // ... and both waves' halves of the mask are written
    const uint64_t live_v = s_live[0] | s_live[1];
    const uint64_t live = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(live_v >> 32)) << 32) |
                          (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)live_v);
    bf16x8 qf[KB];
    read_q_frags(q_region, lane, qf);
    lds_barrier();  // both waves hold their Q fragments: the tiles may overwrite the Q rows

    // Tiles: [0, n_sel) selected indices, then the window's; t_end ends the sequence. The live
    // window tiles are those holding keys [max(win_lo, key_lo), min(p + 1, key_hi)).
    const int t_end = n_sel + (window + TK - 1) / TK;
    int w_first = t_end, w_last = -1;
    {
        const int a = max(win_lo, key_lo), b = min(p + 1, key_hi);
        if (window > 0 && a < b) {
            w_first = n_sel + (a - win_lo) / TK;
            w_last = n_sel + (b - 1 - win_lo) / TK;
        }
    }
    auto next_tile = [&](int t) -> int {  // first live tile after t, else t_end (workgroup-uniform)
        const int t1 = t + 1;
        if (t1 < n_sel) {
            const uint64_t m = live & (~0ull << t1);
            if (m) return (int)__builtin_ctzll(m);
        }
        const int w = max(t1, w_first);
        return w <= w_last ? w : t_end;
    };

    // Row pipeline of tile t for slot lane % 32 (lanes 32-63 repeat lanes 0-31):
    //  a) the selected index (a load; -1 past the list or for a window tile);
    //  b) the slot's key and whether it counts (a slot outside the set reads key 0, a written
    //     key whose value meets a zero probability) and, paged, its block id (a load);
    //  c) the key's row, clamped into the cache.
    const int slot = lane & (TK - 1);
    auto stage_a = [&](int t) -> int {
        const int i = t * TK + slot;
        return t < n_sel && i < topk ? idx_row[i] : -1;
    };
    auto stage_b = [&](int t, int ia, bool& ok) -> int {
        int key;
        if (t < n_sel) {
            ok = sel_ok(ia);
            key = ia;
        } else {
            const int w = (t - n_sel) * TK + slot;
            key = win_lo + w;
            ok = t < t_end && w < window && key <= p && key >= key_lo && key < key_hi;
        }
        return ok ? key : 0;
    };
    auto stage_b_load = [&](int key) -> int {
        if constexpr (PAGED) return bt_row[min(key >> 6, bt_stride - 1)];
        return 0;
    };
    auto stage_c = [&](int key, int blk) -> int {
        const int row = PAGED ? blk * 64 + (key & 63) : key;
        return max(min(row, last_row), 0);
    };

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
    // Lane offsets re-derived every tile (laundered through an empty asm), so the compiler forms
    // a handful of base addresses per tile and reaches the rest through immediate offsets.
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

    // Loads of a tile whose slot rows are `rows`: latent load i (0..15) of this wave is tile row
    // 2 i + wave, one 1024-byte row; rope load i (0..1) covers tile rows 8 (2 wave + i) + l / 8,
    // lane l filling chunk l % 8 of its row from source chunk (l % 8) ^ ((row / 2) % 8), the
    // swizzle the Q K^T rope reads expect. rope_src gives each lane's source offsets.
    auto lat_load = [&](char* dst, int rows, int i) __attribute__((always_inline)) {
        const int n = 2 * i + wave;
        const uint32_t soff = (uint32_t)__builtin_amdgcn_readlane(rows, n) * (DL * 2);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(lat_rsrc, (lds_void*)(dst + n * LAT_STRIDE), 16, lane * 16, soff, 0,
                                                 0);
    };
    auto rope_src = [&](int rows, uint32_t (&ro)[ROPE_PER_WAVE]) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < ROPE_PER_WAVE; ++i) {
            const int r = 8 * (2 * wave + i) + (lane >> 3);
            const int c = (lane & 7) ^ ((r >> 1) & 7);
            ro[i] = (uint32_t)__shfl(rows, r) * (DR * 2) + c * 16;
        }
    };
    auto rope_load = [&](char* dst, uint32_t voff, int i) __attribute__((always_inline)) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rope_rsrc, (lds_void*)(dst + ROPE_OFF + (2 * wave + i) * 1024), 16,
                                                 voff, 0, 0, 0);
    };

    f32x16 acc_o[NBO];
    float m_ref = -INFINITY;   // reference max (log2 domain) of this lane's row
    float m_true = -INFINITY;  // exact max of the row's scores so far (log2 domain)
    float l_run = 0.0f;        // running sum over this lane's share of the keys
    bool over = false;         // a score of this row passed the reference's slack

    // Q K^T of the tile in kvt, with the next tile's loads (rows `rows`, into nxt) one after
    // every second MFMA, so the vector memory pipe drains them under the matrix core.
    auto qk_tile = [&](const char* kvt, const LaneOffs& lo, char* nxt, int rows, const uint32_t (&ro)[ROPE_PER_WAVE])
        __attribute__((always_inline)) {
        bf16x8 qa[KB];
        auto rd = [&](int kb) __attribute__((always_inline)) {
            const char* ap = kb < KBL ? kvt + lo.lat + kb * 32 : kvt + lo.rope[kb - KBL];
            qa[kb] = *reinterpret_cast<const bf16x8*>(ap);
        };
        f32x16 s = f32x16{};
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < LAT_PER_WAVE; ++i) lat_load(nxt, rows, i);
#pragma unroll
        for (int i = 0; i < ROPE_PER_WAVE; ++i) rope_load(nxt, ro[i], i);
#pragma unroll
        for (int kb = 0; kb < QK_AHEAD; ++kb) rd(kb);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            if (kb + QK_AHEAD < KB) rd(kb + QK_AHEAD);
            s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[kb], qf[kb], s, 0, 0, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x100, QK_AHEAD, 0);
#pragma unroll
        for (int k = 0; k < KB; ++k) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            if (k + QK_AHEAD < KB) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            if (k % 2 == 0) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        return s;
    };

    // P V of the tile in kvp: 32 MFMAs (16 column blocks x two 16-key halves), each reading two
    // transposing 4-key slices of V^T, PV_AHEAD MFMAs ahead.
    auto pv_tile = [&](const char* kvp, const LaneOffs& lo, bf16x8 (&pp)[2]) __attribute__((always_inline)) {
        constexpr int NVB = PV_AHEAD + 1;
        constexpr int NM = 2 * NBO;
        bf16x8 vv[NVB];
        auto vread = [&](int m) __attribute__((always_inline)) {
            const int h = m / NBO, d = m % NBO;
            const char* vb = kvp + lo.v;
            const int o0 = 16 * h * LAT_STRIDE + d * 64;
            const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vb + o0));
            const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vb + (o0 + 2 * LAT_STRIDE)));
            vv[m % NVB] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
        };
        __builtin_amdgcn_sched_barrier(0);
        wide::p_fence(pp);
#pragma unroll
        for (int m = 0; m < PV_AHEAD; ++m) vread(m);
#pragma unroll
        for (int m = 0; m < NM; ++m) {
            if (m + PV_AHEAD < NM) vread(m + PV_AHEAD);
            wide::pv_mfma(acc_o[m % NBO], vv[m % NVB], pp[m / NBO]);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // Pipeline state entering a step: tile t0 (its rows in buffer cur, its valid-slot bits
    // okb0), tile t1 past stage b (key1, okb1, paged block id blk1), tile t2 past stage a (ia2).
    int t0, t1, t2, key1, blk1, ia2;
    uint64_t okb0, okb1;
    auto step = [&](const char* cur, char* nxt) __attribute__((always_inline)) {
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): tile t0's rows and the pipeline's loads landed
        __syncthreads();                     // ... for both waves; buffer nxt is free
        const int rows1 = stage_c(key1, blk1);
        uint32_t ro[ROPE_PER_WAVE];
        rope_src(rows1, ro);
        bool ok2;
        const int key2 = stage_b(t2, ia2, ok2);
        const uint64_t okb2 = __ballot(ok2);
        const int blk2 = stage_b_load(key2);
        const int t3 = next_tile(t2);
        const int ia3 = stage_a(t3);
        const LaneOffs lo = lane_offs();
        f32x16 s = qk_tile(cur, lo, nxt, rows1, ro);
        mask_keys(s, okb0, 0, half);
        wide::Softmax sm;
        bf16x8 pn[2];
#pragma unroll
        for (int k = 0; k < wide::SOFTMAX_PIECES; ++k) sm.piece(k, s, m_ref, scale_log2, pn);
        m_ref = sm.mn;
        m_true = fmaxf(m_true, sm.mloc);
        over = over || sm.over;
        l_run += sm.l;
        pv_tile(cur, lo, pn);
        t0 = t1;
        okb0 = okb1;
        t1 = t2;
        key1 = key2;
        okb1 = okb2;
        blk1 = blk2;
        t2 = t3;
        ia2 = ia3;
    };

    // Pass 0 against first-tile references; pass 1 only if some row of the workgroup passed its
    // reference's slack, against every row's exact max.
    for (int pass = 0;; ++pass) {
#pragma unroll
        for (int d = 0; d < NBO; ++d) wide::o_zero(acc_o[d]);
        l_run = 0.0f;
        m_ref = pass == 0 ? -INFINITY : m_true;
        t0 = next_tile(-1);
        t1 = next_tile(t0);
        t2 = next_tile(t1);
        if (t0 < t_end) {  // workgroup-uniform; no key leaves O = 0, LSE = -inf
            const int ia0 = stage_a(t0), ia1 = stage_a(t1);
            ia2 = stage_a(t2);
            __builtin_amdgcn_s_waitcnt(0x0F70);
            bool ok0, ok1;
            const int key0 = stage_b(t0, ia0, ok0);
            okb0 = __ballot(ok0);
            const int blk0 = stage_b_load(key0);
            key1 = stage_b(t1, ia1, ok1);
            okb1 = __ballot(ok1);
            blk1 = stage_b_load(key1);
            __builtin_amdgcn_s_waitcnt(0x0F70);
            const int rows0 = stage_c(key0, blk0);
            uint32_t ro[ROPE_PER_WAVE];
            rope_src(rows0, ro);
#pragma unroll
            for (int i = 0; i < LAT_PER_WAVE; ++i) lat_load(kv0, rows0, i);
#pragma unroll
            for (int i = 0; i < ROPE_PER_WAVE; ++i) rope_load(kv0, ro[i], i);
            // tile i of the sequence sits in buffer i % 2; past the last live tile the pipeline
            // loads pad rows into the unused buffer
            while (true) {
                step(kv0, kv1);
                if (t0 >= t_end) break;
                step(kv1, kv0);
                if (t0 >= t_end) break;
            }
        }
        __builtin_amdgcn_s_waitcnt(0x0F70);  // loads issued after the last tile landed before LDS is reused
        if (pass > 0) break;
        if (lane == 0) s_redo[wave] = __ballot(over) != 0;
        __syncthreads();
        const int redo = s_redo[0] | s_redo[1];
        __syncthreads();
        if (!redo) break;  // workgroup-uniform
    }
    __syncthreads();  // both waves are past their last tile: the buffers take the O rows
    wide::o_read_fence(acc_o);

    // Epilogue: the normalised O rows of this wave go through its buffer so that each global
    // store writes one whole 1 KB row: 8-byte chunk c of row r at chunk c ^ r (r < 32), distinct
    // bank slots for the row-per-lane writes; a row's 16-byte slot l holds chunks 2l ^ r and
    // 2l + 1 ^ r, swapped when r is odd.
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    char* const region = wave == 0 ? kv0 : kv1;
    char* const lrow = region + l32 * (DL * 2);
#pragma unroll
    for (int d = 0; d < NBO; ++d) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            bf16x4 y;
#pragma unroll
            for (int e = 0; e < 4; ++e) y[e] = (__bf16)(acc_o[d][4 * g + e] * inv);
            const int c = (d * 32 + 8 * g + 4 * half) / 4;
            *reinterpret_cast<bf16x4*>(lrow + 8 * (c ^ l32)) = y;
        }
    }
    if (valid && half == 0) lse_out[grow] = (m_ref + __builtin_amdgcn_logf(l_tot)) * kLn2;
    const int n_valid = __builtin_amdgcn_readfirstlane(__popcll(__ballot(valid)) / 2);  // a prefix of the 32
    __bf16* const o_wave = o_out + (grow - l32) * DL + 8 * lane;  // this wave's first row
#pragma unroll
    for (int r = 0; r < 32; ++r) {
        if (r >= n_valid) break;  // wave-uniform
        uint4 v = *reinterpret_cast<const uint4*>(region + r * (DL * 2) + 16 * (lane ^ (r >> 1)));
        if (r & 1) v = uint4{v.z, v.w, v.x, v.y};
        *reinterpret_cast<uint4*>(o_wave + r * DL) = v;
    }
    sched::mark_empty_slices(lse0, grow, valid && half == 0, wk.split, wk.nsplit, kv_splits, split_stride, H);
}

template <bool PAGED>
hipError_t launch_wide(const mla_partial_args& a, hipStream_t stream) {
    const int64_t grid = (int64_t)a.T_loc * ((a.H + BM - 1) / BM) * a.kv_splits;
    hipLaunchKernelGGL((sparse_wide_kernel<PAGED>), dim3((unsigned)grid), dim3(NTW), 0, stream, (const __bf16*)a.q,
                       (const char*)a.latent_kv, (const char*)a.rope_k, a.cu_seqlens_q, a.vrow_kv_start, a.positions,
                       a.topk_idx, a.topk, a.window, a.n_vrows, a.H, a.N_kv, a.scale * kLog2e, (__bf16*)a.o_partial,
                       a.lse, a.kv_splits, a.split_stride, a.vrow_kv_len, a.block_table, a.bt_stride, a.vrow_req,
                       a.kv_splits > 1 ? a.vrow_splits : nullptr);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_sparse_wide_partial(const mla_partial_args& a, hipStream_t stream) {
    return a.block_table ? launch_wide<true>(a, stream) : launch_wide<false>(a, stream);
}

}  // namespace mla
