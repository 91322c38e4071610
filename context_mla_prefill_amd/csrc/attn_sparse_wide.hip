// Rank-local sparse MLA partial attention ("[DeepSeekV4][PCP] Enable context-parallel prefill
// for hybrid KV and MegaMoE", "Purpose") over bf16 latent rows -- a bf16 cache, or the workspace
// that pcp_kv_dequant_fp8 fills from an fp8 cache once per step (sparse BF16 CP prefill on a
// dequantised workspace: "DeepSeek-V4.1: Prefill support CP with multistream forward prepare
// (4/N)", commit list, "Reuse shared compressed KV dequantization in V4.1 CP prefill") -- or
// over an fp8-e4m3 cache with one fp32 scale per 64 rows, dequantised in the kernel (fp8 MLA
// cache, block 64: "[Feature][PCP] Add DeepSeek-V4.1-Flash support", "vLLM Launch Arguments").
// The key set of a query is that of sparse_keys.h: its selected indices in [0, p] outside the
// window, plus the window, inside the key range of its split.
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
//  * fp8 cache (FP8): one bf16 tile buffer (37 KB) and two 20 KB staging slots (78.6 KB of LDS:
//    still two workgroups per CU). A tile's fp8 rows (two keys per
//    wave-wide load), rope rows and 64-row scales are gathered two tiles ahead into a slot; at
//    the top of its step the workgroup dequantises the slot into the tile buffer,
//    bf16_rne(fp32(e4m3) * scale), the arithmetic of pcp_kv_dequant_fp8, so the two paths give
//    the same bf16 tiles and the same partials bit for bit. The dequantisation runs between
//    barriers; the gathers have two tiles of compute to land.
#include <type_traits>

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
static_assert(TILE_BYTES >= 32 * Q_CHUNKS * 16 && TILE_BYTES >= 32 * DL * 2,
              "a wave's Q rows and O rows fit a tile buffer");
static_assert(2 * TILE_BYTES + 1024 <= 160 * 1024 / 2, "two workgroups per CU");
static_assert(2 * (LAT_PER_WAVE + ROPE_PER_WAVE) == KB, "one load after every second Q K^T MFMA");
// fp8 staging slot: the 32 keys' E4M3 latent rows (512 bytes each), their bf16 rope rows (in the
// tile buffer's swizzled order) and the 64-row scale of each key.
constexpr int ST_ROPE = TK * DL;
constexpr int ST_SCALE = ST_ROPE + TK * DR * 2;
constexpr int STAGE_BYTES = ST_SCALE + TK * 4;
constexpr int LAT8_PER_WAVE = TK / 4;                              // fp8 latent loads (two keys each)
constexpr int FP8_LOADS = LAT8_PER_WAVE + ROPE_PER_WAVE + 1;       // per wave and tile, with the scales
constexpr int Q_HALF = 16 * Q_CHUNKS * 16;                         // 16 Q rows
constexpr int O_HALF = 16 * DL * 2;                                // 16 O rows
static_assert(STAGE_BYTES >= Q_HALF && STAGE_BYTES >= O_HALF, "16 Q or O rows fit a staging slot");
static_assert(TILE_BYTES + 2 * STAGE_BYTES + 2048 <= 160 * 1024 / 2, "two fp8 workgroups per CU");
static_assert(FP8_LOADS <= KB / 3, "one fp8 load after every third Q K^T MFMA");

// bf16_rne(fp32(e4m3) * sc) of the 16 E4M3FN codes of w (OCP decode on gfx950), in order.
__device__ __forceinline__ void dequant16(const uint4& w, float sc, bf16x8& lo, bf16x8& hi) {
    const uint32_t wv[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const auto a = __builtin_amdgcn_cvt_pk_f32_fp8(wv[j], false);  // bytes 0, 1 of the word
        const auto b = __builtin_amdgcn_cvt_pk_f32_fp8(wv[j], true);   // bytes 2, 3
        bf16x8& o = j < 2 ? lo : hi;
        const int e = 4 * (j & 1);
        o[e] = (__bf16)(a[0] * sc);
        o[e + 1] = (__bf16)(a[1] * sc);
        o[e + 2] = (__bf16)(b[0] * sc);
        o[e + 3] = (__bf16)(b[1] * sc);
    }
}

// The same values when sc is a power of two 2^e with -117 <= e <= 119: fp32(e4m3) * 2^e is
// then exact in bf16 (4 significant bits; the nonzero E4M3FN magnitudes 2^-9 .. 448 times
// such a scale stay normal and finite), and gfx950's scaled conversion computes it
// directly, two codes per instruction (it applies the power of two of its scale operand).
__device__ __forceinline__ void dequant16_pow2(const uint4& w, float sc, bf16x8& lo, bf16x8& hi) {
    const uint32_t wv[4] = {w.x, w.y, w.z, w.w};
    uint32_t o[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        o[2 * j] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(wv[j], sc, false));
        o[2 * j + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(wv[j], sc, true));
    }
    lo = __builtin_bit_cast(bf16x8, uint4{o[0], o[1], o[2], o[3]});
    hi = __builtin_bit_cast(bf16x8, uint4{o[4], o[5], o[6], o[7]});
}

// sc is +2^e with -117 <= e <= 119 (the library's quantiser makes power-of-two scales).
__device__ __forceinline__ bool pow2_scale(float sc) {
    const uint32_t b = __float_as_uint(sc);
    return ((b & 0x807FFFFFu) | (b - (10u << 23) > (236u << 23) ? 1u : 0u)) == 0;
}

template <bool PAGED, bool FP8>
__global__ __launch_bounds__(NTW, 1) void sparse_wide_kernel(
    const __bf16* __restrict__ q, const char* __restrict__ lat, const float* __restrict__ kv_scale,
    const char* __restrict__ rope,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ vrow_kv_start, const int32_t* __restrict__ positions,
    const int32_t* __restrict__ topk_idx, int topk, int window, int n_vrows, int H, int64_t N_kv, float scale_log2,
    __bf16* __restrict__ o_out, float* __restrict__ lse_out, int kv_splits, int64_t split_stride,
    const int32_t* __restrict__ vrow_kv_len, const int32_t* __restrict__ block_table, int bt_stride,
    const int32_t* __restrict__ vrow_req, const int32_t* __restrict__ vrow_splits) {
    // bf16 rows: two tile buffers. fp8 rows: the tile buffer kv0 and two staging slots. Separate
    // LDS objects, so the compiler can tell that loads streaming into one never touch another.
    // kv0 first holds wave 0's Q rows and last its O rows; wave 1's are in kv1 (bf16) or in the
    // two staging slots, 16 rows each (fp8).
    constexpr int KV1_BYTES = FP8 ? STAGE_BYTES : TILE_BYTES;
    __shared__ __attribute__((aligned(1024))) char kv0[TILE_BYTES];
    __shared__ __attribute__((aligned(16))) char kv1[KV1_BYTES];
    __shared__ __attribute__((aligned(16))) char kv2[FP8 ? STAGE_BYTES : 16];
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
    // packed, the cache's first row when paged) and of the 64-row scales; the caller keeps the
    // cache's latent bytes below 2^32.
    // Every row is clamped into the cache before an offset is formed from it (a paged block id
    // outside the cache reads a wrong row of the cache, never memory outside it).
    constexpr int LAT_ROW = FP8 ? DL : DL * 2;  // bytes of a cached latent row
    const int64_t row_base = PAGED ? 0 : wk.kv0;
    const int last_row = (int)(N_kv - 1 - row_base);
    const __amdgpu_buffer_rsrc_t lat_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(lat + row_base * LAT_ROW), 0, (int)(uint32_t)((N_kv - row_base) * LAT_ROW), kBufferFlags);
    const __amdgpu_buffer_rsrc_t scale_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void*)kv_scale, 0, FP8 ? (int)(uint32_t)(((N_kv + 63) / 64) * 4) : 0, kBufferFlags);
    const __amdgpu_buffer_rsrc_t rope_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(rope + row_base * (DR * 2)), 0, (int)(uint32_t)((N_kv - row_base) * (DR * 2)), kBufferFlags);
    const int32_t* bt_row = PAGED ? block_table + (int64_t)vrow_req[wk.lo_v] * bt_stride : nullptr;

    // This wave's 32 Q rows (at the start) and O rows (at the end) in two halves of 16 rows:
    // adjacent in its tile buffer, or for wave 1 over fp8 rows one half per staging slot.
    char* const r_lo = wave == 0 ? kv0 : kv1;
    char* const q_hi = FP8 && wave == 1 ? kv2 : r_lo + Q_HALF;
    char* const o_hi = FP8 && wave == 1 ? kv2 : r_lo + O_HALF;
    // Q rows: whole-row direct-to-LDS copies (16 rows are 18 loads), in flight while the
    // live-tile mask is built; chunk c of row r at chunk r * 72 + (c ^ q_swizzle(r)) of its half.
    {
        const __amdgpu_buffer_rsrc_t q_rsrc = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(q + (int64_t)wk.tok * H * DQK), 0, H * DQK * 2, kBufferFlags);
        const int row0 = wk.hg * BM + wave * 32;
#pragma unroll
        for (int i = 0; i < 2 * Q_HALF / 1024; ++i) {
            const int L = 64 * i + lane;
            const int r = L / Q_CHUNKS;
            const int c = (L - r * Q_CHUNKS) ^ q_swizzle(r);
            const int row = min(row0 + r, H - 1);  // rows past H read row H-1 (never stored)
            lds_dma16(q_rsrc, (uint32_t)(row * (Q_CHUNKS * 16) + c * 16),
                      i < Q_HALF / 1024 ? r_lo + 1024 * i : q_hi + 1024 * (i - Q_HALF / 1024));
        }
    }

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
    {
        const int r = l32;
        const char* qb = r < 16 ? r_lo + 16 * (r * Q_CHUNKS) : q_hi + 16 * ((r - 16) * Q_CHUNKS);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
            qf[kb] = *reinterpret_cast<const bf16x8*>(qb + 16 * ((2 * kb + half) ^ q_swizzle(r)));
    }
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
        const uint32_t soff = (uint32_t)__builtin_amdgcn_readlane(rows, n) * LAT_ROW;
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
    auto rope_load = [&](char* rope_dst, uint32_t voff, int i) __attribute__((always_inline)) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rope_rsrc, (lds_void*)(rope_dst + (2 * wave + i) * 1024), 16,
                                                 voff, 0, 0, 0);
    };
    // fp8 rows into a staging slot: latent load i (0..7) of this wave fills slots n = 4 i + 2 wave
    // (lanes 0-31) and n + 1 (lanes 32-63), 512 bytes each; the scale of slot 16 wave + l comes
    // from lane l < 16 (scale_src gives each lane's source offset).
    auto lat8_load = [&](char* st, int rows, int i) __attribute__((always_inline)) {
        const int n = 4 * i + 2 * wave;
        const int ra = __builtin_amdgcn_readlane(rows, n), rb = __builtin_amdgcn_readlane(rows, n + 1);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(lat_rsrc, (lds_void*)(st + n * DL), 16,
                                                 (uint32_t)(half ? rb : ra) * DL + l32 * 16, 0, 0, 0);
    };
    auto scale_src = [&](int rows) __attribute__((always_inline)) -> uint32_t {
        return (uint32_t)((row_base + __shfl(rows, 16 * wave + (lane & 15))) >> 6) * 4;
    };
    auto scale_load = [&](char* st, uint32_t voff) __attribute__((always_inline)) {
        if (lane < 16)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(scale_rsrc, (lds_void*)(st + ST_SCALE + 64 * wave), 4, voff, 0,
                                                     0, 0);
    };
    // A staging slot into the tile buffer kv0: each thread converts 8 chunks of 16 codes (chunk
    // k: tile row k / 32, codes 16 (k % 32) ..) in two batches of 4, a batch's reads all issued
    // before any is converted; the rope rows are copied.
    auto dequant = [&](const char* st) __attribute__((always_inline)) {
        constexpr int NCH = TK * DL / 16 / NTW, BATCH = 4;
        static_assert(NCH % BATCH == 0, "whole batches");
        // the scales of this thread's chunks (chunk c: tile row (c NTW + tid) / 32); when all of
        // the wave's are powers of two the scaled conversion does the tile (the library's
        // quantiser writes such scales), else the multiply, with the same results
        float sc[NCH];
#pragma unroll
        for (int c = 0; c < NCH; ++c)
            sc[c] = *reinterpret_cast<const float*>(st + ST_SCALE + 4 * ((c * NTW + tid) >> 5));
        // pow2_scale of every one, as one test: no mantissa or sign bit in any, and the least
        // and largest bit patterns (exponents) in range
        uint32_t mant = 0, lo = ~0u, hi = 0;
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            const uint32_t b = __float_as_uint(sc[c]);
            mant |= b & 0x807FFFFFu;
            lo = min(lo, b);
            hi = max(hi, b);
        }
        const bool p2 = mant == 0 && lo >= (10u << 23) && hi <= (246u << 23);
        const bool fast = __builtin_amdgcn_ballot_w64(!p2) == 0;  // wave-uniform
        auto convert = [&](auto fast_tag) __attribute__((always_inline)) {
#pragma unroll
            for (int b0 = 0; b0 < NCH; b0 += BATCH) {
                uint4 raw[BATCH];
#pragma unroll
                for (int i = 0; i < BATCH; ++i) raw[i] = *reinterpret_cast<const uint4*>(st + 16 * ((b0 + i) * NTW + tid));
#pragma unroll
                for (int i = 0; i < BATCH; ++i) {
                    const int k = (b0 + i) * NTW + tid;
                    bf16x8 lo, hi;
                    if constexpr (decltype(fast_tag)::value)
                        dequant16_pow2(raw[i], sc[b0 + i], lo, hi);
                    else
                        dequant16(raw[i], sc[b0 + i], lo, hi);
                    char* const dst = kv0 + (k >> 5) * LAT_STRIDE + 32 * (k & 31);
                    *reinterpret_cast<bf16x8*>(dst) = lo;
                    *reinterpret_cast<bf16x8*>(dst + 16) = hi;
                }
            }
        };
        if (fast)
            convert(std::true_type{});
        else
            convert(std::false_type{});
#pragma unroll
        for (int j = 0; j < TK * DR * 2 / 16 / NTW; ++j) {
            const int k = j * NTW + tid;
            *reinterpret_cast<uint4*>(kv0 + ROPE_OFF + 16 * k) = *reinterpret_cast<const uint4*>(st + ST_ROPE + 16 * k);
        }
    };

    f32x16 acc_o[NBO];
    float m_ref = -INFINITY;   // reference max (log2 domain) of this lane's row
    float m_true = -INFINITY;  // exact max of the row's scores so far (log2 domain)
    float l_run = 0.0f;        // running sum over this lane's share of the keys
    bool over = false;         // a score of this row passed the reference's slack

    // Q K^T of the tile in kvt, with a later tile's NLOADS loads (issue_loads) one after every
    // GAP-th MFMA, so the vector memory pipe drains them under the matrix core.
    auto qk_tile = [&](const char* kvt, const LaneOffs& lo, auto issue_loads, auto nloads, auto gap)
        __attribute__((always_inline)) {
        constexpr int NLOADS = decltype(nloads)::value, GAP = decltype(gap)::value;
        bf16x8 qa[KB];
        auto rd = [&](int kb) __attribute__((always_inline)) {
            const char* ap = kb < KBL ? kvt + lo.lat + kb * 32 : kvt + lo.rope[kb - KBL];
            qa[kb] = *reinterpret_cast<const bf16x8*>(ap);
        };
        f32x16 s = f32x16{};
        __builtin_amdgcn_sched_barrier(0);
        issue_loads();
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
            if (k % GAP == 0 && k / GAP < NLOADS) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
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

    // One tile: scores, key mask (okb: its valid slots), softmax and P V on the tile in kvt, with
    // a later tile's loads (issue_loads) among its Q K^T MFMAs.
    auto compute_tile = [&](const char* kvt, uint64_t okb, auto issue_loads, auto nloads, auto gap)
        __attribute__((always_inline)) {
        const LaneOffs lo = lane_offs();
        f32x16 s = qk_tile(kvt, lo, issue_loads, nloads, gap);
        mask_keys(s, okb, 0, half);
        wide::Softmax sm;
        bf16x8 pn[2];
#pragma unroll
        for (int k = 0; k < wide::SOFTMAX_PIECES; ++k) sm.piece(k, s, m_ref, scale_log2, pn);
        m_ref = sm.mn;
        m_true = fmaxf(m_true, sm.mloc);
        over = over || sm.over;
        l_run += sm.l;
        pv_tile(kvt, lo, pn);
    };
    // A tile's loads: bf16 rows into a tile buffer, or fp8 rows, rope rows and scales into a slot.
    auto issue_bf16 = [&](char* dst, int rows, const uint32_t (&ro)[ROPE_PER_WAVE]) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < LAT_PER_WAVE; ++i) lat_load(dst, rows, i);
#pragma unroll
        for (int i = 0; i < ROPE_PER_WAVE; ++i) rope_load(dst + ROPE_OFF, ro[i], i);
    };
    auto issue_fp8 = [&](char* st, int rows, const uint32_t (&ro)[ROPE_PER_WAVE], uint32_t so)
        __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < LAT8_PER_WAVE; ++i) lat8_load(st, rows, i);
#pragma unroll
        for (int i = 0; i < ROPE_PER_WAVE; ++i) rope_load(st + ST_ROPE, ro[i], i);
        scale_load(st, so);
    };

    // Row pipeline across steps. D tiles separate the one computed and the one whose rows load
    // during it (bf16: the next; fp8: the one after, two tiles ahead, so that a tile's rows
    // load into one slot while the other slot still holds the next tile). Entering a step: tiles
    // tq[0..D+1] of the sequence; okb[0..D] their valid-slot bits; tq[D] past stage b (key_d,
    // blk_d); tq[D+1] past stage a (ia_n). A step runs stage c of tq[D] (its rows load during
    // this step), stage b of tq[D+1] and stage a of the tile after it.
    constexpr int D = FP8 ? 2 : 1;
    int tq[D + 2], key_d, blk_d, ia_n;
    uint64_t okb[D + 1];
    auto step = [&](auto top, const char* kvt, char* dst) __attribute__((always_inline)) {
        top();
        const int rows = stage_c(key_d, blk_d);
        uint32_t ro[ROPE_PER_WAVE];
        rope_src(rows, ro);
        const uint32_t so = FP8 ? scale_src(rows) : 0u;
        bool ok;
        const int key_n = stage_b(tq[D + 1], ia_n, ok);
        const uint64_t okb_n = __ballot(ok);
        const int blk_n = stage_b_load(key_n);
        const int t_n = next_tile(tq[D + 1]);
        const int ia_nn = stage_a(t_n);
        if constexpr (FP8)
            compute_tile(kvt, okb[0], [&]() __attribute__((always_inline)) { issue_fp8(dst, rows, ro, so); },
                         std::integral_constant<int, FP8_LOADS>{}, std::integral_constant<int, 3>{});
        else
            compute_tile(kvt, okb[0], [&]() __attribute__((always_inline)) { issue_bf16(dst, rows, ro); },
                         std::integral_constant<int, LAT_PER_WAVE + ROPE_PER_WAVE>{}, std::integral_constant<int, 2>{});
#pragma unroll
        for (int i = 0; i <= D; ++i) tq[i] = tq[i + 1];
        tq[D + 1] = t_n;
#pragma unroll
        for (int i = 0; i < D; ++i) okb[i] = okb[i + 1];
        okb[D] = okb_n;
        key_d = key_n;
        blk_d = blk_n;
        ia_n = ia_nn;
    };
    // Step tops. bf16: tile tq[0]'s rows and the pipeline's loads landed for both waves, and the
    // other buffer is free. fp8: every load issued so far landed for both waves, tq[0]'s (two
    // steps old) and the next tile's (one step old, in the other slot); tq[0]'s slot is
    // dequantised into the tile buffer, which the barrier after it completes and the slot
    // frees. Waiting only for all but the newest FP8_LOADS loads would cover tq[0] if loads
    // retired in issue order, but with such a wait alone reads of the slot saw rows that had
    // not landed; the full wait measured no slower, the newest loads having had a step.
    auto top_bf16 = [&]() __attribute__((always_inline)) {
        __builtin_amdgcn_s_waitcnt(0x0F70);
        __syncthreads();
    };
    auto top_fp8 = [&](const char* st) __attribute__((always_inline)) {
        asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
        dequant(st);
        lds_barrier();
    };

    // Pass 0 against first-tile references; pass 1 only if some row of the workgroup passed its
    // reference's slack, against every row's exact max.
    for (int pass = 0;; ++pass) {
#pragma unroll
        for (int d = 0; d < NBO; ++d) wide::o_zero(acc_o[d]);
        l_run = 0.0f;
        m_ref = pass == 0 ? -INFINITY : m_true;
        tq[0] = next_tile(-1);
#pragma unroll
        for (int i = 1; i <= D + 1; ++i) tq[i] = next_tile(tq[i - 1]);
        if (tq[0] < t_end) {  // workgroup-uniform; no key leaves O = 0, LSE = -inf
            // fill the pipeline: stages a, b of tq[0..D+1], then the loads of tq[0..D-1]
            int ia[D + 2], key[D + 1], blk[D + 1];
#pragma unroll
            for (int i = 0; i <= D + 1; ++i) ia[i] = stage_a(tq[i]);
            __builtin_amdgcn_s_waitcnt(0x0F70);
#pragma unroll
            for (int i = 0; i <= D; ++i) {
                bool ok;
                key[i] = stage_b(tq[i], ia[i], ok);
                okb[i] = __ballot(ok);
                blk[i] = stage_b_load(key[i]);
            }
            __builtin_amdgcn_s_waitcnt(0x0F70);
            key_d = key[D];
            blk_d = blk[D];
            ia_n = ia[D + 1];
#pragma unroll
            for (int i = 0; i < D; ++i) {
                const int rows = stage_c(key[i], blk[i]);
                uint32_t ro[ROPE_PER_WAVE];
                rope_src(rows, ro);
                if constexpr (FP8)
                    issue_fp8(i == 0 ? kv1 : kv2, rows, ro, scale_src(rows));
                else
                    issue_bf16(kv0, rows, ro);
            }
            // tile j of the sequence sits in buffer (bf16) or slot (fp8) j % 2; past the last
            // live tile the pipeline loads pad rows
            while (true) {
                if constexpr (FP8)
                    step([&]() __attribute__((always_inline)) { top_fp8(kv1); }, kv0, kv1);
                else
                    step(top_bf16, kv0, kv1);
                if (tq[0] >= t_end) break;
                if constexpr (FP8)
                    step([&]() __attribute__((always_inline)) { top_fp8(kv2); }, kv0, kv2);
                else
                    step(top_bf16, kv1, kv0);
                if (tq[0] >= t_end) break;
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
    auto o_row = [&](int r) __attribute__((always_inline)) {
        return r < 16 ? r_lo + r * (DL * 2) : o_hi + (r - 16) * (DL * 2);
    };
    char* const lrow = o_row(l32);
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
        uint4 v = *reinterpret_cast<const uint4*>(o_row(r) + 16 * (lane ^ (r >> 1)));
        if (r & 1) v = uint4{v.z, v.w, v.x, v.y};
        *reinterpret_cast<uint4*>(o_wave + r * DL) = v;
    }
    sched::mark_empty_slices(lse0, grow, valid && half == 0, wk.split, wk.nsplit, kv_splits, split_stride, H);
}

template <bool PAGED, bool FP8>
hipError_t launch_wide(const mla_partial_args& a, hipStream_t stream) {
    const int64_t grid = (int64_t)a.T_loc * ((a.H + BM - 1) / BM) * a.kv_splits;
    hipLaunchKernelGGL((sparse_wide_kernel<PAGED, FP8>), dim3((unsigned)grid), dim3(NTW), 0, stream,
                       (const __bf16*)a.q, (const char*)a.latent_kv, a.kv_scale, (const char*)a.rope_k,
                       a.cu_seqlens_q, a.vrow_kv_start, a.positions, a.topk_idx, a.topk, a.window, a.n_vrows, a.H,
                       a.N_kv, a.scale * kLog2e, (__bf16*)a.o_partial, a.lse, a.kv_splits, a.split_stride,
                       a.vrow_kv_len, a.block_table, a.bt_stride, a.vrow_req,
                       a.kv_splits > 1 ? a.vrow_splits : nullptr);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_sparse_wide_partial(const mla_partial_args& a, hipStream_t stream) {
    if (a.kv_dtype == MLA_KV_FP8_E4M3)
        return a.block_table ? launch_wide<true, true>(a, stream) : launch_wide<false, true>(a, stream);
    return a.block_table ? launch_wide<true, false>(a, stream) : launch_wide<false, false>(a, stream);
}

}  // namespace mla
