// Rank-local sparse MLA partial attention over bf16 latent rows: the same key sets as the
// fp8 kernel (sparse_keys.h), read from a bf16 latent array -- a bf16 cache, or the
// workspace that pcp_kv_dequant_fp8 fills from an fp8 cache once per step (the dequantised
// workspace of sparse BF16 CP prefill: "DeepSeek-V4.1: Prefill support CP with multistream
// forward prepare (4/N)", commit list, "Reuse shared compressed KV dequantization in V4.1 CP
// prefill"; the partial itself: "[DeepSeekV4][PCP] Enable context-parallel prefill for hybrid
// KV and MegaMoE", "Purpose").
//
// One workgroup per (token, 64 heads, key split), the dense kernel's wave pairs and per-tile
// compute (attn_core.h). A tile's 64 gathered keys stream HBM -> LDS with no staging: one
// wave-wide direct-to-LDS buffer load per latent row (the row offset, wave-uniform, in an
// SGPR) into one of two latent buffers, so the next tile's rows load during this tile's
// compute; the rope rows (7 per load, per-lane offsets) go to a single buffer once every wave
// has finished this tile's Q K^T reads.
#include "sparse_keys.h"

namespace mla {
namespace {

using namespace attn;

template <int DL, int DR, bool PAGED>
__global__ __launch_bounds__(NT, 1) void sparse_bf16_partial_kernel(
    const __bf16* __restrict__ q, const char* __restrict__ lat, const char* __restrict__ rope,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ vrow_kv_start, const int32_t* __restrict__ positions,
    const int32_t* __restrict__ topk_idx, int topk, int window, int n_vrows, int H, int64_t N_kv, float scale_log2,
    __bf16* __restrict__ o_out, float* __restrict__ lse_out, int kv_splits, int64_t split_stride,
    const int32_t* __restrict__ vrow_kv_len, const int32_t* __restrict__ block_table, int bt_stride,
    const int32_t* __restrict__ vrow_req,
    const int32_t* __restrict__ vrow_splits) {
    using S = Shape<DL, DR>;
    static_assert(DL * 2 == 1024, "one direct-to-LDS load per 1024-byte latent row");
    constexpr int LAT_PER_WAVE = BN / 4;  // latent row loads per wave and tile
    __shared__ __attribute__((aligned(1024))) char kv_lat0[S::ROPE_OFF];  // latent tile double buffer:
    __shared__ __attribute__((aligned(1024))) char kv_lat1[S::ROPE_OFF];  // two separate LDS objects
    __shared__ __attribute__((aligned(16))) char kv_rope[BN * S::ROPE_STRIDE];
    __shared__ int sel[MAX_TOPK];
    __shared__ int win_blk[MAX_WINDOW / BN + 1];
    __shared__ Exchange ex;
    static_assert(S::DQK == 8 * Q_CHUNKS && S::ROPE_OFF >= Q_REGION_BYTES, "Q rows of a wave pair fit a tile buffer");

    const SparseWork wk =
        sparse_work(H, kv_splits, cu, n_vrows, vrow_kv_start, positions, vrow_kv_len, vrow_splits);
    if (wk.split >= wk.nsplit) return;  // a range past the row's count: no keys, nothing to write
    const int tid = threadIdx.x;
    // wave-uniform; read into an SGPR for packed KV only (paged: measured 9 % slower that way)
    const int wave = PAGED ? tid >> 6 : __builtin_amdgcn_readfirstlane(tid >> 6);
    const int pair = wave >> 1;
    const int side = wave & 1;
    const int lane = tid & 63;
    const int half = lane >> 5;
    const int l32 = lane & 31;
    float* const lse0 = lse_out;
    if (kv_splits > 1) {
        o_out += wk.split * split_stride * H * DL;
        lse_out += wk.split * split_stride * H;
    }
    const int head = wk.hg * BM + pair * 32 + l32;
    const bool valid = head < H;  // rows past H (a last head group under 64) stay idle
    const int64_t grow = (int64_t)wk.tok * H + head;
    // Buffer views of the latent and rope rows from row_base (the request's first row when
    // packed, the cache's first row when paged); the caller keeps N_kv * DL * 2 below 2^32.
    const int64_t row_base = PAGED ? 0 : wk.kv0;
    const int last_row = (int)(N_kv - 1 - row_base);
    const __amdgpu_buffer_rsrc_t lat_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(lat + row_base * (DL * 2)), 0, (int)(uint32_t)((N_kv - row_base) * (DL * 2)), kBufferFlags);
    const __amdgpu_buffer_rsrc_t rope_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(rope + row_base * (DR * 2)), 0, (int)(uint32_t)((N_kv - row_base) * (DR * 2)), kBufferFlags);
    const int32_t* bt_row = PAGED ? block_table + (int64_t)vrow_req[wk.lo_v] * bt_stride : nullptr;
    // Q rows first, into the latent buffers (pair 0 into the first, pair 1 into the second):
    // their loads are in flight while the selected-row list is built
    char* const q_region = pair == 0 ? kv_lat0 : kv_lat1;
    dma_q_rows<2>(__builtin_amdgcn_make_buffer_rsrc((void*)(q + (int64_t)wk.tok * H * S::DQK), 0, H * S::DQK * 2,
                                                    kBufferFlags),
                  wk.hg * BM + pair * 32, H, q_region, side, lane);
    const SparseKeys<PAGED> ks = sparse_keys<PAGED>(sel, win_blk, topk_idx, topk, window, wk, bt_row, bt_stride);

    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's Q rows landed
    __syncthreads();                     // ... every wave's, and the selected-row list is written
    bf16x8 qf[S::KB];
    read_q_frags(q_region, lane, qf);

    const int n_tiles = ks.n_tiles;
    // Latent rows of tile t into buffer dst: wave w loads slots 16w .. 16w+15, one row each;
    // lane l of the wave looks up slot 16w + l%16 (lat_rows), load n takes its row by readlane.
    // Rows are clamped into the cache before any offset is formed (a paged block id outside it
    // reads a wrong row, never outside the cache): the latent row goes in the load's scalar
    // offset, which the buffer range check does not cover, and no load relies on that check.
    auto lat_rows = [&](int t) {
        bool ok;
        return max(min(ks.slot_key(t, LAT_PER_WAVE * wave + (lane & (LAT_PER_WAVE - 1)), ok), last_row), 0);
    };
    auto lat_load = [&](int row, char* dst, int n) {
        const uint32_t soff = (uint32_t)__builtin_amdgcn_readlane(row, n) * (DL * 2);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(lat_rsrc, (lds_void*)(dst + (LAT_PER_WAVE * wave + n) * S::LAT_STRIDE),
                                                 16, lane * 16, soff, 0, 0);
    };
    // Rope rows of tile t (7 rows of 144 bytes per load).
    auto load_rope = [&](int t) {
        constexpr int RV = S::ROPE_VECS + 1;
        const int rk = lane / RV;
        const int rc = lane - rk * RV;
        const bool ron = rc < S::ROPE_VECS && rk < S::ROPE_ROWS_PER_LOAD;
#pragma unroll
        for (int i = 0; i < (S::ROPE_LOADS + 3) / 4; ++i) {
            const int n = i * 4 + wave;
            if (n >= S::ROPE_LOADS) break;  // wave-uniform
            const int r = n * S::ROPE_ROWS_PER_LOAD + rk;
            bool ok;
            const int row = max(min(ks.slot_key(t, r < BN ? r : 0, ok), last_row), 0);
            if (ron && r < BN)
                lds_dma16(rope_rsrc, (uint32_t)row * (DR * 2) + rc * 16, kv_rope + n * S::ROPE_ROWS_PER_LOAD * S::ROPE_STRIDE);
        }
    };

    constexpr int NB0 = S::NB / 2;
    f32x16 acc_o[NB0];
#pragma unroll
    for (int d = 0; d < NB0; ++d) acc_o[d] = f32x16{};
    float m_ref = -INFINITY;
    float l_run = 0.0f;
    const LaneOffsets<S> lo(side, lane);

    int t = ks.next_live(0, lane);
    int tn = n_tiles;
    lds_barrier();  // every wave holds its Q fragments: the first tile may overwrite pair 0's rows
    if (t < n_tiles) {
        const int row = lat_rows(t);
#pragma unroll
        for (int n = 0; n < LAT_PER_WAVE; ++n) lat_load(row, kv_lat0, n);
        load_rope(t);
        tn = ks.next_live(t + 1, lane);
    }
    // One tile: everything in flight is this tile's, so wait for all of it; then the next
    // tile's latent rows stream into the other buffer during the compute (one load after every
    // second Q K^T MFMA; past the last tile they load pad rows into the unused buffer), and its
    // rope rows once every wave is past this tile's Q K^T.
    auto step = [&](const char* cur, char* nxt) {
        bool ok;
        ks.slot_key(t, lane, ok);
        const uint64_t bits = __ballot(ok);  // valid slots of tile t (every wave the same)
        const int nrow = lat_rows(tn);
#pragma unroll
        for (int kb = 0; kb < S::KB; ++kb) asm volatile("" : "+a"(qf[kb]));  // Q stays in AGPRs
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): tile t landed for this wave
        __syncthreads();                     // ... for every wave; buffer nxt is free
        const int tnn = tn < n_tiles ? ks.next_live(tn + 1, lane) : n_tiles;
        auto keymask = [&](f32x16& s) { mask_keys(s, bits, side, half); };
        auto rope_next = [&] {
            if (tn < n_tiles) load_rope(tn);
        };
        tile_compute<S, DL, LAT_PER_WAVE>(cur, kv_rope, qf, acc_o, m_ref, l_run, scale_log2, wave, side, lane, lo, ex,
                                          keymask, rope_next, [&](int n) { lat_load(nrow, nxt, n); });
        t = tn;
        tn = tnn;
    };
    while (t < n_tiles) {
        step(kv_lat0, kv_lat1);
        if (t >= n_tiles) break;
        step(kv_lat1, kv_lat0);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // the pad rows past the last tile landed before LDS is reused
    write_rows_staged<S, DL>(acc_o, m_ref, l_run, valid, grow, wave, side, lane, ex, kv_lat0, o_out, lse_out);
    sched::mark_empty_slices(lse0, grow, valid && side == 0 && half == 0, wk.split, wk.nsplit, kv_splits,
                             split_stride, H);
}

template <bool PAGED>
hipError_t launch_sparse_bf16(const mla_partial_args& a, hipStream_t stream) {
    const int64_t grid = (int64_t)a.T_loc * ((a.H + BM - 1) / BM) * a.kv_splits;
    hipLaunchKernelGGL((sparse_bf16_partial_kernel<512, 64, PAGED>), dim3((unsigned)grid), dim3(NT), 0, stream,
                       (const __bf16*)a.q, (const char*)a.latent_kv, (const char*)a.rope_k, a.cu_seqlens_q,
                       a.vrow_kv_start, a.positions, a.topk_idx, a.topk, a.window, a.n_vrows, a.H, a.N_kv,
                       a.scale * kLog2e, (__bf16*)a.o_partial, a.lse, a.kv_splits, a.split_stride, a.vrow_kv_len,
                       a.block_table, a.bt_stride, a.vrow_req,
                       a.kv_splits > 1 ? a.vrow_splits : nullptr);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_sparse_bf16_partial(const mla_partial_args& a, hipStream_t stream) {
    return a.block_table ? launch_sparse_bf16<true>(a, stream) : launch_sparse_bf16<false>(a, stream);
}

}  // namespace mla
