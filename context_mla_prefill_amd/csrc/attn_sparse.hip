// Rank-local sparse MLA partial attention: top-k selected keys plus a sliding window,
// latent KV stored as fp8-e4m3 with one fp32 scale per 64 packed KV rows.
//
// Each PCP rank computes a local partial attention whose LSE/output are merged later with
// the sink applied once ("[DeepSeekV4][PCP] Enable context-parallel prefill for hybrid
// KV and MegaMoE", "Purpose": PCP merge for sparse prefill attention); the fp8 MLA cache
// with block size 64 is the one named in "[Feature][PCP] Add DeepSeek-V4.1-Flash
// support", "vLLM Launch Arguments" (the layout is this library's: E4M3FN codes, one
// fp32 scale per 64 packed rows, rope kept bf16).
//
// The key set (selected indices plus window, counted once) and its tiles are described in
// sparse_keys.h.
//
// Work decomposition: one workgroup per (token, 64 heads), i.e. the same 64 rows and wave
// pairs as the dense kernel, running the same per-tile compute. A tile is 64 key slots:
// first the selected-index slots in 64-wide groups (a group with no valid key is skipped),
// then the window. Per tile:
//   * the fp8 rows of a tile's keys and their 64-row scales are gathered HBM -> LDS staging
//     by direct-to-LDS loads two tiles ahead (two staging slots), so a gather has the
//     compute of a whole tile to land;
//   * the workgroup dequantises the staged rows once into the padded bf16 tile,
//     bf16_rne(fp32(e4m3) * scale[row/64]);
//   * rope rows stream straight into the tile once every wave is done with the previous
//     tile's Q K^T reads.
#include "sparse_keys.h"

namespace mla {
namespace {

using namespace attn;

constexpr int GATHER_LOADS = BN / 2 / 4 + 1;  // per wave and tile: latent loads (2 keys each) + 1 scale load

typedef float f32x2 __attribute__((ext_vector_type(2)));

// bf16_rne(fp32(e4m3) * sc) of the 4 E4M3FN codes of w (OCP decode on gfx950).
__device__ __forceinline__ void dequant4(uint32_t w, float sc, __bf16* out) {
    const f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
    const f32x2 b = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
    out[0] = (__bf16)(a.x * sc);
    out[1] = (__bf16)(a.y * sc);
    out[2] = (__bf16)(b.x * sc);
    out[3] = (__bf16)(b.y * sc);
}

template <int DL, int DR, bool PAGED>
__global__ __launch_bounds__(NT, 1) void sparse_partial_kernel(
    const __bf16* __restrict__ q, const uint8_t* __restrict__ lat8, const float* __restrict__ kv_scale,
    const char* __restrict__ rope, const int32_t* __restrict__ cu, const int32_t* __restrict__ vrow_kv_start,
    const int32_t* __restrict__ positions, const int32_t* __restrict__ topk_idx, int topk, int window,
    int n_vrows, int H, int64_t N_kv, float scale_log2, __bf16* __restrict__ o_out, float* __restrict__ lse_out,
    int kv_splits, int64_t split_stride, const int32_t* __restrict__ vrow_kv_len,
    const int32_t* __restrict__ block_table, int bt_stride, const int32_t* __restrict__ vrow_req,
    const int32_t* __restrict__ vrow_splits) {
    using S = Shape<DL, DR>;
    static_assert(DL == 512, "the fp8 staging assumes 512-byte latent rows");
    __shared__ __attribute__((aligned(1024))) char kv_lat[S::ROPE_OFF];        // bf16 latent rows of the current tile
    __shared__ __attribute__((aligned(16))) char kv_rope[BN * S::ROPE_STRIDE];  // and their rope rows
    __shared__ __attribute__((aligned(1024))) uint8_t stage[2][BN * DL];    // fp8 rows of the next two tiles
    __shared__ float stage_scale[2][BN];
    __shared__ int sel[MAX_TOPK];            // KV row of each selected key of the set, -1 otherwise
    __shared__ int win_blk[MAX_WINDOW / BN + 1];  // paged: cache blocks the window spans
    __shared__ uint64_t tmask[2];            // valid-key bits per staging slot
    __shared__ Exchange ex;
    static_assert(S::DQK == 8 * Q_CHUNKS && S::ROPE_OFF >= Q_REGION_BYTES && sizeof(stage) >= Q_REGION_BYTES,
                  "Q rows of a wave pair fit a tile buffer");

    const SparseWork wk =
        sparse_work(H, kv_splits, cu, n_vrows, vrow_kv_start, positions, vrow_kv_len, vrow_splits);
    if (wk.split >= wk.nsplit) return;  // a range past the row's count: no keys, nothing to write
    const int tok = wk.tok;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: keep it in SGPRs
    const int pair = wave >> 1;
    const int side = wave & 1;
    const int lane = tid & 63;
    const int half = lane >> 5;
    const int l32 = lane & 31;

    const int64_t kv0 = wk.kv0;
    float* const lse0 = lse_out;
    if (kv_splits > 1) {
        o_out += wk.split * split_stride * H * DL;
        lse_out += wk.split * split_stride * H;
    }
    const int head = wk.hg * BM + pair * 32 + l32;
    const bool valid = head < H;  // rows past H (a last head group under 64) stay idle
    const int64_t grow = (int64_t)tok * H + head;
    // Keys are addressed by row relative to row_base: the request's first row for packed KV
    // (row = key position), 0 for paged KV (row = block_table entry * 64 + position % 64).
    // Buffer views: fp8 latent rows of DL bytes, bf16 rope rows, and the 64-row scales of
    // the whole cache. The caller keeps N_kv * DL below 2^32.
    const int64_t row_base = PAGED ? 0 : kv0;
    const int last_row = (int)(N_kv - 1 - row_base);
    const __amdgpu_buffer_rsrc_t lat_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(lat8 + row_base * DL), 0, (int)(uint32_t)((N_kv - row_base) * DL), kBufferFlags);
    const __amdgpu_buffer_rsrc_t rope_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(rope + row_base * (DR * 2)), 0, (int)(uint32_t)((N_kv - row_base) * (DR * 2)), kBufferFlags);
    const __amdgpu_buffer_rsrc_t scale_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void*)kv_scale, 0, (int)(uint32_t)(((N_kv + 63) / 64) * 4), kBufferFlags);
    const int32_t* bt_row = PAGED ? block_table + (int64_t)vrow_req[wk.lo_v] * bt_stride : nullptr;
    // Q rows first, through LDS (pair 0 into the bf16 tile, pair 1 into the staging slots):
    // their loads are in flight while the selected-row list is built
    char* const q_region = pair == 0 ? kv_lat : (char*)stage;
    dma_q_rows<2>(__builtin_amdgcn_make_buffer_rsrc((void*)(q + (int64_t)tok * H * S::DQK), 0, H * S::DQK * 2,
                                                    kBufferFlags),
                  wk.hg * BM + pair * 32, H, q_region, side, lane);
    const SparseKeys<PAGED> ks = sparse_keys<PAGED>(sel, win_blk, topk_idx, topk, window, wk, bt_row, bt_stride);

    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's Q rows landed
    __syncthreads();                     // ... every wave's, and the selected-row list is written
    bf16x8 qf[S::KB];
    read_q_frags(q_region, lane, qf);

    const int n_tiles = ks.n_tiles;
    auto slot_key = [&](int t, int j, bool& ok) -> int { return ks.slot_key(t, j, ok); };
    auto next_live = [&](int t) -> int { return ks.next_live(t, lane); };
    // Gathers tile t into staging slot b: fp8 latent rows (wave-wide load n moves keys 2n and
    // 2n+1, 32 lanes x 16 bytes each), the 64-row scale of each key (wave w: keys 16w..16w+15)
    // and the valid-key bits. Every wave issues exactly GATHER_LOADS loads.
    auto gather_latent = [&](int t, int b) {
#pragma unroll
        for (int i = 0; i < BN / 2 / 4; ++i) {
            const int n = i * 4 + wave;
            bool ok;
            const int key = max(min(slot_key(t, 2 * n + half, ok), last_row), 0);
            lds_dma16(lat_rsrc, (uint32_t)key * DL + l32 * 16, (char*)stage[b] + n * 1024);
        }
        {
            bool ok;
            const int key = max(min(slot_key(t, 16 * wave + (lane & 15), ok), last_row), 0);
            if (lane < 16)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(scale_rsrc, (lds_void*)&stage_scale[b][16 * wave], 4,
                                                         (uint32_t)((row_base + key) >> 6) * 4, 0, 0, 0);
        }
        if (wave == 0) {
            bool ok;
            slot_key(t, lane, ok);
            const uint64_t bits = __ballot(ok);
            if (lane == 0) tmask[b] = bits;
        }
    };
    // Rope rows of tile t straight into the bf16 tile (7 rows of 144 bytes per load).
    auto gather_rope = [&](int t) {
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
            const int key = max(min(slot_key(t, r < BN ? r : 0, ok), last_row), 0);
            if (ron && r < BN)
                lds_dma16(rope_rsrc, (uint32_t)key * (DR * 2) + rc * 16, kv_rope + n * S::ROPE_ROWS_PER_LOAD * S::ROPE_STRIDE);
        }
    };
    // Dequantises staging slot b into the bf16 tile: thread handles 16-byte chunks tid,
    // tid+256, ... (consecutive lanes read consecutive LDS bytes). All of a thread's staged
    // chunks and scales are read before any is converted, so their LDS latencies overlap.
    auto convert = [&](int b) {
        constexpr int NCH = BN * DL / 16 / NT;
        uint4 raw[NCH];
        float sc[NCH];
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
            const int k = i * NT + tid;
            raw[i] = *reinterpret_cast<const uint4*>(stage[b] + k * 16);
            sc[i] = stage_scale[b][k / (DL / 16)];
        }
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
            const int k = i * NT + tid;
            const int r = k / (DL / 16);
            const int c = k - r * (DL / 16);
            bf16x8 o0, o1;
            __bf16 v[16];
            dequant4(raw[i].x, sc[i], v);
            dequant4(raw[i].y, sc[i], v + 4);
            dequant4(raw[i].z, sc[i], v + 8);
            dequant4(raw[i].w, sc[i], v + 12);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                o0[e] = v[e];
                o1[e] = v[8 + e];
            }
            char* dst = kv_lat + r * S::LAT_STRIDE + c * 32;
            *reinterpret_cast<bf16x8*>(dst) = o0;
            *reinterpret_cast<bf16x8*>(dst + 16) = o1;
        }
    };

    constexpr int NB0 = S::NB / 2;
    f32x16 acc_o[NB0];
#pragma unroll
    for (int d = 0; d < NB0; ++d) acc_o[d] = f32x16{};
    float m_ref = -INFINITY;
    float l_run = 0.0f;
    const LaneOffsets<S> lo(side, lane);

    // Issue order keeps "all but the newest GATHER_LOADS loads" equal to "everything the
    // current tile needs": latent(t), rope(t), latent(next).
    int t = next_live(0);
    int tn = n_tiles;
    int b = 0;
    lds_barrier();  // every wave holds its Q fragments: the gathers may overwrite pair 1's rows
    if (t < n_tiles) {
        tn = next_live(t + 1);
        gather_latent(t, 0);
        gather_rope(t);
        gather_latent(tn, 1);  // tn may be past the last tile: loads of pad_row, never used
    }
    while (t < n_tiles) {
#pragma unroll
        for (int kb = 0; kb < S::KB; ++kb) asm volatile("" : "+a"(qf[kb]));  // Q stays in AGPRs
        __builtin_amdgcn_s_waitcnt(0x0F70 | GATHER_LOADS);  // vmcnt(GATHER_LOADS): tile t landed
        __syncthreads();                                     // ... for every wave
        convert(b);
        const uint64_t bits = tmask[b];
        __syncthreads();  // bf16 tile complete; staging slot b free
        const int tnn = tn < n_tiles ? next_live(tn + 1) : n_tiles;
        auto keymask = [&](f32x16& s) { mask_keys(s, bits, side, half); };
        auto prefetch = [&] {  // after every wave's Q K^T reads of tile t
            if (tn < n_tiles) gather_rope(tn);
            gather_latent(tnn, b);
        };
        tile_compute<S, DL>(kv_lat, kv_rope, qf, acc_o, m_ref, l_run, scale_log2, wave, side, lane, lo, ex, keymask,
                            prefetch);
        t = tn;
        tn = tnn;
        b ^= 1;
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // the unused last gather landed before LDS is released
    write_rows_staged<S, DL>(acc_o, m_ref, l_run, valid, grow, wave, side, lane, ex, kv_lat, o_out, lse_out);
    sched::mark_empty_slices(lse0, grow, valid && side == 0 && half == 0, wk.split, wk.nsplit, kv_splits,
                             split_stride, H);
}

template <bool PAGED>
hipError_t launch_sparse(const mla_partial_args& a, hipStream_t stream) {
    const int64_t grid = (int64_t)a.T_loc * ((a.H + BM - 1) / BM) * a.kv_splits;
    hipLaunchKernelGGL((sparse_partial_kernel<512, 64, PAGED>), dim3((unsigned)grid), dim3(NT), 0, stream,
                       (const __bf16*)a.q, (const uint8_t*)a.latent_kv, a.kv_scale, (const char*)a.rope_k,
                       a.cu_seqlens_q, a.vrow_kv_start, a.positions, a.topk_idx, a.topk, a.window, a.n_vrows, a.H,
                       a.N_kv, a.scale * kLog2e, (__bf16*)a.o_partial, a.lse, a.kv_splits, a.split_stride,
                       a.vrow_kv_len, a.block_table, a.bt_stride, a.vrow_req,
                       a.kv_splits > 1 ? a.vrow_splits : nullptr);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_sparse_partial(const mla_partial_args& a, hipStream_t stream) {
    return a.block_table ? launch_sparse<true>(a, stream) : launch_sparse<false>(a, stream);
}

}  // namespace mla
