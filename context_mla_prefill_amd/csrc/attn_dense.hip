// Rank-local causal MLA partial attention (dense), bf16 MFMA on gfx950, for the small
// 64 + 16 shape (latent 64, rope 16). The 512 + 64 shape runs the 128-row kernel of
// attn_dense_wide.hip.
//
// Absorbed MLA is multi-query attention with one latent KV head: key = latent || rope,
// value = latent. Every rank attends its local rows against the full all-gathered
// latent KV ("[Core] Add MRV2 virtual-batch PCP for MLA", "DualChunkSwap
// partitioning") and returns the normalised partial output and its natural-log LSE
// without the sink, which the merge applies once ("[DeepSeekV4][PCP] Enable
// context-parallel prefill for hybrid KV and MegaMoE", "Purpose").
//
// Work decomposition
//  * A workgroup (4 waves) owns BM = 64 rows of one virtual row, where a row is a
//    (token, head) pair: all heads share the KV, so token x head is the M dimension.
//    The waves form two pairs; a pair owns 32 rows and both of its waves keep the full
//    Q of those rows in registers for the whole KV loop.
//  * KV tiles of BN = 64 keys move HBM -> LDS with direct-to-LDS loads into a double
//    buffer (the next tile streams in while the current one is used) and are shared by
//    all heads and waves.
//  * Scores are computed transposed, S^T = K Q^T (v_mfma_f32_32x32x16_bf16, A = K from
//    LDS, B = Q^T from registers); wave s of a pair scores keys [32 s, 32 s + 32) of the
//    tile. Each lane then holds scores of ONE query row, so the row max needs one
//    cross-half exchange and the running sum stays per lane until the epilogue.
//  * The output is accumulated transposed, O^T += V^T P^T; wave s of a pair owns output
//    columns [DL/2 s, DL/2 s + DL/2) and needs P for all 64 keys, so the two waves swap
//    their bf16 P fragments through LDS. The P fragment is the score accumulator
//    re-packed in place; V^T comes from transposing LDS reads (ds_read_b64_tr_b16) in
//    the key order the score layout gives each lane.
//  * Online softmax with a lazy reference max: the reference of a row moves only when a
//    tile max exceeds it by more than kRescale (log2 units). Tiles that move no
//    reference (nearly all of them) need no max exchange and no O rescale; a tile that
//    does takes a workgroup-uniform slow path with one extra barrier.
//  * Work order (work_order.h): virtual rows in the caller's order, else last row first;
//    inside a row its tiles from the last to the first, so the long late-chunk tiles start
//    first and the short ones fill the tail.
#include "attn_core.h"
#include "work_order.h"

namespace mla {
namespace {

using namespace attn;

// LDS image of one KV tile of the dense kernel: latent rows at a stride of DL*2 + 16
// bytes (inside every block of 16 keys, key (score row) r sits in LDS row kperm(r):
// conflict-free Q K^T and V^T reads), rope rows after them at a stride of DR*2 + 16;
// several rows per direct-to-LDS load, loads predicated per lane.
template <int DL, int DR>
struct DenseTile {
    static constexpr int DQK = DL + DR;
    static constexpr int KB = DQK / 16;  // 16-wide k-blocks of Q K^T
    static constexpr int NB = DL / 32;   // 32-wide column blocks of O
    static constexpr int LAT_VECS = DL / 8;
    static constexpr int ROPE_VECS = DR / 8;
    static constexpr int LAT_STRIDE = DL * 2 + 16;
    static constexpr int ROPE_STRIDE = DR * 2 + 16;
    static constexpr int ROPE_OFF = BN * LAT_STRIDE;
    static constexpr int TILE_BYTES = ROPE_OFF + BN * ROPE_STRIDE;
    static constexpr int LAT_ROWS_PER_LOAD = 64 / (LAT_VECS + 1);
    static constexpr int ROPE_ROWS_PER_LOAD = 64 / (ROPE_VECS + 1);
    static constexpr int LAT_LOADS = (BN + LAT_ROWS_PER_LOAD - 1) / LAT_ROWS_PER_LOAD;
    static constexpr int ROPE_LOADS = (BN + ROPE_ROWS_PER_LOAD - 1) / ROPE_ROWS_PER_LOAD;
    static_assert(DQK % 16 == 0 && DL % 32 == 0 && DR % 8 == 0, "tile shape");
    static_assert(LAT_ROWS_PER_LOAD >= 1 && DL * 2 < 1024, "several latent rows per load (the small shape)");
};

// Where the keys of one tile live: KV row of its first key and how many keys it has.
struct TileRows {
    int64_t row0;
    int rows;  // 1..BN
};

// Every load of a tile, lanes that would land on a pad switched off. Keys past the tile's
// extent repeat its last key. Wave w issues loads w, w+4, ...
template <class T, int DL, int DR>
__device__ __forceinline__ void narrow_load_tile(char* dst, const char* __restrict__ lat,
                                                 const char* __restrict__ rope, TileRows tr, int wave, int lane) {
    constexpr int LV = T::LAT_VECS + 1, RV = T::ROPE_VECS + 1;
    const int lk = lane / LV;
    const int lc = lane - lk * LV;
    const bool lon = lc < T::LAT_VECS && lk < T::LAT_ROWS_PER_LOAD;
    const int rk = lane / RV;
    const int rc = lane - rk * RV;
    const bool ron = rc < T::ROPE_VECS && rk < T::ROPE_ROWS_PER_LOAD;
#pragma unroll
    for (int i = 0; i < (T::LAT_LOADS + 3) / 4; ++i) {
        const int n = i * 4 + wave;
        if (n >= T::LAT_LOADS) break;
        const int r = n * T::LAT_ROWS_PER_LOAD + lk;
        const int64_t j = tr.row0 + min(r, tr.rows - 1);
        if (lon && r < BN)
            lds_dma16(lat + j * (DL * 2) + lc * 16, dst + n * T::LAT_ROWS_PER_LOAD * T::LAT_STRIDE);
    }
#pragma unroll
    for (int i = 0; i < (T::ROPE_LOADS + 3) / 4; ++i) {
        const int n = i * 4 + ((wave + 2) & 3);
        if (n >= T::ROPE_LOADS) break;
        const int r = n * T::ROPE_ROWS_PER_LOAD + rk;
        const int64_t j = tr.row0 + min(r, tr.rows - 1);
        if (ron && r < BN)
            lds_dma16(rope + j * (DR * 2) + rc * 16,
                      dst + T::ROPE_OFF + n * T::ROPE_ROWS_PER_LOAD * T::ROPE_STRIDE);
    }
}

template <int DL, int DR, bool PAGED>
__global__ __launch_bounds__(NT, 1) void dense_partial_kernel(
    const __bf16* __restrict__ q, const char* __restrict__ lat, const char* __restrict__ rope,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ vrow_kv_start,
    const int32_t* __restrict__ positions, int n_vrows, int H, int64_t N_kv, float scale_log2,
    __bf16* __restrict__ o_out, float* __restrict__ lse_out, int kv_splits, int64_t split_stride,
    const int32_t* __restrict__ vrow_kv_len, const int32_t* __restrict__ block_table, int bt_stride,
    const int32_t* __restrict__ vrow_req, const int32_t* __restrict__ vrow_splits,
    const int32_t* __restrict__ vrow_order) {
    using T = DenseTile<DL, DR>;
    __shared__ __attribute__((aligned(1024))) char kv_lds0[T::TILE_BYTES];  // KV tile double buffer:
    __shared__ __attribute__((aligned(1024))) char kv_lds1[T::TILE_BYTES];  // two separate objects
    __shared__ __attribute__((aligned(16))) uint4 Px[NT / 64][2][64];  // P fragment exchange
    __shared__ float mx[NT / 64][64];                                  // tile maxima / row sums
    __shared__ int flag[NT / 64];
    __shared__ int s_maxpos[NT / 64];
    int* sh = reinterpret_cast<int*>(&Px[0][0][0]);  // scan scratch, used before the KV loop only

    // workgroup = (virtual row, row tile, key range)
    const sched::DenseWork wk =
        sched::find_work<BM, NT>((int)blockIdx.x, cu, n_vrows, H, vrow_splits, vrow_order, kv_splits, sh);
    const int v = wk.v, tile = wk.tile, split = wk.split;
    if (v < 0) return;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int pair = wave >> 1;
    const int side = wave & 1;    // keys [32 side, +32) of each tile; O columns [DL/2 side, +DL/2)
    const int lane = tid & 63;
    const int half = lane >> 5;   // which 8-element half of a 16-wide k-block this lane holds
    const int l32 = lane & 31;

    const int tok0 = cu[v];
    const int nrows = (cu[v + 1] - tok0) * H;
    const int rloc = tile * BM + pair * 32 + l32;  // row inside the virtual row
    const bool valid = rloc < nrows;
    const int64_t grow = (int64_t)tok0 * H + rloc;  // global row (token-major, then head)
    const int pos = valid ? positions[tok0 + rloc / H] : -1;
    const int64_t kv0 = __builtin_amdgcn_readfirstlane(vrow_kv_start[v]);

    // KV extent of the tile: largest position among its rows, plus one.
    int mp = pos;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) mp = max(mp, __shfl_xor(mp, off));
    if (lane == 0) s_maxpos[wave] = mp;

    // Q^T fragments: lane holds row l32, elements [16 kb + 8 half, +8) of every k-block.
    bf16x8 qf[T::KB];
    {
        const __bf16* qrow = q + grow * T::DQK + 8 * half;
#pragma unroll
        for (int kb = 0; kb < T::KB; ++kb)
            qf[kb] = valid ? *reinterpret_cast<const bf16x8*>(qrow + kb * 16) : bf16x8{};
    }
    __syncthreads();
    int kv_hi = s_maxpos[0];
#pragma unroll
    for (int w = 1; w < NT / 64; ++w) kv_hi = max(kv_hi, s_maxpos[w]);
    kv_hi = kv_hi + 1;
    // Key range of this split: whole 64-key tiles [key_lo, key_hi) of the request's KV.
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
    const int kt0 = __builtin_amdgcn_readfirstlane(key_lo / BN);
    // smallest position among this wave's rows: key blocks at or below it need no mask
    int pmin = valid ? pos : INT32_MAX;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) pmin = min(pmin, __shfl_xor(pmin, off));
    pmin = __builtin_amdgcn_readfirstlane(pmin);
    // last key (request-relative) a load may touch
    const int64_t last = PAGED ? (int64_t)kv_hi - 1 : min((int64_t)kv_hi - 1, N_kv - 1 - kv0);
    // Paged KV: block ids of 64 consecutive tiles [bw_base, bw_base + 64), one per lane,
    // read by v_readlane; the next 64 are fetched one tile before they are needed.
    const int32_t* bt_row = PAGED ? block_table + (int64_t)vrow_req[v] * bt_stride : nullptr;
    const int nblk = (int)(last >> 6) + 1;
    // Block ids outside the cache are clamped into it as the window loads (the keys they map read
    // wrong rows of the cache, never memory outside it); the cache holds whole blocks, so every tile -- one block, or the last key
    // alone -- stays inside it.
    const int blk_max = (int)(N_kv >> 6) - 1;
    int bw_base = 0, bw_v = 0;
    auto bw_load = [&](int base) {
        bw_base = base;
        bw_v = min(max(bt_row[min(base + lane, min(nblk, bt_stride) - 1)], 0), blk_max);
    };
    // KV rows of tile kt (request-relative keys clamped to `last`).
    auto tile_rows = [&](int kt) -> TileRows {
        const int64_t tb = min((int64_t)kt * BN, last);
        TileRows tr;
        tr.rows = (int)min((int64_t)BN, last - tb + 1);
        if constexpr (PAGED) {
            const int t = (int)(tb >> 6);
            tr.row0 = (int64_t)__builtin_amdgcn_readlane(bw_v, t - bw_base) * 64 + (tb & 63);
            if (t == bw_base + 63) bw_load(bw_base + 64);
        } else {
            tr.row0 = kv0 + tb;
        }
        return tr;
    };

    constexpr int NB0 = T::NB / 2;  // O column blocks per wave
    f32x16 acc_o[NB0];
#pragma unroll
    for (int d = 0; d < NB0; ++d) acc_o[d] = f32x16{};
    float m_ref = -INFINITY;  // lazy reference max (log2 domain) of this lane's row
    float l_run = 0.0f;       // running sum over this lane's share of the keys

    // Per-lane LDS offsets inside a tile (everything else is an immediate):
    //  * Q K^T reads: LDS row of score row l32, 8 elements at 8*half of each k-block;
    //  * V^T reads: LDS row of score row 4*half + (lane%16)/4 of a 16-key block, dims
    //    16*((lane/16)%2) + 4*(lane%4); the second read of an MFMA is 2 rows further.
    const int krow = 32 * side + 16 * (l32 >> 4) + kperm(l32 & 15);
    const int k_lat_off = krow * T::LAT_STRIDE + 16 * half;
    int k_rope_off[T::KB - DL / 16];
#pragma unroll
    for (int kb = 0; kb < T::KB - DL / 16; ++kb)
        k_rope_off[kb] = T::ROPE_OFF + krow * T::ROPE_STRIDE + 16 * half + 32 * kb;
    const int v_off = kperm(4 * half + ((lane & 15) >> 2)) * T::LAT_STRIDE + 2 * (16 * ((lane >> 4) & 1) + 4 * (lane & 3));

    const int n_tiles = (kv_hi + BN - 1) / BN;

    // One KV tile: wait for it, publish it, then scores, softmax, P exchange and P V on
    // it while the next tile streams into the other buffer. The two buffers are distinct
    // LDS objects, so the compiler can tell that the streaming loads never touch the tile
    // being read and does not wait for them.
    auto tile_step = [&](const char* kvt, char* nxt, int kt) {
#pragma unroll
        for (int kb = 0; kb < T::KB; ++kb) asm volatile("" : "+a"(qf[kb]));  // Q stays in AGPRs
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's loads of tile kt landed
        __syncthreads();                     // ... and every wave's; the other buffer is free
        if (kt + 1 < n_tiles) narrow_load_tile<T, DL, DR>(nxt, lat, rope, tile_rows(kt + 1), wave, lane);
        // S^T[key, row] for keys 32*side + 8*(i/4) + 4*half + i%4 of this tile, row l32.
        f32x16 s = f32x16{};
        {
            const char* kl = kvt + k_lat_off;
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int kb = 0; kb < T::KB; ++kb) {
                const char* ap = kb < DL / 16 ? kl + kb * 32 : kvt + k_rope_off[kb - DL / 16];
                const bf16x8 a = *reinterpret_cast<const bf16x8*>(ap);
                s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kb], s, 0, 0, 0);
            }
            // QK_AHEAD operand reads in flight ahead of the MFMA chain.
            constexpr int AHEAD = T::KB < QK_AHEAD ? T::KB : QK_AHEAD;
            __builtin_amdgcn_sched_group_barrier(0x100, AHEAD, 0);
#pragma unroll
            for (int kb = 0; kb < T::KB - AHEAD; ++kb) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, AHEAD, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
        // V^T operands of the first P V MFMAs (key-block-major: kb = m / NB0, d = m % NB0):
        // they do not depend on P, so their LDS reads run under the softmax.
        constexpr int NM = NB0 * 4;
        constexpr int PA = NM < PV_AHEAD ? NM : PV_AHEAD;
        constexpr int NVB = PA + 1;
        // Byte offsets from the tile base; every read is addressed by one offset from kvt (a
        // chain of pointer steps hides from alias analysis that the reads stay inside this
        // tile, and the compiler then waits for the next tile's loads in the middle of P V).
        const int v_own = v_off + (32 * side) * T::LAT_STRIDE;
        const int v_oth = v_off + (32 * (side ^ 1)) * T::LAT_STRIDE;
        s16x4 vlo[NVB], vhi[NVB];
        auto vread = [&](int m) {
            const int kb = m / NB0, d = m % NB0;
            const int o0 = (kb < 2 ? v_own : v_oth) + (16 * (kb & 1)) * T::LAT_STRIDE + (side * NB0 + d) * 64;
            vlo[m % NVB] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(kvt + o0));
            vhi[m % NVB] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(kvt + (o0 + 2 * T::LAT_STRIDE)));
        };
#pragma unroll
        for (int m = 0; m < PA; ++m) vread(m);
        if (kt * BN + 32 * side + 31 > pmin) {  // wave-uniform: a causal diagonal crosses these keys
            const int rel = pos - kt * BN;      // keys of this tile up to rel are visible
#pragma unroll
            for (int i = 0; i < 16; ++i) s[i] = score_key(side, half, i) <= rel ? s[i] : -INFINITY;
        }
        float smax = s[0];
#pragma unroll
        for (int i = 1; i < 16; ++i) smax = fmaxf(smax, s[i]);
        smax = fmaxf(smax, half_swap(smax));
        const float mloc = smax * scale_log2;  // max over this wave's 32 keys (log2 units)
        // Fast path: P against the current reference, published with a "needs a new
        // reference" flag; the slow path (any wave flagged) agrees on the pair max first.
        const bool need = mloc > m_ref + kRescale;
        float m_use = m_ref == -INFINITY ? 0.0f : m_ref;
        float pf[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) pf[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], scale_log2, -m_use));
        bf16x8 pk[2];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            pk[0][j] = (__bf16)pf[j];
            pk[1][j] = (__bf16)pf[8 + j];
        }
        Px[wave][0][lane] = __builtin_bit_cast(uint4, pk[0]);
        Px[wave][1][lane] = __builtin_bit_cast(uint4, pk[1]);
        mx[wave][lane] = mloc;
        const bool any_need = __ballot(need) != 0;
        if (lane == 0) flag[wave] = any_need;
        lds_barrier();
        int slow = 0;
#pragma unroll
        for (int w = 0; w < NT / 64; ++w) slow |= flag[w];
        if (slow) {  // workgroup-uniform
            const float m_pair = fmaxf(mloc, mx[wave ^ 1][lane]);
            const bool bump = m_pair > m_ref + kRescale;
            const float m_new = bump ? m_pair : m_ref;
            m_use = m_new == -INFINITY ? 0.0f : m_new;
            const float alpha = bump ? __builtin_amdgcn_exp2f(m_ref - m_use) : 1.0f;
            l_run *= alpha;
            m_ref = m_new;
#pragma unroll
            for (int d = 0; d < NB0; ++d) acc_o[d] *= alpha;
#pragma unroll
            for (int i = 0; i < 16; ++i) pf[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], scale_log2, -m_use));
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                pk[0][j] = (__bf16)pf[j];
                pk[1][j] = (__bf16)pf[8 + j];
            }
            __syncthreads();  // everyone has read the flags and the fast-path P
            Px[wave][0][lane] = __builtin_bit_cast(uint4, pk[0]);
            Px[wave][1][lane] = __builtin_bit_cast(uint4, pk[1]);
            __syncthreads();
        }
        float lsum = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) lsum += pf[i];
        l_run += lsum;
        // P^T fragments: our two key blocks (tile rows 32*side + [0,32)) and the partner's
        // (rows 32*(1-side) + [0,32)); the matching V rows are picked by address.
        const bf16x8 po0 = __builtin_bit_cast(bf16x8, Px[wave ^ 1][0][lane]);
        const bf16x8 po1 = __builtin_bit_cast(bf16x8, Px[wave ^ 1][1][lane]);

        // O^T[dim, row] += V^T[dim, key] P^T[key, row] over this wave's column blocks.
        // Element j of the lane's k-slice of a 16-key block is key
        // 16 kb + 8 (j/4) + 4 half + j%4: two transposing reads of 4 keys each. Key-block
        // major: the own key blocks first, so the partner's P has 16 MFMAs to arrive.
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int m = 0; m < NM; ++m) {  // PA MFMAs' worth of V^T reads in flight
            const int kb = m / NB0, d = m % NB0;
            const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(vlo[m % NVB], vhi[m % NVB], 0, 1, 2, 3, 4, 5, 6, 7));
            const bf16x8 b = kb == 0 ? pk[0] : kb == 1 ? pk[1] : kb == 2 ? po0 : po1;
            acc_o[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc_o[d], 0, 0, 0);
            if (m + PA < NM) vread(m + PA);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    if (kt0 < n_tiles) {  // workgroup-uniform; an empty key range leaves O = 0, LSE = -inf
        if constexpr (PAGED) bw_load(min(kt0, nblk - 1) & ~63);
        narrow_load_tile<T, DL, DR>(kv_lds0, lat, rope, tile_rows(kt0), wave, lane);
        for (int kt = kt0; kt < n_tiles; kt += 2) {
            tile_step(kv_lds0, kv_lds1, kt);
            if (kt + 1 >= n_tiles) break;
            tile_step(kv_lds1, kv_lds0, kt + 1);
        }
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // loads issued after the last tile landed before LDS is released

    // Row sums: this lane's share + the other half-wave's + the partner wave's.
    float l_w = l_run + __shfl_xor(l_run, 32);
    __syncthreads();
    mx[wave][lane] = l_w;
    __syncthreads();
    const float l_tot = l_w + mx[wave ^ 1][lane];
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    if (valid) {
        __bf16* orow = o_out + grow * DL;
#pragma unroll
        for (int d = 0; d < NB0; ++d) {
            const int db = side * NB0 + d;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                bf16x4 y;
#pragma unroll
                for (int e = 0; e < 4; ++e) y[e] = (__bf16)(acc_o[d][4 * g + e] * inv);
                *reinterpret_cast<bf16x4*>(orow + db * 32 + 8 * g + 4 * half) = y;
            }
        }
        if (side == 0 && half == 0) lse_out[grow] = (m_ref + __builtin_amdgcn_logf(l_tot)) * kLn2;
    }
    sched::mark_empty_slices(lse0, grow, valid && side == 0 && half == 0, split, wk.nsplit, kv_splits,
                             split_stride, H);
}

template <int DL, int DR, bool PAGED>
hipError_t launch_dense(const mla_partial_args& a, hipStream_t stream) {
    const int64_t grid = (((int64_t)a.T_loc * a.H + BM - 1) / BM + a.n_vrows) * a.kv_splits;
    hipLaunchKernelGGL((dense_partial_kernel<DL, DR, PAGED>), dim3((unsigned)grid), dim3(NT), 0, stream,
                       (const __bf16*)a.q, (const char*)a.latent_kv, (const char*)a.rope_k, a.cu_seqlens_q,
                       a.vrow_kv_start, a.positions, a.n_vrows, a.H, a.N_kv, a.scale * kLog2e,
                       (__bf16*)a.o_partial, a.lse, a.kv_splits, a.split_stride, a.vrow_kv_len, a.block_table,
                       a.bt_stride, a.vrow_req, a.kv_splits > 1 ? a.vrow_splits : nullptr, a.vrow_order);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_dense_partial(const mla_partial_args& a, hipStream_t stream) {
    if (a.D_latent == 512) return launch_dense_wide_partial(a, stream);  // 128-row workgroups
    return a.block_table ? launch_dense<64, 16, true>(a, stream) : launch_dense<64, 16, false>(a, stream);
}

}  // namespace mla
