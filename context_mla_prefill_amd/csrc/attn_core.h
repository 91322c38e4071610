// Shared pieces of the MLA partial-attention kernels (dense causal and top-k sparse):
// fragment types, the workgroup shape, the key-row permutation of an LDS tile, the
// direct-to-LDS load, and the per-tile compute on one LDS-resident KV tile (transposed
// Q K^T, online softmax with a lazy reference max, the wave-pair P exchange, transposed
// P V) used by the sparse kernel. The dense kernel runs the same per-tile arithmetic in
// its own copy, whose Q K^T section also issues the next tile's loads between MFMAs.
#pragma once

#include <math.h>

#include "internal.h"

namespace mla {
namespace attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int BM = 64;   // rows (token x head) per workgroup: two wave pairs of 32 rows
constexpr int BN = 64;   // keys per KV tile (32 per wave of a pair)
constexpr int NT = 256;  // threads per workgroup
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescale = 8.0f;  // log2 headroom before the running max is moved
constexpr int QK_AHEAD = 8;       // Q K^T operand reads kept in flight ahead of the MFMA chain
constexpr int PV_AHEAD = 4;       // P V MFMAs' worth of V^T reads kept in flight

template <int DL, int DR>
struct Shape {
    static constexpr int DQK = DL + DR;
    static constexpr int KB = DQK / 16;      // 16-wide k-blocks of Q K^T
    static constexpr int NB = DL / 32;       // 32-wide column blocks of O
    static constexpr int LAT_VECS = DL / 8;      // 16-byte chunks of a latent row
    static constexpr int ROPE_VECS = DR / 8;     // 16-byte chunks of a rope row
    // LDS tile: latent rows at a stride of DL*2 + 16 bytes (one direct-to-LDS load per
    // row when DL*2 == 1024, several rows per load otherwise), then rope rows at a
    // stride of DR*2 + 16 bytes. The 16-byte pad puts consecutive rows on different
    // banks for both the row reads of Q K^T and the transposing reads of P V.
    static constexpr int LAT_STRIDE = DL * 2 + 16;
    static constexpr int ROPE_STRIDE = DR * 2 + 16;
    static constexpr int ROPE_OFF = BN * LAT_STRIDE;
    static constexpr int TILE_BYTES = ROPE_OFF + BN * ROPE_STRIDE;
    // rows written per wave-wide load (a load covers 64 lanes x 16 bytes)
    static constexpr int LAT_ROWS_PER_LOAD = 64 / (LAT_VECS + 1) > 0 ? 64 / (LAT_VECS + 1) : 1;
    static constexpr int ROPE_ROWS_PER_LOAD = 64 / (ROPE_VECS + 1);
    static constexpr int LAT_LOADS = DL * 2 == 1024 ? BN : (BN + LAT_ROWS_PER_LOAD - 1) / LAT_ROWS_PER_LOAD;
    static constexpr int ROPE_LOADS = (BN + ROPE_ROWS_PER_LOAD - 1) / ROPE_ROWS_PER_LOAD;
    static_assert(DQK % 16 == 0 && DL % 32 == 0 && DR % 8 == 0, "tile shape");
};

// One wave-wide direct-to-LDS load: lane l copies 16 bytes from `src` to LDS address
// lds_base + 16*l.
__device__ __forceinline__ void lds_dma16(const void* src, char* lds_base) {
    __builtin_amdgcn_global_load_lds(src, (lds_void*)lds_base, 16, 0, 0);
}

// Buffer-resource flags (gfx9 raw buffer: 32-bit data format, no swizzle).
constexpr int kBufferFlags = 0x00020000;

// Direct-to-LDS buffer load: lane l copies 16 bytes from byte offset voff of the buffer to
// LDS address lds_base + 16*l. Buffer (not global) loads: the compiler counts a global
// (flat-family) load into LDS as an LDS access of unknown order and then waits for every
// LDS read at once instead of keeping operand reads in flight.
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, char* lds_base) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)lds_base, 16, voff, 0, 0, 0);
}

// Workgroup barrier that orders LDS only: waits for this wave's LDS operations but not for
// its loads into LDS, which stay in flight across it (__syncthreads() also waits for every
// outstanding vector-memory load).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Value of x in lane l ^ 32: one VALU lane swap of the two half-waves, no LDS round trip.
__device__ __forceinline__ float half_swap(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(int, x), __builtin_bit_cast(int, x), false, false);
    return __builtin_bit_cast(float, (int)((__lane_id() < 32) ? r[1] : r[0]));
}

// LDS the two waves of a pair exchange through.
struct Exchange {
    uint4 Px[NT / 64][2][64];  // bf16 P fragments
    float mx[NT / 64][64];     // tile maxima (slow path) and row sums (epilogue)
    int flag[NT / 64];         // "needs a new reference max" per wave
};

// Score row -> LDS key row. Inside every block of 16 keys, score row r lives in LDS row
// kperm(r) = 4*(r%4) + 2*((r/8)%2) + (r/4)%2. With the 1040-byte row stride (an odd number
// of 16-byte bank slots) this makes both read patterns bank-conflict free: the Q K^T row
// reads (16 lanes on 16 distinct rows of a block) and the transposing V^T reads (each
// 16-lane group reads the 4 key rows one tr-read covers, which kperm places 4 rows apart).
__device__ __forceinline__ constexpr int kperm(int r) { return 4 * (r & 3) + 2 * ((r >> 3) & 1) + ((r >> 2) & 1); }

// Tile key (0..63) of score s[i] of a lane in half `half` of wave side `side`: score row
// m = 8*(i/4) + 4*half + i%4 of this wave's 32 rows.
__device__ __forceinline__ int score_key(int side, int half, int i) {
    return 32 * side + 16 * (i >> 3) + kperm(8 * ((i >> 2) & 1) + 4 * half + (i & 3));
}

// Sets to -inf the scores s[i] whose tile key score_key(side, half, i) has a clear bit in
// `bits`. score_key(side, half, i) = 32 side + half + off(i) with the constant
// off(i) = 16 (i/8) + 4 (i%4) + 2 ((i/4)%2), so one shift per lane and constant bit tests do it.
__device__ __forceinline__ void mask_keys(f32x16& s, uint64_t bits, int side, int half) {
    const uint32_t w = (uint32_t)(bits >> (32 * side + half));
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int off = 16 * (i >> 3) + 4 * (i & 3) + 2 * ((i >> 2) & 1);
        s[i] = (w >> off) & 1u ? s[i] : -INFINITY;
    }
}

// Per-lane LDS offsets inside a tile (everything else is an immediate):
//  * Q K^T reads: LDS row of score row l32, 8 elements at 8*half of each 16-wide k-block
//    (latent offsets from the latent rows' base, rope offsets from the rope rows' base);
//  * V^T reads (first of the two per MFMA): LDS row of score row 4*half + (lane%16)/4 of
//    the key block, dims 16*((lane/16)%2) + 4*(lane%4); the second read is 2 rows further.
template <class S>
struct LaneOffsets {
    int k_lat, k_rope, v;
    __device__ __forceinline__ LaneOffsets(int side, int lane) {
        const int half = lane >> 5, l32 = lane & 31;
        const int krow = 32 * side + 16 * (l32 >> 4) + kperm(l32 & 15);
        k_lat = krow * S::LAT_STRIDE + 16 * half;
        k_rope = krow * S::ROPE_STRIDE + 16 * half;
        v = kperm(4 * half + ((lane & 15) >> 2)) * S::LAT_STRIDE + 2 * (16 * ((lane >> 4) & 1) + 4 * (lane & 3));
    }
};

// Scores, softmax and P V of one LDS-resident tile for this wave: latent rows at kvl, rope
// rows at kvr (separate LDS objects, so loads streaming into one are not taken to alias
// reads of the other).
//  mask(s):          applies -inf to scores of keys the row must not see (s[i] is tile
//                    key score_key(side, half, i), for row l32);
//  after_exchange(): runs right after the barrier that publishes the P fragments, when
//                    every wave has finished its Q K^T reads of this tile;
//  issue(i):         (NLOADS > 0) issues vector-memory load i of NLOADS; the loads are
//                    scheduled one after every LOAD_GAP-th Q K^T MFMA, so the vector memory
//                    pipe drains them while the matrix core runs instead of stalling the wave
//                    on a burst.
struct NoLoads {
    __device__ __forceinline__ void operator()(int) const {}
};
constexpr int LOAD_GAP = 2;

template <class S, int DL, int NLOADS = 0, class Mask, class Hook, class Issue = NoLoads>
__device__ __forceinline__ void tile_compute(const char* kvl, const char* kvr, const bf16x8 (&qf)[S::KB],
                                             f32x16 (&acc_o)[S::NB / 2],
                                             float& m_ref, float& l_run, float scale_log2, int wave, int side,
                                             int lane, const LaneOffsets<S>& lo, Exchange& ex, Mask&& mask,
                                             Hook&& after_exchange, Issue&& issue = Issue{}) {
    static_assert(NLOADS <= S::KB / LOAD_GAP, "loads fit among the Q K^T MFMAs");
    constexpr int NB0 = S::NB / 2;
    // S^T[key, row] for keys 32*side + 8*(i/4) + 4*half + i%4 of this tile, row l32.
    f32x16 s = f32x16{};
    {
        const char* kl = kvl + lo.k_lat;
        const char* kr = kvr + lo.k_rope;
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < NLOADS; ++i) issue(i);
#pragma unroll
        for (int kb = 0; kb < S::KB; ++kb) {
            const char* ap = kb < DL / 16 ? kl + kb * 32 : kr + (kb - DL / 16) * 32;
            const bf16x8 a = *reinterpret_cast<const bf16x8*>(ap);
            s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kb], s, 0, 0, 0);
        }
        // Keep QK_AHEAD operand reads in flight ahead of the MFMA chain.
        constexpr int AHEAD = S::KB < QK_AHEAD ? S::KB : QK_AHEAD;
        __builtin_amdgcn_sched_group_barrier(0x100, AHEAD, 0);
#pragma unroll
        for (int kb = 0; kb < S::KB - AHEAD; ++kb) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            if (kb % LOAD_GAP == 0 && kb / LOAD_GAP < NLOADS) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, AHEAD, 0);
        __builtin_amdgcn_sched_barrier(0);
    }
    mask(s);
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
    ex.Px[wave][0][lane] = __builtin_bit_cast(uint4, pk[0]);
    ex.Px[wave][1][lane] = __builtin_bit_cast(uint4, pk[1]);
    ex.mx[wave][lane] = mloc;
    const bool any_need = __ballot(need) != 0;
    if (lane == 0) ex.flag[wave] = any_need;
    lds_barrier();
    after_exchange();
    int slow = 0;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) slow |= ex.flag[w];
    if (slow) {  // workgroup-uniform
        const float m_pair = fmaxf(mloc, ex.mx[wave ^ 1][lane]);
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
        lds_barrier();  // everyone has read the flags and the fast-path P
        ex.Px[wave][0][lane] = __builtin_bit_cast(uint4, pk[0]);
        ex.Px[wave][1][lane] = __builtin_bit_cast(uint4, pk[1]);
        lds_barrier();
    }
    float lsum = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) lsum += pf[i];
    l_run += lsum;
    // P^T fragments: our two key blocks (tile rows 32*side + [0,32)) and the partner's
    // (rows 32*(1-side) + [0,32)); the matching V rows are picked by address.
    const bf16x8 po0 = __builtin_bit_cast(bf16x8, ex.Px[wave ^ 1][0][lane]);
    const bf16x8 po1 = __builtin_bit_cast(bf16x8, ex.Px[wave ^ 1][1][lane]);

    // O^T[dim, row] += V^T[dim, key] P^T[key, row] over this wave's column blocks.
    // Element j of the lane's k-slice of a 16-key block is key
    // 16 kb + 8 (j/4) + 4 half + j%4: two transposing reads of 4 keys each.
    __builtin_amdgcn_sched_barrier(0);
    // Byte offsets from the tile base, each read addressed by one offset from kvl (a chain of
    // pointer steps would hide from alias analysis that the reads stay inside this tile's
    // buffer, and the compiler would then wait for loads streaming into the other one).
    const int v_own = lo.v + (32 * side) * S::LAT_STRIDE;
    const int v_oth = lo.v + (32 * (side ^ 1)) * S::LAT_STRIDE;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {  // own key blocks first: the partner's P has time to arrive
#pragma unroll
        for (int d = 0; d < NB0; ++d) {
            const int o0 = (kb < 2 ? v_own : v_oth) + (16 * (kb & 1)) * S::LAT_STRIDE + (side * NB0 + d) * 64;
            const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(kvl + o0));
            const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(kvl + (o0 + 2 * S::LAT_STRIDE)));
            const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            const bf16x8 b = kb == 0 ? pk[0] : kb == 1 ? pk[1] : kb == 2 ? po0 : po1;
            acc_o[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc_o[d], 0, 0, 0);
        }
    }
    {
        // two transposing reads per MFMA, PV_AHEAD MFMAs' worth of reads in flight
        constexpr int NM = NB0 * 4;
        constexpr int AHEAD = NM < PV_AHEAD ? NM : PV_AHEAD;
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * AHEAD, 0);
#pragma unroll
        for (int m = 0; m < NM - AHEAD; ++m) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, AHEAD, 0);
        __builtin_amdgcn_sched_barrier(0);
    }
}

// Normalises O by the row sum (this lane's share, the other half-wave's and the partner
// wave's) and writes this wave's output columns and, once per row, the natural-log LSE.
template <class S, int DL>
__device__ __forceinline__ void write_rows(const f32x16 (&acc_o)[S::NB / 2], float m_ref, float l_run, bool valid,
                                           int64_t grow, int wave, int side, int lane, Exchange& ex,
                                           __bf16* __restrict__ o_out, float* __restrict__ lse_out) {
    constexpr int NB0 = S::NB / 2;
    const int half = lane >> 5;
    float l_w = l_run + __shfl_xor(l_run, 32);
    __syncthreads();
    ex.mx[wave][lane] = l_w;
    __syncthreads();
    const float l_tot = l_w + ex.mx[wave ^ 1][lane];
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
}

}  // namespace attn
}  // namespace mla
