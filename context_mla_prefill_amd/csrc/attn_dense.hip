// Rank-local causal MLA partial attention (dense), bf16 MFMA on gfx950.
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
//    all heads and waves. 16-byte chunks are XOR-swizzled by row to spread LDS banks.
//  * Scores are computed transposed, S^T = K Q^T (v_mfma_f32_32x32x16_bf16, A = K from
//    LDS, B = Q^T from registers); wave s of a pair scores keys [32 s, 32 s + 32) of the
//    tile. Each lane then holds scores of ONE query row, so the row max needs one
//    cross-half exchange and the running sum stays per lane until the epilogue.
//  * The output is accumulated transposed, O^T += V^T P^T; wave s of a pair owns output
//    columns [256 s, 256 s + 256) and needs P for all 64 keys, so the two waves swap
//    their bf16 P fragments through LDS. The P fragment is the score accumulator
//    re-packed in place; V^T comes from transposing LDS reads (ds_read_b64_tr_b16) in
//    the key order the score layout gives each lane.
//  * Online softmax with a lazy reference max: the reference of a row moves only when a
//    tile max exceeds it by more than kRescale (log2 units). Tiles that move no
//    reference (nearly all of them) need no max exchange and no O rescale; a tile that
//    does takes a workgroup-uniform slow path with one extra barrier.
//  * Workgroups are launched longest-first (reverse of the flattened tile order), so
//    the long late-chunk tiles start first and the short ones fill the tail.
#include <math.h>

#include "internal.h"

namespace mla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

constexpr int BM = 64;   // rows per workgroup: two wave pairs of 32 rows
constexpr int BN = 64;   // keys per KV tile (32 per wave of a pair)
constexpr int NT = 256;  // threads per workgroup
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescale = 8.0f;
constexpr int QK_AHEAD = 8;  // Q K^T operand reads kept in flight ahead of the MFMA chain
constexpr int PV_AHEAD = 4;  // P V MFMAs' worth of V^T reads kept in flight  // log2 headroom before the running max is moved

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

__device__ __forceinline__ int block_scan_incl(int v, int* sh) {
    const int t = threadIdx.x;
    sh[t] = v;
    __syncthreads();
    for (int off = 1; off < NT; off <<= 1) {
        const int add = t >= off ? sh[t - off] : 0;
        __syncthreads();
        sh[t] += add;
        __syncthreads();
    }
    const int r = sh[t];
    __syncthreads();
    return r;
}

// Finds the (virtual row, tile) of this workgroup. Tiles are numbered longest-first:
// virtual rows from last to first, and inside a row from its last tile to its first.
__device__ __forceinline__ void find_tile(int ridx, const int32_t* __restrict__ cu, int n_vrows, int H,
                                          int* sh, int& v_out, int& tile_out) {
    __shared__ int s_v, s_tile, s_carry;
    if (threadIdx.x == 0) {
        s_v = -1;
        s_tile = 0;
        s_carry = 0;
    }
    __syncthreads();
    for (int base = 0; base < n_vrows; base += NT) {
        const int k = base + threadIdx.x;
        const int v = n_vrows - 1 - k;
        int cnt = 0;
        if (k < n_vrows) {
            const int len = cu[v + 1] - cu[v];
            cnt = len > 0 ? (int)(((int64_t)len * H + BM - 1) / BM) : 0;
        }
        const int incl = block_scan_incl(cnt, sh);
        const int lo = s_carry + incl - cnt;
        if (k < n_vrows && ridx >= lo && ridx < lo + cnt) {
            s_v = v;
            s_tile = cnt - 1 - (ridx - lo);
        }
        __syncthreads();
        if (threadIdx.x == NT - 1) s_carry += incl;
        __syncthreads();
        if (s_v >= 0) break;
    }
    v_out = s_v;
    tile_out = s_tile;
}

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// One wave-wide direct-to-LDS load: lane l copies 16 bytes from `src` to LDS address
// lds_base + 16*l.
__device__ __forceinline__ void lds_dma16(const void* src, char* lds_base) {
    __builtin_amdgcn_global_load_lds(src, (lds_void*)lds_base, 16, 0, 0);
}

// Issues the direct-to-LDS loads of KV tile kt (keys [kt*BN, kt*BN+BN) of the request)
// into `dst`. A load writes 64 consecutive 16-byte LDS chunks, one per lane; lanes that
// would land on a row pad are switched off. Keys past the tile's extent repeat the last
// valid row (finite values; their scores are masked). Wave w issues loads w, w+4, ...
template <class S, int DL, int DR>
__device__ __forceinline__ void load_tile(char* dst, const char* __restrict__ lat, const char* __restrict__ rope,
                                          int64_t kv0, int kt, int kv_hi, int64_t N_kv, int wave, int lane) {
    constexpr int LV = S::LAT_VECS + 1, RV = S::ROPE_VECS + 1;
    const int lk = DL * 2 == 1024 ? 0 : lane / LV;            // row of the load this lane fills
    const int lc = DL * 2 == 1024 ? lane : lane - lk * LV;    // 16-byte chunk inside that row
    const bool lon = DL * 2 == 1024 || (lc < S::LAT_VECS && lk < S::LAT_ROWS_PER_LOAD);
    const int rk = lane / RV;
    const int rc = lane - rk * RV;
    const bool ron = rc < S::ROPE_VECS && rk < S::ROPE_ROWS_PER_LOAD;
    const int64_t last = min((int64_t)kv_hi - 1, N_kv - 1 - kv0);
#pragma unroll
    for (int i = 0; i < (S::LAT_LOADS + 3) / 4; ++i) {
        const int n = i * 4 + wave;
        if (n >= S::LAT_LOADS) break;
        const int r = n * S::LAT_ROWS_PER_LOAD + lk;
        const int64_t j = min((int64_t)kt * BN + r, last);
        if (lon && r < BN)
            lds_dma16(lat + (kv0 + j) * (DL * 2) + lc * 16, dst + n * S::LAT_ROWS_PER_LOAD * S::LAT_STRIDE);
    }
#pragma unroll
    for (int i = 0; i < (S::ROPE_LOADS + 3) / 4; ++i) {
        const int n = i * 4 + ((wave + 2) & 3);
        if (n >= S::ROPE_LOADS) break;
        const int r = n * S::ROPE_ROWS_PER_LOAD + rk;
        const int64_t j = min((int64_t)kt * BN + r, last);
        if (ron && r < BN)
            lds_dma16(rope + (kv0 + j) * (DR * 2) + rc * 16,
                      dst + S::ROPE_OFF + n * S::ROPE_ROWS_PER_LOAD * S::ROPE_STRIDE);
    }
}

template <int DL, int DR>
__global__ __launch_bounds__(NT, 1) void dense_partial_kernel(
    const __bf16* __restrict__ q, const char* __restrict__ lat, const char* __restrict__ rope,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ vrow_kv_start,
    const int32_t* __restrict__ positions, int n_vrows, int H, int64_t N_kv, float scale_log2,
    __bf16* __restrict__ o_out, float* __restrict__ lse_out) {
    using S = Shape<DL, DR>;
    __shared__ __attribute__((aligned(1024))) char kv_lds0[S::TILE_BYTES];  // KV tile double buffer:
    __shared__ __attribute__((aligned(1024))) char kv_lds1[S::TILE_BYTES];  // two separate objects
    __shared__ __attribute__((aligned(16))) uint4 Px[NT / 64][2][64];  // P fragment exchange
    __shared__ float mx[NT / 64][64];                                  // tile-max exchange (slow path)
    __shared__ int flag[NT / 64];
    __shared__ int sh[NT];
    __shared__ int s_maxpos[NT / 64];

    int v, tile;
    find_tile((int)blockIdx.x, cu, n_vrows, H, sh, v, tile);
    v = __builtin_amdgcn_readfirstlane(v);  // workgroup-uniform: keep it in SGPRs
    tile = __builtin_amdgcn_readfirstlane(tile);
    if (v < 0) return;

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
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
    bf16x8 qf[S::KB];
    {
        const __bf16* qrow = q + grow * S::DQK + 8 * half;
#pragma unroll
        for (int kb = 0; kb < S::KB; ++kb)
            qf[kb] = valid ? *reinterpret_cast<const bf16x8*>(qrow + kb * 16) : bf16x8{};
    }
    __syncthreads();
    int kv_hi = s_maxpos[0];
#pragma unroll
    for (int w = 1; w < NT / 64; ++w) kv_hi = max(kv_hi, s_maxpos[w]);
    kv_hi = __builtin_amdgcn_readfirstlane(kv_hi + 1);
    // smallest position among this wave's rows: key blocks at or below it need no mask
    int pmin = valid ? pos : INT32_MAX;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) pmin = min(pmin, __shfl_xor(pmin, off));
    pmin = __builtin_amdgcn_readfirstlane(pmin);

    constexpr int NB0 = S::NB / 2;  // O column blocks per wave
    f32x16 acc_o[NB0];
#pragma unroll
    for (int d = 0; d < NB0; ++d) acc_o[d] = f32x16{};
    float m_ref = -INFINITY;  // lazy reference max (log2 domain) of this lane's row
    float l_run = 0.0f;       // running sum over this lane's share of the keys

    // Per-lane LDS offsets inside a tile (everything else is an immediate):
    //  * Q K^T reads: key row 32*side + l32, 8 elements at 8*half of each 16-wide k-block;
    //  * V^T reads: key row 4*half + (lane%16)/4 (+16 kb, +8), dims 16*((lane/16)%2) + 4*(lane%4).
    const int k_lat_off = (32 * side + l32) * S::LAT_STRIDE + 16 * half;
    const int k_rope_off = S::ROPE_OFF + (32 * side + l32) * S::ROPE_STRIDE + 16 * half;
    const int v_off = (4 * half + ((lane & 15) >> 2)) * S::LAT_STRIDE +
                      2 * (16 * ((lane >> 4) & 1) + 4 * (lane & 3));

    const int n_tiles = (kv_hi + BN - 1) / BN;

    // One KV tile: wait for it, publish it, start streaming the next tile into the other
    // buffer, then scores, softmax, P exchange and P V on this one. The two buffers are
    // distinct LDS objects, so the compiler can tell that the streaming loads never
    // touch the tile being read and does not wait for them.
    auto tile_step = [&](const char* kvt, char* nxt, int kt) {
#pragma unroll
        for (int kb = 0; kb < S::KB; ++kb) asm volatile("" : "+a"(qf[kb]));
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's loads of tile kt landed
        __syncthreads();                     // ... and every wave's; the other buffer is free
        if (kt + 1 < n_tiles) load_tile<S, DL, DR>(nxt, lat, rope, kv0, kt + 1, kv_hi, N_kv, wave, lane);
        // S^T[key, row] for keys 32*side + 8*(i/4) + 4*half + i%4 of this tile, row l32.
        f32x16 s = f32x16{};
        {
            const char* kl = kvt + k_lat_off;
            const char* kr = kvt + k_rope_off;
            __builtin_amdgcn_sched_barrier(0);
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
            }
            __builtin_amdgcn_sched_group_barrier(0x008, AHEAD, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
        const int key0 = kt * BN + 32 * side + 4 * half;  // key of s[0]
        if (kt * BN + 32 * side + 31 > pmin) {  // wave-uniform: a causal diagonal crosses these keys
#pragma unroll
            for (int i = 0; i < 16; ++i) s[i] = key0 + 8 * (i >> 2) + (i & 3) <= pos ? s[i] : -INFINITY;
        }
        float smax = s[0];
#pragma unroll
        for (int i = 1; i < 16; ++i) smax = fmaxf(smax, s[i]);
        smax = fmaxf(smax, __shfl_xor(smax, 32));
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
        __syncthreads();
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
        // 16 kb + 8 (j/4) + 4 half + j%4: two transposing reads of 4 keys each.
        __builtin_amdgcn_sched_barrier(0);
        const char* v_own = kvt + v_off + (32 * side) * S::LAT_STRIDE;
        const char* v_oth = kvt + v_off + (32 * (side ^ 1)) * S::LAT_STRIDE;
#pragma unroll
        for (int d = 0; d < NB0; ++d) {
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                const char* p0 = (kb < 2 ? v_own : v_oth) + (16 * (kb & 1)) * S::LAT_STRIDE + (side * NB0 + d) * 64;
                const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p0);
                const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p0 + 8 * S::LAT_STRIDE));
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
    };

    load_tile<S, DL, DR>(kv_lds0, lat, rope, kv0, 0, kv_hi, N_kv, wave, lane);
    for (int kt = 0; kt < n_tiles; kt += 2) {
        tile_step(kv_lds0, kv_lds1, kt);
        if (kt + 1 >= n_tiles) break;
        tile_step(kv_lds1, kv_lds0, kt + 1);
    }

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
}

template <int DL, int DR>
hipError_t launch_dense(const mla_partial_args& a, hipStream_t stream) {
    const int64_t grid = ((int64_t)a.T_loc * a.H + BM - 1) / BM + a.n_vrows;
    hipLaunchKernelGGL((dense_partial_kernel<DL, DR>), dim3((unsigned)grid), dim3(NT), 0, stream,
                       (const __bf16*)a.q, (const char*)a.latent_kv, (const char*)a.rope_k, a.cu_seqlens_q,
                       a.vrow_kv_start, a.positions, a.n_vrows, a.H, a.N_kv, a.scale * kLog2e,
                       (__bf16*)a.o_partial, a.lse);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_dense_partial(const mla_partial_args& a, hipStream_t stream) {
    if (a.D_latent == 512) return launch_dense<512, 64>(a, stream);
    return launch_dense<64, 16>(a, stream);
}

hipError_t launch_sparse_partial(const mla_partial_args&, hipStream_t) { return hipErrorNotSupported; }

}  // namespace mla
