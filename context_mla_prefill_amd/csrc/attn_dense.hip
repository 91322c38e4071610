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
//  * A workgroup (4 waves) owns BM = 128 rows of one virtual row, where a row is a
//    (token, head) pair: all heads share the KV, so token x head is the M dimension.
//    Each wave owns 32 rows; its Q rows live in registers for the whole KV loop.
//  * KV tiles of BN keys are staged HBM -> LDS once per workgroup and shared by all
//    heads and waves.
//  * Scores are computed transposed, S^T = K Q^T (v_mfma_f32_32x32x16_bf16, A = K from
//    LDS, B = Q^T from registers), so each lane holds scores of ONE query row: the
//    online-softmax max needs one cross-half exchange and the running sum stays
//    per-lane until the epilogue.
//  * The output is accumulated transposed, O^T += V^T P^T, so the P fragment is the
//    score accumulator re-packed to bf16 in place (no LDS round trip) and the per-row
//    rescale is a per-lane scalar. The key order inside a 16-key MFMA block is the
//    one the score layout gives each lane; V^T is read in that same order.
//  * Workgroups are launched longest-first (reverse of the flattened tile order), so
//    the long late-chunk tiles start first and the short ones fill the tail.
#include <math.h>

#include "internal.h"

namespace mla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BM = 64;   // rows per workgroup: two wave pairs of 32 rows
constexpr int BN = 32;   // keys per KV tile
constexpr int NT = 256;  // threads per workgroup
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescale = 8.0f;  // log2 headroom before the running max is moved

template <int DL, int DR>
struct Shape {
    static constexpr int DQK = DL + DR;
    static constexpr int KB = DQK / 16;      // 16-wide k-blocks of Q K^T
    static constexpr int NB = DL / 32;       // 32-wide column blocks of O
    static constexpr int STRIDE = DQK + 8;   // LDS row stride (bf16): +16 B breaks bank aliasing
    static constexpr int VECS = DQK / 8;     // 16-byte vectors per key row
    static constexpr int LAT_VECS = DL / 8;
    static constexpr int ROPE_VECS = DR / 8;
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

template <int DL, int DR>
__global__ __launch_bounds__(NT, 1) void dense_partial_kernel(
    const __bf16* __restrict__ q, const uint4* __restrict__ lat, const uint4* __restrict__ rope,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ vrow_kv_start,
    const int32_t* __restrict__ positions, int n_vrows, int H, int64_t N_kv, float scale_log2,
    __bf16* __restrict__ o_out, float* __restrict__ lse_out) {
    using S = Shape<DL, DR>;
    __shared__ __attribute__((aligned(16))) __bf16 Ks[BN * S::STRIDE];
    __shared__ __attribute__((aligned(16))) float4 Sx[NT / 64][4][64];  // partial-score exchange
    __shared__ int sh[NT];
    __shared__ int s_maxpos[NT / 64];

    int v, tile;
    find_tile((int)blockIdx.x, cu, n_vrows, H, sh, v, tile);
    if (v < 0) return;

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int pair = wave >> 1;
    const int side = wave & 1;    // which half of the QK k-blocks and of the O columns
    const int lane = tid & 63;
    const int half = lane >> 5;   // which 8-element half of a 16-wide k-block this lane holds
    const int l32 = lane & 31;

    const int tok0 = cu[v];
    const int nrows = (cu[v + 1] - tok0) * H;
    const int rloc = tile * BM + pair * 32 + l32;  // row inside the virtual row
    const bool valid = rloc < nrows;
    const int64_t grow = (int64_t)tok0 * H + rloc;  // global row (token-major, then head)
    const int pos = valid ? positions[tok0 + rloc / H] : -1;
    const int64_t kv0 = vrow_kv_start[v];

    // KV extent of the tile: largest position among its rows, plus one.
    int mp = pos;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) mp = max(mp, __shfl_xor(mp, off));
    if (lane == 0) s_maxpos[wave] = mp;

    // Q^T fragments of this wave's k-blocks: lane holds row l32, elements
    // [16 kb + 8 half, +8) of each block.
    constexpr int KB0 = (S::KB + 1) / 2;  // k-blocks of side 0; side 1 takes the rest
    constexpr int NB0 = S::NB / 2;        // O column blocks per side
    const int kb_lo = side ? KB0 : 0;
    const int kb_n = side ? S::KB - KB0 : KB0;
    bf16x8 qf[KB0];
    {
        const __bf16* qrow = q + grow * S::DQK + 8 * half;
#pragma unroll
        for (int k = 0; k < KB0; ++k) {
            qf[k] = (valid && k < kb_n) ? *reinterpret_cast<const bf16x8*>(qrow + (kb_lo + k) * 16)
                                        : bf16x8{};
        }
    }
    __syncthreads();
    int kv_hi = s_maxpos[0];
#pragma unroll
    for (int w = 1; w < NT / 64; ++w) kv_hi = max(kv_hi, s_maxpos[w]);
    kv_hi += 1;

    f32x16 acc_o[NB0];
#pragma unroll
    for (int d = 0; d < NB0; ++d) acc_o[d] = f32x16{};
    float m_run = -INFINITY;  // running (lazy) max of log2-domain scores of this lane's row
    float l_run = 0.0f;       // running sum over this lane's half of the keys

    const int n_tiles = (kv_hi + BN - 1) / BN;
    for (int kt = 0; kt < n_tiles; ++kt) {
        __syncthreads();
        // Stage KV rows [kt*BN, kt*BN + BN) of this request: latent || rope, zero past the end.
        for (int c = tid; c < BN * S::VECS; c += NT) {
            const int key = c / S::VECS;
            const int vec = c - key * S::VECS;
            const int64_t j = (int64_t)kt * BN + key;
            uint4 val = {0u, 0u, 0u, 0u};
            if (j < kv_hi && kv0 + j < N_kv) {
                val = vec < S::LAT_VECS ? lat[(kv0 + j) * S::LAT_VECS + vec]
                                        : rope[(kv0 + j) * S::ROPE_VECS + (vec - S::LAT_VECS)];
            }
            *reinterpret_cast<uint4*>(&Ks[key * S::STRIDE + vec * 8]) = val;
        }
        __syncthreads();

        // Partial S^T[key, row] over this wave's k-blocks, keys 8*(i/4) + 4*half + i%4.
        f32x16 s = f32x16{};
        {
            const __bf16* kp = &Ks[l32 * S::STRIDE + 8 * half + kb_lo * 16];
#pragma unroll
            for (int k = 0; k < KB0; ++k) {
                if (k < kb_n) {
                    const bf16x8 a = *reinterpret_cast<const bf16x8*>(kp + k * 16);
                    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[k], s, 0, 0, 0);
                }
            }
        }
        // Exchange partial scores with the other wave of the pair; both then hold the
        // same full scores (a + b == b + a exactly) and run the same softmax.
#pragma unroll
        for (int c = 0; c < 4; ++c) Sx[wave][c][lane] = make_float4(s[4 * c], s[4 * c + 1], s[4 * c + 2], s[4 * c + 3]);
        __syncthreads();
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const float4 o = Sx[wave ^ 1][c][lane];
            s[4 * c] += o.x;
            s[4 * c + 1] += o.y;
            s[4 * c + 2] += o.z;
            s[4 * c + 3] += o.w;
        }

        float mloc = -INFINITY;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int j = kt * BN + 8 * (i >> 2) + 4 * half + (i & 3);
            const float x = j <= pos ? s[i] * scale_log2 : -INFINITY;
            s[i] = x;
            mloc = fmaxf(mloc, x);
        }
        // Lazy rescale: the reference max only moves when the tile max exceeds it by more
        // than kRescale (log2 units), so p <= 2^kRescale and the O rescale is rare.
        // Numerator and denominator share the reference, so the result is unchanged.
        const float m_tile = fmaxf(mloc, __shfl_xor(mloc, 32));
        const bool bump = m_tile > m_run + kRescale;  // also true on the first live tile
        const float m_new = bump ? m_tile : m_run;
        const float m_use = m_new == -INFINITY ? 0.0f : m_new;
        const float alpha = bump ? __builtin_amdgcn_exp2f(m_run - m_use) : 1.0f;
        float lsum = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const float p = __builtin_amdgcn_exp2f(s[i] - m_use);
            s[i] = p;
            lsum += p;
        }
        l_run = l_run * alpha + lsum;
        m_run = m_new;
        if (__ballot(bump)) {
#pragma unroll
            for (int d = 0; d < NB0; ++d) acc_o[d] *= alpha;
        }

        bf16x8 pk[2];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            pk[0][j] = (__bf16)s[j];
            pk[1][j] = (__bf16)s[8 + j];
        }
        // O^T[dim, row] += V^T[dim, key] P^T[key, row] over this wave's column blocks;
        // element j of the lane's k-slice is key 16*kb2 + 8*(j/4) + 4*half + j%4, the
        // order the score layout produced.
#pragma unroll
        for (int d = 0; d < NB0; ++d) {
            const int db = side * NB0 + d;
#pragma unroll
            for (int kb2 = 0; kb2 < 2; ++kb2) {
                bf16x8 a;
                const __bf16* vp = &Ks[(16 * kb2 + 4 * half) * S::STRIDE + db * 32 + l32];
#pragma unroll
                for (int j = 0; j < 8; ++j) a[j] = vp[(8 * (j >> 2) + (j & 3)) * S::STRIDE];
                acc_o[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pk[kb2], acc_o[d], 0, 0, 0);
            }
        }
    }

    const float l_tot = l_run + __shfl_xor(l_run, 32);
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
        if (side == 0 && half == 0) lse_out[grow] = (m_run + __builtin_amdgcn_logf(l_tot)) * kLn2;
    }
}

template <int DL, int DR>
hipError_t launch_dense(const mla_partial_args& a, hipStream_t stream) {
    const int64_t grid = ((int64_t)a.T_loc * a.H + BM - 1) / BM + a.n_vrows;
    hipLaunchKernelGGL((dense_partial_kernel<DL, DR>), dim3((unsigned)grid), dim3(NT), 0, stream,
                       (const __bf16*)a.q, (const uint4*)a.latent_kv, (const uint4*)a.rope_k, a.cu_seqlens_q,
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
