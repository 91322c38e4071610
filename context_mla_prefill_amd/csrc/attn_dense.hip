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
#include "attn_core.h"

namespace mla {
namespace {

using namespace attn;

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
    __shared__ Exchange ex;
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

    const LaneOffsets<S> lo(side, lane);
    const int n_tiles = (kv_hi + BN - 1) / BN;

    // One KV tile: wait for it, publish it, start streaming the next tile into the other
    // buffer, then scores, softmax, P exchange and P V on this one. The two buffers are
    // distinct LDS objects, so the compiler can tell that the streaming loads never
    // touch the tile being read and does not wait for them.
    auto tile_step = [&](const char* kvt, char* nxt, int kt) {
#pragma unroll
        for (int kb = 0; kb < S::KB; ++kb) asm volatile("" : "+a"(qf[kb]));  // Q stays in AGPRs
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's loads of tile kt landed
        __syncthreads();                     // ... and every wave's; the other buffer is free
        if (kt + 1 < n_tiles) load_tile<S, DL, DR>(nxt, lat, rope, kv0, kt + 1, kv_hi, N_kv, wave, lane);
        const int key0 = kt * BN + 32 * side + 4 * half;  // key of s[0]
        auto causal = [&](f32x16& s) {
            if (kt * BN + 32 * side + 31 > pmin) {  // wave-uniform: a causal diagonal crosses these keys
#pragma unroll
                for (int i = 0; i < 16; ++i) s[i] = key0 + 8 * (i >> 2) + (i & 3) <= pos ? s[i] : -INFINITY;
            }
        };
        tile_compute<S, DL>(kvt, qf, acc_o, m_ref, l_run, scale_log2, wave, side, lane, lo, ex, causal, [] {});
    };

    load_tile<S, DL, DR>(kv_lds0, lat, rope, kv0, 0, kv_hi, N_kv, wave, lane);
    for (int kt = 0; kt < n_tiles; kt += 2) {
        tile_step(kv_lds0, kv_lds1, kt);
        if (kt + 1 >= n_tiles) break;
        tile_step(kv_lds1, kv_lds0, kt + 1);
    }
    write_rows<S, DL>(acc_o, m_ref, l_run, valid, grow, wave, side, lane, ex, o_out, lse_out);
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


}  // namespace mla
