// Log-sum-exp merge of per-rank partial attention into global token order, with the
// per-head sink in the final denominator exactly once.
//
// "[DeepSeekV4][PCP] Enable context-parallel prefill for hybrid KV and MegaMoE",
// "Purpose": each rank computes a local partial attention, LSE and output are then
// merged globally and attn_sink is applied only once; "Main challenges": the sink
// must not be applied on each rank. Global order restore: "[Core] Add MRV2
// virtual-batch PCP for MLA", "DualChunkSwap partitioning".
//
// Per (token t, head h): M = max(s_h, max_k L_k), D = exp(s_h-M) + sum_k exp(L_k-M),
// O = sum_k exp(L_k-M) O_k / D, LSE = M + log D, all in fp32; O stored bf16 (RNE).
//
// HBM-bound streaming: one workgroup per (token, group of heads), a group being as many
// whole heads as one round of loads covers (NT * UNROLL 16-byte vectors; 16 heads of 512).
// Its first threads turn the token's contributor LSEs and the sinks into per-(contributor,
// head) weights in LDS; then the workgroup streams the group's output elements, 16 bytes per
// thread and UNROLL vectors in flight, reading each contributor's rows (contiguous bf16) with
// full-width coalesced non-temporal loads (every byte is read at most once; a contributor
// whose weight is zero is not read).
#include <math.h>

#include "internal.h"

namespace mla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int NT = 256;
constexpr int MAXP = 64;
constexpr int UNROLL = 4;  // vectors per thread in flight

__global__ __launch_bounds__(NT) void merge_kernel(
    const u32x4* __restrict__ o_cat, const float* __restrict__ lse_cat,
    const int32_t* __restrict__ merge_src, int P, int S, int64_t split_stride, int H, int G, int HG, int64_t R_total,
    const float* __restrict__ sink, u32x4* __restrict__ o_out, float* __restrict__ lse_out) {
    __shared__ int rows[MAXP];
    __shared__ int n_rows;
    // exp(L_k - M) / D per contributor and head, [P * S][H] floats in dynamic LDS sized by the
    // launch (a few hundred bytes for 4 ranks of 16 heads, so many workgroups share a CU)
    extern __shared__ float wts_dyn[];
    auto wts = [&](int k, int h) -> float& { return wts_dyn[k * H + h]; };
    const int n_groups = (H + HG - 1) / HG;
    const int64_t t = blockIdx.x / n_groups;
    const int h_lo = (int)(blockIdx.x - t * n_groups) * HG;  // heads [h_lo, h_hi) of token t
    const int h_hi = min(H, h_lo + HG);
    const int tid = threadIdx.x;
    if (tid == 0) {  // contributors: every rank's row, in each of its S split slices
        int n = 0;
        for (int k = 0; k < P; ++k) {
            const int64_t r0 = merge_src[t * P + k];
            if (r0 < 0) continue;
            for (int s = 0; s < S; ++s) {
                const int64_t r = r0 + s * split_stride;
                if (r < R_total) rows[n++] = (int)r;
            }
        }
        n_rows = n;
    }
    __syncthreads();
    const int n = n_rows;
    for (int h = h_lo + tid; h < h_hi; h += NT) {
        const float sig = sink ? sink[h] : -INFINITY;
        float M = sig;
        for (int k = 0; k < n; ++k) M = fmaxf(M, lse_cat[(int64_t)rows[k] * H + h]);
        float D = 0.0f;
        for (int k = 0; k < n; ++k) wts(k, h) = 0.0f;
        if (M != -INFINITY) {
            D = sig == -INFINITY ? 0.0f : expf(sig - M);
            for (int k = 0; k < n; ++k) {
                const float w = expf(lse_cat[(int64_t)rows[k] * H + h] - M);
                wts(k, h) = w;
                D += w;
            }
        }
        const float inv = D > 0.0f ? 1.0f / D : 0.0f;
        for (int k = 0; k < n; ++k) wts(k, h) *= inv;
        if (lse_out) lse_out[t * H + h] = M == -INFINITY ? -INFINITY : M + logf(D);
    }
    __syncthreads();
    const int V = H * G;  // 16-byte vectors of a token's output
    const int V_hi = h_hi * G;  // this group's vectors: [h_lo * G, V_hi)
    const u32x4* src_base = o_cat;
    u32x4* dst = o_out + t * V;
    for (int v0 = h_lo * G + tid; v0 < V_hi; v0 += NT * UNROLL) {
        float acc[UNROLL][8];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u)
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[u][j] = 0.0f;
        for (int k = 0; k < n; ++k) {
            const u32x4* src = src_base + (int64_t)rows[k] * V;
            u32x4 raw[UNROLL];
            float w[UNROLL];
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) {
                const int v = v0 + u * NT;
                w[u] = v < V_hi ? wts(k, v / G) : 0.0f;
                // a zero weight (LSE -inf: an empty key range, or a slice the row does not use)
                // reads nothing: such a slice's output may never have been written
                raw[u] = w[u] != 0.0f ? __builtin_nontemporal_load(src + v) : u32x4{0u, 0u, 0u, 0u};
            }
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) {
                const bf16x8 x = __builtin_bit_cast(bf16x8, raw[u]);
#pragma unroll
                for (int j = 0; j < 8; ++j) acc[u][j] += w[u] * (float)x[j];
            }
        }
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int v = v0 + u * NT;
            if (v < V_hi) {
                bf16x8 y;
#pragma unroll
                for (int j = 0; j < 8; ++j) y[j] = (__bf16)acc[u][j];
                __builtin_nontemporal_store(__builtin_bit_cast(u32x4, y), dst + v);
            }
        }
    }
}

}  // namespace

hipError_t launch_merge(const void* o_cat, const float* lse_cat, const int32_t* merge_src,
                        int32_t P, int64_t T_glob, int32_t H, int32_t D_v, int64_t R_total,
                        int32_t kv_splits, int64_t split_stride, const float* sink, void* o_out,
                        float* lse_out, hipStream_t stream) {
    const int G = D_v / 8;
    const int HG = max(1, NT * UNROLL / G);  // heads per workgroup
    const int64_t grid = T_glob * ((H + HG - 1) / HG);
    const size_t wts_bytes = (size_t)min(P * kv_splits, MAXP) * H * sizeof(float);
    hipLaunchKernelGGL(merge_kernel, dim3((unsigned)grid), dim3(NT), wts_bytes, stream, (const u32x4*)o_cat, lse_cat,
                       merge_src, P, kv_splits, split_stride, H, G, HG, R_total, sink, (u32x4*)o_out, lse_out);
    return hipGetLastError();
}

}  // namespace mla
