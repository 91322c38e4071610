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
// HBM-bound streaming: D_v/8 consecutive threads own one (t, h) row and each moves 16
// bytes per contributor, so every contributor row is read with full-width coalesced
// loads and the output row written the same way.
#include <math.h>

#include "internal.h"

namespace mla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__global__ __launch_bounds__(256) void merge_kernel(
    const uint4* __restrict__ o_cat, const float* __restrict__ lse_cat,
    const int32_t* __restrict__ merge_src, int P, int64_t n_rows, int H, int G, int64_t R_total,
    const float* __restrict__ sink, uint4* __restrict__ o_out, float* __restrict__ lse_out) {
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t row = gid / G;
    if (row >= n_rows) return;
    const int v = (int)(gid - row * G);
    const int64_t t = row / H;
    const int h = (int)(row - t * H);
    const float sig = sink ? sink[h] : -INFINITY;
    const int32_t* src = merge_src + t * P;
    float M = sig;
    for (int k = 0; k < P; ++k) {
        const int64_t r = src[k];
        if (r >= 0 && r < R_total) M = fmaxf(M, lse_cat[r * H + h]);
    }
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    float D = 0.0f;
    if (M != -INFINITY) {
        D = (sig == -INFINITY) ? 0.0f : expf(sig - M);
        for (int k = 0; k < P; ++k) {
            const int64_t r = src[k];
            if (r < 0 || r >= R_total) continue;
            const float w = expf(lse_cat[r * H + h] - M);
            D += w;
            const uint4 raw = o_cat[(r * H + h) * G + v];
            const bf16x8 x = __builtin_bit_cast(bf16x8, raw);
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[j] += w * (float)x[j];
        }
    }
    const float inv = D > 0.0f ? 1.0f / D : 0.0f;
    bf16x8 y;
#pragma unroll
    for (int j = 0; j < 8; ++j) y[j] = (__bf16)(acc[j] * inv);
    o_out[row * G + v] = __builtin_bit_cast(uint4, y);
    if (v == 0 && lse_out) lse_out[row] = (M == -INFINITY) ? -INFINITY : M + logf(D);
}

}  // namespace

hipError_t launch_merge(const void* o_cat, const float* lse_cat, const int32_t* merge_src,
                        int32_t P, int64_t T_glob, int32_t H, int32_t D_v, int64_t R_total,
                        const float* sink, void* o_out, float* lse_out, hipStream_t stream) {
    const int G = D_v / 8;
    const int64_t n_rows = T_glob * H;
    const int64_t blocks = (n_rows * G + 255) / 256;
    hipLaunchKernelGGL(merge_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, (const uint4*)o_cat,
                       lse_cat, merge_src, P, n_rows, H, G, R_total, sink, (uint4*)o_out, lse_out);
    return hipGetLastError();
}

}  // namespace mla
