// Slot-mapped latent-KV insert: the one-GPU stand-in for the latent-KV all-gather
// ("[Core] Add MRV2 virtual-batch PCP for MLA", "DualChunkSwap partitioning": the
// latent KV is all-gathered so every rank holds the full KV for cache insertion and
// attention). Each local row is copied byte for byte to its packed-KV slot.
//
// One thread moves one 16-byte vector; a row's latent and rope vectors are handled by
// consecutive threads so global reads and writes stay coalesced.
#include <math.h>

#include "internal.h"

namespace mla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__global__ __launch_bounds__(256) void kv_insert_kernel(
    const uint4* __restrict__ lat_src, const uint4* __restrict__ rope_src,
    const int32_t* __restrict__ slot, int T_loc, int lat_vecs, int rope_vecs, int64_t N_kv,
    uint4* __restrict__ lat_dst, uint4* __restrict__ rope_dst) {
    const int per_row = lat_vecs + rope_vecs;
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= (int64_t)T_loc * per_row) return;
    const int row = (int)(gid / per_row);
    const int v = (int)(gid - (int64_t)row * per_row);
    const int64_t s = slot[row];
    if (s < 0 || s >= N_kv) return;
    if (v < lat_vecs) {
        lat_dst[s * lat_vecs + v] = lat_src[(int64_t)row * lat_vecs + v];
    } else {
        const int u = v - lat_vecs;
        rope_dst[s * rope_vecs + u] = rope_src[(int64_t)row * rope_vecs + u];
    }
}

// ---------------------------------------------------------------------------------------
// Quantise-on-insert into an fp8-e4m3 cache with one fp32 scale per 64-row block
// ("[Feature][PCP] Add DeepSeek-V4.1-Flash support", "vLLM Launch Arguments": fp8 MLA KV
// cache, block size 64). A block is opened by the call that writes its first row: that
// call sets its scale from the rows it writes there; rows written into a block that an
// earlier call opened use the stored scale. Three launches in stream order:
//   1. the scale word of every block opened here is set to "amax 0, pending" (bit 31 marks
//      a word that still holds an amax rather than a scale; scales are positive, bit 31
//      clear);
//   2. one wave per row folds the row's max |x| into its block word with an atomic max
//      when that word is pending (non-negative fp32 bits order like their values);
//   3. one wave per row turns a pending word into the scale, the smallest power of two not
//      below fp32(amax / 448) and not below 2^-126 (1 when amax is 0) -- every row of a
//      block computes the same value, so racing writers agree -- then writes its codes
//      e4m3fn_rne(clamp(x / scale, -448, 448)) and copies its rope row.
// A power-of-two scale costs at most one binade of the code range and makes each decoded
// value code * scale exact in bf16, which the attention kernel converts two codes per
// instruction.
constexpr uint32_t kPending = 0x80000000u;

// Smallest normal power of two >= r, for r >= 0 finite (2^-126 for r below it).
__device__ __forceinline__ float pow2_at_least(float r) {
    uint32_t b = __float_as_uint(r);
    if (b < 0x00800000u) return __uint_as_float(0x00800000u);
    if (b & 0x007FFFFFu) b = (b & 0x7F800000u) + 0x00800000u;
    return __uint_as_float(b);
}

__global__ __launch_bounds__(256) void fp8_block_reset(const int32_t* __restrict__ slot, int T, int64_t N_kv,
                                                       uint32_t* __restrict__ scale_word) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= T) return;
    const int64_t s = slot[i];
    if (s >= 0 && s < N_kv && (s & 63) == 0) scale_word[s >> 6] = kPending;
}

template <int DL>
__global__ __launch_bounds__(256) void fp8_block_amax(const __bf16* __restrict__ lat, const int32_t* __restrict__ slot,
                                                      int T, int64_t N_kv, uint32_t* __restrict__ scale_word) {
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= T) return;  // wave-uniform
    const int64_t s = slot[row];
    if (s < 0 || s >= N_kv) return;
    float a = 0.0f;
    for (int e = 8 * lane; e < DL; e += 512) {  // 8 elements (16 bytes) per lane
        const bf16x8 x = *reinterpret_cast<const bf16x8*>(lat + (int64_t)row * DL + e);
#pragma unroll
        for (int k = 0; k < 8; ++k) a = fmaxf(a, fabsf((float)x[k]));
    }
    for (int off = 32; off >= 1; off >>= 1) a = fmaxf(a, __shfl_xor(a, off));
    // pending-ness is fixed for the whole launch: set by the previous one, cleared by the next
    if (lane == 0 && (scale_word[s >> 6] & kPending)) atomicMax(scale_word + (s >> 6), kPending | __float_as_uint(a));
}

template <int DL, int DR>
__global__ __launch_bounds__(256) void fp8_quantize_rows(const __bf16* __restrict__ lat, const __bf16* __restrict__ rope,
                                                         const int32_t* __restrict__ slot, int T, int64_t N_kv,
                                                         uint8_t* __restrict__ lat_dst, __bf16* __restrict__ rope_dst,
                                                         uint32_t* __restrict__ scale_word) {
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= T) return;  // wave-uniform
    const int64_t s = slot[row];
    if (s < 0 || s >= N_kv) return;
    const uint32_t w = scale_word[s >> 6];
    float sc;
    if (w & kPending) {
        const float a = __uint_as_float(w & ~kPending);
        sc = a > 0.0f ? pow2_at_least(__fdiv_rn(a, 448.0f)) : 1.0f;
        if (lane == 0) scale_word[s >> 6] = __float_as_uint(sc);
    } else {
        sc = __uint_as_float(w);
    }
    for (int e = 8 * lane; e < DL; e += 512) {  // 8 elements in, 8 codes out per lane
        const bf16x8 x = *reinterpret_cast<const bf16x8*>(lat + (int64_t)row * DL + e);
        float y[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) y[k] = fminf(fmaxf(__fdiv_rn((float)x[k], sc), -448.0f), 448.0f);
        // OCP E4M3FN codes, round to nearest even; bytes k of the word are elements k
        int lo = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
        lo = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], lo, true);
        int hi = __builtin_amdgcn_cvt_pk_fp8_f32(y[4], y[5], 0, false);
        hi = __builtin_amdgcn_cvt_pk_fp8_f32(y[6], y[7], hi, true);
        *reinterpret_cast<uint2*>(lat_dst + s * DL + e) = make_uint2((uint32_t)lo, (uint32_t)hi);
    }
    for (int e = lane; e < DR; e += 64) rope_dst[s * DR + e] = rope[(int64_t)row * DR + e];
}

template <int DL, int DR>
hipError_t launch_fp8_insert(const void* local_latent, const void* local_rope, const int32_t* slot, int32_t T,
                             int64_t N_kv, void* kv_latent, void* kv_rope, float* kv_scale, hipStream_t stream) {
    uint32_t* words = reinterpret_cast<uint32_t*>(kv_scale);
    hipLaunchKernelGGL(fp8_block_reset, dim3((unsigned)((T + 255) / 256)), dim3(256), 0, stream, slot, T, N_kv, words);
    hipLaunchKernelGGL((fp8_block_amax<DL>), dim3((unsigned)((T + 3) / 4)), dim3(256), 0, stream,
                       (const __bf16*)local_latent, slot, T, N_kv, words);
    hipLaunchKernelGGL((fp8_quantize_rows<DL, DR>), dim3((unsigned)((T + 3) / 4)), dim3(256), 0, stream,
                       (const __bf16*)local_latent, (const __bf16*)local_rope, slot, T, N_kv, (uint8_t*)kv_latent,
                       (__bf16*)kv_rope, words);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------------------
// Dequantise listed 64-row blocks of an fp8-e4m3 latent cache into a bf16 workspace with the
// cache's row addressing: ws[r] = bf16_rne(fp32(e4m3(code[r])) * scale[r / 64]), the same
// arithmetic (and instructions) as the sparse kernel's in-tile dequantisation. One workgroup
// per block; a thread turns 16 codes (16 bytes) into 16 bf16 values (32 bytes) per step.
typedef float f32x2 __attribute__((ext_vector_type(2)));

template <int DL>
__global__ __launch_bounds__(256) void fp8_dequant_blocks(const uint8_t* __restrict__ codes,
                                                          const float* __restrict__ scale,
                                                          const int32_t* __restrict__ blocks, int64_t N_kv,
                                                          __bf16* __restrict__ ws) {
    const int64_t blk = blocks[blockIdx.x];
    if (blk < 0 || blk * 64 >= N_kv) return;  // workgroup-uniform
    const float sc = scale[blk];
    constexpr int CH = DL / 16;  // 16-byte chunks per row
    for (int k = threadIdx.x; k < 64 * CH; k += 256) {
        const int64_t r = blk * 64 + k / CH;
        if (r >= N_kv) break;  // rows past the cache end: the rest of this thread's chunks too
        const int c = k % CH;
        const uint4 raw = *reinterpret_cast<const uint4*>(codes + r * DL + c * 16);
        const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
        bf16x8 o[2];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8(w[q], false);
            const f32x2 b = __builtin_amdgcn_cvt_pk_f32_fp8(w[q], true);
            o[q >> 1][4 * (q & 1) + 0] = (__bf16)(a.x * sc);
            o[q >> 1][4 * (q & 1) + 1] = (__bf16)(a.y * sc);
            o[q >> 1][4 * (q & 1) + 2] = (__bf16)(b.x * sc);
            o[q >> 1][4 * (q & 1) + 3] = (__bf16)(b.y * sc);
        }
        bf16x8* dst = reinterpret_cast<bf16x8*>(ws + r * DL + c * 16);
        dst[0] = o[0];
        dst[1] = o[1];
    }
}

}  // namespace

hipError_t launch_kv_dequant_fp8(const void* kv_latent, const float* kv_scale, int64_t N_kv, int32_t D_latent,
                                 const int32_t* blocks, int32_t n_blocks, void* ws, hipStream_t stream) {
    if (D_latent == 512)
        hipLaunchKernelGGL((fp8_dequant_blocks<512>), dim3((unsigned)n_blocks), dim3(256), 0, stream,
                           (const uint8_t*)kv_latent, kv_scale, blocks, N_kv, (__bf16*)ws);
    else
        hipLaunchKernelGGL((fp8_dequant_blocks<64>), dim3((unsigned)n_blocks), dim3(256), 0, stream,
                           (const uint8_t*)kv_latent, kv_scale, blocks, N_kv, (__bf16*)ws);
    return hipGetLastError();
}

hipError_t launch_kv_insert_fp8(const void* local_latent, const void* local_rope, const int32_t* slot, int32_t T,
                                int32_t D_latent, int32_t D_rope, int64_t N_kv, void* kv_latent, void* kv_rope,
                                float* kv_scale, hipStream_t stream) {
    if (D_latent == 512)
        return launch_fp8_insert<512, 64>(local_latent, local_rope, slot, T, N_kv, kv_latent, kv_rope, kv_scale, stream);
    return launch_fp8_insert<64, 16>(local_latent, local_rope, slot, T, N_kv, kv_latent, kv_rope, kv_scale, stream);
}

hipError_t launch_kv_insert(const void* local_latent, const void* local_rope, const int32_t* slot,
                            int32_t T_loc, int32_t latent_bytes, int32_t rope_bytes, int64_t N_kv,
                            void* kv_latent, void* kv_rope, hipStream_t stream) {
    const int lv = latent_bytes / 16, rv = rope_bytes / 16;
    const int64_t total = (int64_t)T_loc * (lv + rv);
    const int64_t blocks = (total + 255) / 256;
    hipLaunchKernelGGL(kv_insert_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       (const uint4*)local_latent, (const uint4*)local_rope, slot, T_loc, lv, rv, N_kv,
                       (uint4*)kv_latent, (uint4*)kv_rope);
    return hipGetLastError();
}

}  // namespace mla
