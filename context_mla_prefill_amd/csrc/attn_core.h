// Shared pieces of the MLA partial-attention kernels: fragment types, the 64-row workgroup
// shape of the four-wave dense kernel, the direct-to-LDS loads, the key-row permutation of an
// LDS tile and the score-key layout of the transposed Q K^T MFMA, and the key mask.
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

}  // namespace attn
}  // namespace mla
