// Per-wave tile compute of the "wide" attention kernels, in which every wave owns 32 query rows
// outright: their Q^T operand fragments stay in VGPRs, their whole 512-column output O^T in
// AGPRs, and the softmax of a row never leaves the wave (absorbed MLA as multi-query attention,
// latent rows as values: "[Core] Add MRV2 virtual-batch PCP for MLA", "DualChunkSwap
// partitioning"; partial O and LSE for the merge: "[DeepSeekV4][PCP] Enable context-parallel
// prefill for hybrid KV and MegaMoE", "Purpose").
//
// Softmax against a fixed per-row reference: a row's reference is the max of its first tile with
// a visible key; later probabilities 2^(s - ref) are taken against it as long as every later
// score stays within 2^kRefSlack of it, so O is never rescaled. A kernel tracks each row's exact
// max as well and redoes its pass against it when some row passes the slack.
#pragma once

#include "attn_core.h"

namespace mla {
namespace wide {

using attn::bf16x8;
using attn::f32x16;

constexpr float kRefSlack = 32.0f;  // log2 headroom of the fixed reference
constexpr int NBO = 16;             // 32-column blocks of a 512-wide O row

// O lives in AGPRs and is written by P V MFMAs issued as inline asm, which the compiler's hazard
// tracking does not see as MFMAs. The one place where ordinary instructions read O (the
// epilogue) first waits out the last MFMA's write latency; the asm statement takes O as operands
// so it stays ordered after the MFMAs.
#define MLA_O_OPERANDS(o)                                                                                   \
    "+a"(o[0]), "+a"(o[1]), "+a"(o[2]), "+a"(o[3]), "+a"(o[4]), "+a"(o[5]), "+a"(o[6]), "+a"(o[7]),         \
        "+a"(o[8]), "+a"(o[9]), "+a"(o[10]), "+a"(o[11]), "+a"(o[12]), "+a"(o[13]), "+a"(o[14]), "+a"(o[15])
__device__ __forceinline__ void o_read_fence(f32x16 (&o)[NBO]) {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : MLA_O_OPERANDS(o));
}

// Zeroes an O block where it lives (an MFMA of zero operands with a zero accumulator writes zeros
// to its 16 AGPRs), so every value of O is defined in AGPRs and the compiler never moves O
// through VGPRs.
__device__ __forceinline__ void o_zero(f32x16& o) {
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %1, 0" : "=a"(o) : "v"(bf16x8{}));
}

// P is written by VALU instructions and read by the P V MFMAs issued as asm, whose operands the
// compiler's hazard tracking does not see: two wait states between them.
__device__ __forceinline__ void p_fence(bf16x8 (&p)[2]) { asm volatile("s_nop 2" : "+v"(p[0]), "+v"(p[1])); }

// O^T[32 columns of one block] += V^T P^T for one 16-key half of a 32-key tile.
__device__ __forceinline__ void pv_mfma(f32x16& o, const bf16x8& v, const bf16x8& p) {
    asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(o) : "v"(v), "v"(p));
}

// Softmax of one 32-key tile for this lane's row (16 scores per lane, the other 16 of the row in
// the lane 32 away), in pieces a kernel can interleave with MFMAs: pieces 0-8 the row max, the
// reference (set by the first tile with a visible key) and whether the max passed the
// reference's slack; 9-24 the probabilities against the reference (rounded to bf16, in
// pk[0] for scores 0-7 and pk[1] for 8-15) and their sum.
struct Softmax {
    float a[8], mloc, mn, mu, x[16], l;
    bool over;
    __device__ __forceinline__ void piece(int k, const f32x16& s, float m_ref, float scale_log2, bf16x8 (&pk)[2]) {
        if (k < 4) {
            a[2 * k] = fmaxf(s[4 * k], s[4 * k + 1]);
            a[2 * k + 1] = fmaxf(s[4 * k + 2], s[4 * k + 3]);
        } else if (k == 4) {
            a[0] = fmaxf(a[0], a[1]);
            a[2] = fmaxf(a[2], a[3]);
        } else if (k == 5) {
            a[4] = fmaxf(a[4], a[5]);
            a[6] = fmaxf(a[6], a[7]);
        } else if (k == 6) {
            a[0] = fmaxf(fmaxf(a[0], a[2]), fmaxf(a[4], a[6]));
        } else if (k == 7) {
            a[0] = fmaxf(a[0], attn::half_swap(a[0]));
        } else if (k == 8) {
            mloc = a[0] * scale_log2;
            mn = m_ref == -INFINITY ? mloc : m_ref;
            over = mloc > mn + kRefSlack;
            mu = mn == -INFINITY ? 0.0f : mn;
            l = 0.0f;
        } else if (k < 17) {
            const int j = k - 9;  // scores 2j, 2j+1
            x[2 * j] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[2 * j], scale_log2, -mu));
            x[2 * j + 1] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[2 * j + 1], scale_log2, -mu));
        } else if (k < 25) {
            const int j = k - 17;
            pk[j >> 2][2 * (j & 3)] = (__bf16)x[2 * j];
            pk[j >> 2][2 * (j & 3) + 1] = (__bf16)x[2 * j + 1];
            l += x[2 * j] + x[2 * j + 1];
        }
    }
};
constexpr int SOFTMAX_PIECES = 25;

}  // namespace wide
}  // namespace mla
