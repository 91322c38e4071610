// Slot-mapped latent-KV insert: the one-GPU stand-in for the latent-KV all-gather
// ("[Core] Add MRV2 virtual-batch PCP for MLA", "DualChunkSwap partitioning": the
// latent KV is all-gathered so every rank holds the full KV for cache insertion and
// attention). Each local row is copied byte for byte to its packed-KV slot.
//
// One thread moves one 16-byte vector; a row's latent and rope vectors are handled by
// consecutive threads so global reads and writes stay coalesced.
#include "internal.h"

namespace mla {
namespace {

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

}  // namespace

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
