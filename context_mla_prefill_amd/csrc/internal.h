// Internal declarations shared by the library's translation units (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mla_pcp.h"

namespace mla {

// Sets the thread-local error message and returns the status.
mla_status fail(mla_status s, const char* fmt, ...);
// Converts the last HIP error after a launch into a status.
mla_status check_launch(const char* what);

// Launchers (arguments already validated by the C entry points).
hipError_t launch_partition(const int32_t* q_lens, const int32_t* kv_lens, const int32_t* kv_start,
                            int32_t n_req, int32_t P, int64_t T_glob, int32_t n_vrows,
                            int64_t T_loc_total, const int32_t* block_table, int32_t bt_stride,
                            int32_t* cu_glob, int32_t* cu_q, int32_t* vrow_req,
                            int32_t* vrow_kv_start, int32_t* vrow_kv_len, int32_t* local_gidx,
                            int32_t* positions, int32_t* slot, int32_t* merge_src,
                            hipStream_t stream);

hipError_t launch_kv_insert(const void* local_latent, const void* local_rope, const int32_t* slot,
                            int32_t T_loc, int32_t latent_bytes, int32_t rope_bytes, int64_t N_kv,
                            void* kv_latent, void* kv_rope, hipStream_t stream);

hipError_t launch_merge(const void* o_cat, const float* lse_cat, const int32_t* merge_src,
                        int32_t P, int64_t T_glob, int32_t H, int32_t D_v, int64_t R_total,
                        int32_t kv_splits, int64_t split_stride, const float* sink, void* o_out,
                        float* lse_out, hipStream_t stream);

hipError_t launch_kv_insert_fp8(const void* local_latent, const void* local_rope, const int32_t* slot,
                                int32_t T, int32_t D_latent, int32_t D_rope, int64_t N_kv, void* kv_latent,
                                void* kv_rope, float* kv_scale, hipStream_t stream);

hipError_t launch_kv_dequant_fp8(const void* kv_latent, const float* kv_scale, int64_t N_kv, int32_t D_latent,
                                 const int32_t* blocks, int32_t n_blocks, void* ws, hipStream_t stream);

hipError_t launch_topk_select(const float* scores, int64_t ld, const int32_t* positions, int32_t T, int32_t k,
                              int32_t* topk_idx, hipStream_t stream);

hipError_t launch_dense_partial(const mla_partial_args& a, hipStream_t stream);
hipError_t launch_dense_wide_partial(const mla_partial_args& a, hipStream_t stream);
hipError_t launch_sparse_wide_partial(const mla_partial_args& a, hipStream_t stream);

}  // namespace mla
