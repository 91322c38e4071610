// C entry points: host-side validation, then one or two kernel launches on the caller's
// stream. Nothing here allocates device memory or synchronises.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "internal.h"

namespace mla {

static thread_local char g_err[512] = "";

mla_status fail(mla_status s, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return s;
}

mla_status check_launch(const char* what) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(MLA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return MLA_OK;
}

static bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace mla

using namespace mla;

extern "C" {

int mla_pcp_abi_version(void) { return MLA_PCP_ABI_VERSION; }

const char* mla_pcp_last_error(void) { return g_err; }

mla_status pcp_plan_sizes(const int32_t* q_lens, const int32_t* kv_lens, int32_t n_req, int32_t P,
                          int32_t* T_loc, int32_t* n_vrows, int64_t* T_glob) {
    if (n_req < 0) return fail(MLA_ERR_INVALID_ARG, "pcp_plan_sizes: n_req=%d < 0", n_req);
    if (P < 1 || P > 64) return fail(MLA_ERR_INVALID_ARG, "pcp_plan_sizes: P=%d outside 1..64", P);
    if ((n_req > 0 && (!q_lens || !kv_lens)) || !T_loc || !n_vrows || !T_glob)
        return fail(MLA_ERR_INVALID_ARG, "pcp_plan_sizes: null pointer");
    int64_t tg = 0, nkv = 0, nv = 0, tot = 0;
    int64_t loc[64] = {0};
    for (int32_t b = 0; b < n_req; ++b) {
        const int64_t q = q_lens[b], kv = kv_lens[b];
        if (q < 0 || kv < 0 || q > kv)
            return fail(MLA_ERR_INVALID_ARG, "pcp_plan_sizes: request %d has q_len=%lld kv_len=%lld",
                        b, (long long)q, (long long)kv);
        tg += q;
        nkv += kv;
        if (q >= 2 * (int64_t)P) {
            // rank r holds chunks r and 2P-1-r of the array_split sizes
            const int64_t n = 2 * (int64_t)P, base = q / n, extra = q % n;
            for (int r = 0; r < P; ++r) {
                const int64_t c1 = r, c2 = n - 1 - r;
                loc[r] += base + (c1 < extra) + base + (c2 < extra);
            }
            nv += 2;
        } else {
            for (int r = 0; r < P; ++r) loc[r] += q;
            nv += 1;
        }
    }
    for (int r = 0; r < P; ++r) tot += loc[r];
    if (nkv > INT32_MAX || tot > INT32_MAX || tg > INT32_MAX || nv > INT32_MAX)
        return fail(MLA_ERR_INVALID_ARG, "pcp_plan_sizes: totals exceed int32 (kv=%lld rows=%lld)",
                    (long long)nkv, (long long)tot);
    for (int r = 0; r < P; ++r) T_loc[r] = (int32_t)loc[r];
    *n_vrows = (int32_t)nv;
    *T_glob = tg;
    return MLA_OK;
}

mla_status pcp_partition(const int32_t* q_lens, const int32_t* kv_lens, const int32_t* kv_start,
                         int32_t n_req, int32_t P, int64_t T_glob, int32_t n_vrows,
                         int64_t T_loc_total, const int32_t* block_table, int32_t bt_stride,
                         int32_t* cu_seqlens_glob, int32_t* cu_seqlens_q,
                         int32_t* vrow_req, int32_t* vrow_kv_start, int32_t* vrow_kv_len,
                         int32_t* local_gidx, int32_t* positions, int32_t* slot,
                         int32_t* merge_src, void* stream) {
    if (n_req < 0 || P < 1 || P > 64 || T_glob < 0 || T_glob > INT32_MAX || n_vrows < 0 ||
        T_loc_total < 0 || T_loc_total > INT32_MAX)
        return fail(MLA_ERR_INVALID_ARG, "pcp_partition: sizes out of range (n_req=%d P=%d)", n_req, P);
    if (n_vrows < n_req || n_vrows > 2 * (int64_t)n_req)
        return fail(MLA_ERR_INVALID_ARG, "pcp_partition: n_vrows=%d inconsistent with n_req=%d",
                    n_vrows, n_req);
    if (!cu_seqlens_glob || !cu_seqlens_q)
        return fail(MLA_ERR_INVALID_ARG, "pcp_partition: null output pointer");
    if (n_req > 0 && (!q_lens || !kv_lens || !kv_start || !vrow_req || !vrow_kv_start || !vrow_kv_len))
        return fail(MLA_ERR_INVALID_ARG, "pcp_partition: null pointer");
    if (T_loc_total > 0 && (!local_gidx || !positions || !slot))
        return fail(MLA_ERR_INVALID_ARG, "pcp_partition: null per-row output");
    if (T_glob > 0 && !merge_src) return fail(MLA_ERR_INVALID_ARG, "pcp_partition: null merge_src");
    if (block_table && bt_stride < 1) return fail(MLA_ERR_INVALID_ARG, "pcp_partition: bt_stride < 1");
    hipError_t e = launch_partition(q_lens, kv_lens, kv_start, n_req, P, T_glob, n_vrows, T_loc_total,
                                    block_table, bt_stride, cu_seqlens_glob, cu_seqlens_q, vrow_req, vrow_kv_start, vrow_kv_len,
                                    local_gidx, positions, slot, merge_src, (hipStream_t)stream);
    if (e != hipSuccess) return fail(MLA_ERR_HIP, "pcp_partition: %s", hipGetErrorString(e));
    return MLA_OK;
}

mla_status pcp_kv_insert(const void* local_latent, const void* local_rope, const int32_t* slot,
                         int32_t T_loc, int32_t D_latent, int32_t D_rope, int32_t kv_dtype,
                         int64_t N_kv, void* kv_latent, void* kv_rope, void* stream) {
    if (T_loc < 0 || N_kv < 0) return fail(MLA_ERR_INVALID_ARG, "pcp_kv_insert: negative size");
    if (!(D_latent == 512 || D_latent == 64) || !(D_rope == 64 || D_rope == 16))
        return fail(MLA_ERR_UNSUPPORTED, "pcp_kv_insert: dims %d+%d unsupported", D_latent, D_rope);
    if (kv_dtype != MLA_KV_BF16 && kv_dtype != MLA_KV_FP8_E4M3)
        return fail(MLA_ERR_UNSUPPORTED, "pcp_kv_insert: kv_dtype %d", kv_dtype);
    if (T_loc == 0) return MLA_OK;
    if (!local_latent || !local_rope || !slot || !kv_latent || !kv_rope)
        return fail(MLA_ERR_INVALID_ARG, "pcp_kv_insert: null pointer");
    if (!aligned16(local_latent) || !aligned16(local_rope) || !aligned16(kv_latent) || !aligned16(kv_rope))
        return fail(MLA_ERR_INVALID_ARG, "pcp_kv_insert: buffers must be 16-byte aligned");
    const int32_t lb = D_latent * (kv_dtype == MLA_KV_BF16 ? 2 : 1), rb = D_rope * 2;
    hipError_t e = launch_kv_insert(local_latent, local_rope, slot, T_loc, lb, rb, N_kv, kv_latent,
                                    kv_rope, (hipStream_t)stream);
    if (e != hipSuccess) return fail(MLA_ERR_HIP, "pcp_kv_insert: %s", hipGetErrorString(e));
    return MLA_OK;
}

mla_status pcp_kv_insert_fp8(const void* local_latent, const void* local_rope, const int32_t* slot,
                             int32_t T, int32_t D_latent, int32_t D_rope, int64_t N_kv, void* kv_latent,
                             void* kv_rope, float* kv_scale, void* stream) {
    if (T < 0 || N_kv < 0 || N_kv > INT32_MAX) return fail(MLA_ERR_INVALID_ARG, "pcp_kv_insert_fp8: sizes out of range");
    if (!((D_latent == 512 && D_rope == 64) || (D_latent == 64 && D_rope == 16)))
        return fail(MLA_ERR_UNSUPPORTED, "pcp_kv_insert_fp8: dims %d+%d unsupported", D_latent, D_rope);
    if (T == 0) return MLA_OK;
    if (!local_latent || !local_rope || !slot || !kv_latent || !kv_rope || !kv_scale)
        return fail(MLA_ERR_INVALID_ARG, "pcp_kv_insert_fp8: null pointer");
    if (!aligned16(local_latent) || !aligned16(local_rope) || !aligned16(kv_latent) || !aligned16(kv_rope))
        return fail(MLA_ERR_INVALID_ARG, "pcp_kv_insert_fp8: buffers must be 16-byte aligned");
    hipError_t e = launch_kv_insert_fp8(local_latent, local_rope, slot, T, D_latent, D_rope, N_kv, kv_latent, kv_rope,
                                        kv_scale, (hipStream_t)stream);
    if (e != hipSuccess) return fail(MLA_ERR_HIP, "pcp_kv_insert_fp8: %s", hipGetErrorString(e));
    return MLA_OK;
}

mla_status sparse_topk_select(const float* scores, int64_t ld, const int32_t* positions, int32_t T, int32_t k,
                              int32_t* topk_idx, void* stream) {
    if (T < 0 || ld < 1 || ld % 4 != 0)
        return fail(MLA_ERR_INVALID_ARG, "sparse_topk_select: sizes out of range (T=%d, ld=%lld; ld %% 4 == 0)", T,
                    (long long)ld);
    if (k < 1 || k > 2048) return fail(MLA_ERR_UNSUPPORTED, "sparse_topk_select: k=%d outside 1..2048", k);
    if (T == 0) return MLA_OK;
    if (!scores || !positions || !topk_idx) return fail(MLA_ERR_INVALID_ARG, "sparse_topk_select: null pointer");
    if (!aligned16(scores)) return fail(MLA_ERR_INVALID_ARG, "sparse_topk_select: scores must be 16-byte aligned");
    hipError_t e = launch_topk_select(scores, ld, positions, T, k, topk_idx, (hipStream_t)stream);
    if (e != hipSuccess) return fail(MLA_ERR_HIP, "sparse_topk_select: %s", hipGetErrorString(e));
    return MLA_OK;
}

mla_status pcp_kv_dequant_fp8(const void* kv_latent, const float* kv_scale, int64_t N_kv, int32_t D_latent,
                              const int32_t* blocks, int32_t n_blocks, void* ws, void* stream) {
    if (N_kv < 0 || N_kv > INT32_MAX || n_blocks < 0)
        return fail(MLA_ERR_INVALID_ARG, "pcp_kv_dequant_fp8: sizes out of range");
    if (D_latent != 512 && D_latent != 64)
        return fail(MLA_ERR_UNSUPPORTED, "pcp_kv_dequant_fp8: D_latent=%d unsupported (512, 64)", D_latent);
    if (n_blocks == 0 || N_kv == 0) return MLA_OK;
    if (!kv_latent || !kv_scale || !blocks || !ws) return fail(MLA_ERR_INVALID_ARG, "pcp_kv_dequant_fp8: null pointer");
    if (!aligned16(kv_latent) || !aligned16(ws))
        return fail(MLA_ERR_INVALID_ARG, "pcp_kv_dequant_fp8: buffers must be 16-byte aligned");
    hipError_t e = launch_kv_dequant_fp8(kv_latent, kv_scale, N_kv, D_latent, blocks, n_blocks, ws,
                                         (hipStream_t)stream);
    if (e != hipSuccess) return fail(MLA_ERR_HIP, "pcp_kv_dequant_fp8: %s", hipGetErrorString(e));
    return MLA_OK;
}

// The sparse kernels address KV rows through 32-bit buffer offsets: N_kv * 512 < 2^32 for
// fp8 rows, N_kv * 1024 < 2^32 for bf16 rows.
constexpr int64_t kSparseMaxKv = (int64_t(1) << 23) - 1;
constexpr int64_t kSparseMaxKvBf16 = (int64_t(1) << 22) - 1;

mla_status mla_prefill_partial(const mla_partial_args* a, void* stream) {
    if (!a) return fail(MLA_ERR_INVALID_ARG, "mla_prefill_partial: null args");
    if (a->T_loc < 0 || a->n_vrows < 0 || a->N_kv < 0 || a->N_kv > INT32_MAX)
        return fail(MLA_ERR_INVALID_ARG, "mla_prefill_partial: sizes out of range");
    if (a->H < 1 || a->H > 128)
        return fail(MLA_ERR_UNSUPPORTED, "mla_prefill_partial: H=%d outside 1..128", a->H);
    if ((int64_t)a->T_loc * a->H > INT32_MAX)
        return fail(MLA_ERR_INVALID_ARG, "mla_prefill_partial: T_loc*H exceeds int32");
    const bool big = a->D_latent == 512 && a->D_rope == 64;
    const bool tiny = a->D_latent == 64 && a->D_rope == 16;
    if (!big && !tiny)
        return fail(MLA_ERR_UNSUPPORTED, "mla_prefill_partial: dims %d+%d unsupported (512+64, 64+16)",
                    a->D_latent, a->D_rope);
    if (a->kv_dtype != MLA_KV_BF16 && a->kv_dtype != MLA_KV_FP8_E4M3)
        return fail(MLA_ERR_UNSUPPORTED, "mla_prefill_partial: kv_dtype %d", a->kv_dtype);
    if (!(a->scale > 0.0f) || a->scale > 1e30f)
        return fail(MLA_ERR_INVALID_ARG, "mla_prefill_partial: scale must be positive and finite");
    const bool sparse = a->topk_idx != nullptr;
    if (sparse) {
        if (a->topk < 0 || a->topk > 2048)
            return fail(MLA_ERR_UNSUPPORTED, "mla_prefill_partial: topk=%d outside 0..2048", a->topk);
        if (a->window < 0 || a->window > 4096)
            return fail(MLA_ERR_UNSUPPORTED, "mla_prefill_partial: window=%d outside 0..4096", a->window);
        if (!big) return fail(MLA_ERR_UNSUPPORTED, "mla_prefill_partial: sparse path needs 512+64 dims");
        const int64_t max_kv = a->kv_dtype == MLA_KV_FP8_E4M3 ? kSparseMaxKv : kSparseMaxKvBf16;
        if (a->N_kv > max_kv)
            return fail(MLA_ERR_UNSUPPORTED, "mla_prefill_partial: sparse path takes at most %d KV rows of this dtype",
                        (int)max_kv);
    } else if (a->kv_dtype != MLA_KV_BF16) {
        return fail(MLA_ERR_UNSUPPORTED, "mla_prefill_partial: dense path takes bf16 KV");
    }
    if (a->kv_splits < 1 || a->kv_splits > 64)
        return fail(MLA_ERR_INVALID_ARG, "mla_prefill_partial: kv_splits=%d outside 1..64", a->kv_splits);
    if (a->kv_splits > 1 && (a->split_stride < a->T_loc || !a->vrow_kv_len ||
                             a->split_stride * (a->kv_splits - 1) + a->T_loc > INT32_MAX / a->H))
        return fail(MLA_ERR_INVALID_ARG, "mla_prefill_partial: split KV needs split_stride >= T_loc, "
                                         "vrow_kv_len and outputs within int32 rows*H");
    if ((((int64_t)a->T_loc * a->H + 63) / 64 + a->n_vrows) * a->kv_splits > INT32_MAX)
        return fail(MLA_ERR_INVALID_ARG, "mla_prefill_partial: too many workgroups");
    if (a->block_table && (!a->vrow_req || a->bt_stride < 1))
        return fail(MLA_ERR_INVALID_ARG, "mla_prefill_partial: block_table needs vrow_req and bt_stride >= 1");
    if (a->block_table && a->N_kv % 64 != 0)
        return fail(MLA_ERR_INVALID_ARG, "mla_prefill_partial: a paged cache holds whole 64-row blocks (N_kv %% 64 != 0)");
    if (a->T_loc == 0) return MLA_OK;
    if (a->N_kv < 1) return fail(MLA_ERR_INVALID_ARG, "mla_prefill_partial: T_loc > 0 with an empty KV cache");
    if (!a->q || !a->latent_kv || !a->rope_k || !a->cu_seqlens_q || !a->vrow_kv_start ||
        !a->positions || !a->o_partial || !a->lse)
        return fail(MLA_ERR_INVALID_ARG, "mla_prefill_partial: null pointer");
    if (a->n_vrows < 1) return fail(MLA_ERR_INVALID_ARG, "mla_prefill_partial: T_loc > 0 with no virtual rows");
    if (a->kv_dtype == MLA_KV_FP8_E4M3 && !a->kv_scale)
        return fail(MLA_ERR_INVALID_ARG, "mla_prefill_partial: fp8 KV needs kv_scale");
    if (!aligned16(a->q) || !aligned16(a->latent_kv) || !aligned16(a->rope_k) || !aligned16(a->o_partial))
        return fail(MLA_ERR_INVALID_ARG, "mla_prefill_partial: q/KV/output must be 16-byte aligned");
    hipError_t e = !sparse ? launch_dense_partial(*a, (hipStream_t)stream)
                   : launch_sparse_wide_partial(*a, (hipStream_t)stream);
    if (e != hipSuccess) return fail(MLA_ERR_HIP, "mla_prefill_partial: %s", hipGetErrorString(e));
    return MLA_OK;
}

mla_status pcp_lse_merge(const void* o_cat, const float* lse_cat, const int32_t* merge_src,
                         int32_t P, int64_t T_glob, int32_t H, int32_t D_v, int64_t R_total,
                         int32_t kv_splits, int64_t split_stride, const float* sink, void* o_out,
                         float* lse_out, void* stream) {
    if (P < 1 || P > 64 || T_glob < 0 || H < 1 || R_total < 0 || T_glob * (int64_t)H > INT32_MAX ||
        R_total * (int64_t)H > INT32_MAX)
        return fail(MLA_ERR_INVALID_ARG, "pcp_lse_merge: sizes out of range (P=%d H=%d)", P, H);
    if (kv_splits < 1 || P * kv_splits > 64 || split_stride < 0)
        return fail(MLA_ERR_INVALID_ARG, "pcp_lse_merge: kv_splits=%d with P=%d (P*kv_splits <= 64)",
                    kv_splits, P);
    if (D_v < 8 || D_v > 1024 || D_v % 8 != 0)
        return fail(MLA_ERR_UNSUPPORTED, "pcp_lse_merge: D_v=%d must be a multiple of 8 in 8..1024", D_v);
    if (H > 128) return fail(MLA_ERR_UNSUPPORTED, "pcp_lse_merge: H=%d above 128", H);
    if (T_glob == 0) return MLA_OK;
    if (!merge_src || !o_out || (R_total > 0 && (!o_cat || !lse_cat)))
        return fail(MLA_ERR_INVALID_ARG, "pcp_lse_merge: null pointer");
    if ((o_cat && !aligned16(o_cat)) || !aligned16(o_out))
        return fail(MLA_ERR_INVALID_ARG, "pcp_lse_merge: O buffers must be 16-byte aligned");
    hipError_t e = launch_merge(o_cat, lse_cat, merge_src, P, T_glob, H, D_v, R_total, kv_splits, split_stride,
                                sink, o_out, lse_out, (hipStream_t)stream);
    if (e != hipSuccess) return fail(MLA_ERR_HIP, "pcp_lse_merge: %s", hipGetErrorString(e));
    return MLA_OK;
}

}  // extern "C"
