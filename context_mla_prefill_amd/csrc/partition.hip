// DualChunkSwap plan on the GPU.
//
// "[Core] Add MRV2 virtual-batch PCP for MLA", sections "PCP algorithm" and
// "DualChunkSwap partitioning": every prefill is split on its own into 2P contiguous
// chunks and rank r receives chunks r and 2P-1-r; decode rows (and, as read here,
// prefills shorter than 2P) are replicated on every rank. Chunk sizes follow
// numpy.array_split: chunk c holds q/(2P) tokens plus one when c < q mod 2P.
//
// Two kernels:
//  * plan_vrows: one workgroup walks the requests in tiles of 256 and block-scans the
//    per-request counts (tokens, virtual rows, tokens per rank) to fill the global and
//    per-rank cu_seqlens and the virtual-row tables.
//  * plan_tokens: one thread per global token finds its request (binary search), its
//    chunk and rank, and writes its local row(s) and its merge_src row.
#include "internal.h"

namespace mla {
namespace {

constexpr int kScanThreads = 256;
constexpr int kMaxP = 64;

// Sizes of chunk c (and its first token) for q tokens split into n array_split chunks.
__device__ __forceinline__ void chunk_of(int q, int n, int c, int& start, int& size) {
    const int base = q / n, extra = q % n;
    size = base + (c < extra ? 1 : 0);
    start = c * base + (c < extra ? c : extra);
}

// Inclusive block scan of one int per thread (256 threads).
__device__ int block_scan_incl(int v, int* sh) {
    const int t = threadIdx.x;
    sh[t] = v;
    __syncthreads();
    for (int off = 1; off < kScanThreads; off <<= 1) {
        const int add = t >= off ? sh[t - off] : 0;
        __syncthreads();
        sh[t] += add;
        __syncthreads();
    }
    const int r = sh[t];
    __syncthreads();
    return r;
}

__global__ __launch_bounds__(kScanThreads) void plan_vrows(
    const int32_t* __restrict__ q_lens, const int32_t* __restrict__ kv_lens,
    const int32_t* __restrict__ kv_start, int n_req, int P, int n_vrows,
    int32_t* __restrict__ cu_glob, int32_t* __restrict__ cu_q, int32_t* __restrict__ vrow_req,
    int32_t* __restrict__ vrow_kv_start, int32_t* __restrict__ vrow_kv_len) {
    __shared__ int sh[kScanThreads];
    __shared__ int carry[2 + kMaxP];
    const int t = threadIdx.x;
    for (int i = t; i < 2 + P; i += kScanThreads) carry[i] = 0;
    if (t == 0) cu_glob[0] = 0;
    for (int r = t; r < P; r += kScanThreads) cu_q[(int64_t)r * (n_vrows + 1)] = 0;
    __syncthreads();
    const int n_chunks = 2 * P;
    for (int base = 0; base < n_req; base += kScanThreads) {
        const int b = base + t;
        const bool live = b < n_req;
        const int q = live ? q_lens[b] : 0;
        const int kv = live ? kv_lens[b] : 0;
        const int ks = live ? kv_start[b] : 0;
        const bool split = q >= n_chunks;
        const int nv = live ? (split ? 2 : 1) : 0;
        const int p0 = kv - q;
        // global token offsets
        const int q_incl = block_scan_incl(q, sh);
        const int q_excl = carry[0] + q_incl - q;
        // virtual-row index of this request's first virtual row (same on every rank)
        const int nv_incl = block_scan_incl(nv, sh);
        const int v0 = carry[1] + nv_incl - nv;
        if (live) cu_glob[b + 1] = q_excl + q;
        for (int r = 0; r < P; ++r) {
            int cnt = 0, s1 = 0, z1 = 0, s2 = 0, z2 = 0;
            if (live) {
                if (split) {
                    chunk_of(q, n_chunks, r, s1, z1);
                    chunk_of(q, n_chunks, n_chunks - 1 - r, s2, z2);
                    cnt = z1 + z2;
                } else {
                    cnt = q;
                }
            }
            const int c_incl = block_scan_incl(cnt, sh);
            const int off = carry[2 + r] + c_incl - cnt;  // local token offset on rank r
            if (live) {
                int32_t* cq = cu_q + (int64_t)r * (n_vrows + 1);
                const int64_t vr = (int64_t)r * n_vrows;
                if (split) {
                    if (v0 + 1 < n_vrows) {
                        cq[v0 + 1] = off + z1;
                        cq[v0 + 2] = off + z1 + z2;
                        vrow_req[vr + v0] = b;
                        vrow_req[vr + v0 + 1] = b;
                        vrow_kv_start[vr + v0] = ks;
                        vrow_kv_start[vr + v0 + 1] = ks;
                        vrow_kv_len[vr + v0] = p0 + s1 + z1;
                        vrow_kv_len[vr + v0 + 1] = p0 + s2 + z2;
                    }
                } else if (v0 < n_vrows) {
                    cq[v0 + 1] = off + q;
                    vrow_req[vr + v0] = b;
                    vrow_kv_start[vr + v0] = ks;
                    vrow_kv_len[vr + v0] = kv;
                }
            }
            __syncthreads();
            if (t == kScanThreads - 1) carry[2 + r] += c_incl;
            __syncthreads();
        }
        __syncthreads();
        if (t == kScanThreads - 1) {
            carry[0] += q_incl;
            carry[1] += nv_incl;
        }
        __syncthreads();
    }
}

__global__ __launch_bounds__(256) void plan_tokens(
    const int32_t* __restrict__ q_lens, const int32_t* __restrict__ kv_lens,
    const int32_t* __restrict__ kv_start, int n_req, int P, int T_glob, int n_vrows, int T_loc_total,
    const int32_t* __restrict__ block_table, int bt_stride,
    const int32_t* __restrict__ cu_glob, const int32_t* __restrict__ cu_q,
    const int32_t* __restrict__ vrow_req, int32_t* __restrict__ local_gidx,
    int32_t* __restrict__ positions, int32_t* __restrict__ slot, int32_t* __restrict__ merge_src) {
    const int t = blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= T_glob) return;
    // request of token t: last b with cu_glob[b] <= t
    int lo = 0, hi = n_req;  // invariant: cu_glob[lo] <= t < cu_glob[hi]
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (cu_glob[mid] <= t) lo = mid; else hi = mid;
    }
    const int b = lo;
    const int i = t - cu_glob[b];
    const int q = q_lens[b], kv = kv_lens[b];
    const int pos = kv - q + i;
    // KV row of the token: packed after the request's first row, or through its block
    // (64 rows) in the block table
    // (a table column past bt_stride, from a kv_len the table does not cover, reads its last entry)
    const int sl = block_table ? block_table[(int64_t)b * bt_stride + min(pos >> 6, bt_stride - 1)] * 64 + (pos & 63)
                               : kv_start[b] + pos;
    // first virtual row of request b: lower bound of b in rank 0's vrow_req
    int vlo = 0, vhi = n_vrows;
    while (vlo < vhi) {
        const int mid = (vlo + vhi) >> 1;
        if (vrow_req[mid] < b) vlo = mid + 1; else vhi = mid;
    }
    const int v0 = vlo;
    const int n_chunks = 2 * P;
    int owner = 0, owner_v = v0, owner_i = i;
    const bool split = q >= n_chunks;
    if (split) {
        const int base = q / n_chunks, extra = q % n_chunks;
        const int big = base + 1;
        int c, cs;
        if (i < extra * big) {
            c = i / big;
            cs = c * big;
        } else {
            c = extra + (i - extra * big) / base;
            cs = extra * big + (c - extra) * base;
        }
        owner = c < P ? c : n_chunks - 1 - c;
        owner_v = v0 + (c < P ? 0 : 1);
        owner_i = i - cs;
    }
    int row_off = 0;
    for (int r = 0; r < P; ++r) {
        const int32_t* cq = cu_q + (int64_t)r * (n_vrows + 1);
        const bool holds = !split || r == owner;
        int row = -1;
        if (holds && owner_v < n_vrows) {
            row = row_off + cq[owner_v] + owner_i;
            if (row >= 0 && row < T_loc_total) {
                local_gidx[row] = t;
                positions[row] = pos;
                slot[row] = sl;
            } else {
                row = -1;
            }
        }
        const bool contributes = split ? (r == owner) : (r == 0);
        merge_src[(int64_t)t * P + r] = contributes ? row : -1;
        row_off += cq[n_vrows];
    }
}

}  // namespace

hipError_t launch_partition(const int32_t* q_lens, const int32_t* kv_lens, const int32_t* kv_start,
                            int32_t n_req, int32_t P, int64_t T_glob, int32_t n_vrows,
                            int64_t T_loc_total, const int32_t* block_table, int32_t bt_stride,
                            int32_t* cu_glob, int32_t* cu_q, int32_t* vrow_req,
                            int32_t* vrow_kv_start, int32_t* vrow_kv_len, int32_t* local_gidx,
                            int32_t* positions, int32_t* slot, int32_t* merge_src,
                            hipStream_t stream) {
    hipLaunchKernelGGL(plan_vrows, dim3(1), dim3(kScanThreads), 0, stream, q_lens, kv_lens, kv_start,
                       n_req, P, n_vrows, cu_glob, cu_q, vrow_req, vrow_kv_start, vrow_kv_len);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || T_glob == 0) return e;
    const int blocks = (int)((T_glob + 255) / 256);
    hipLaunchKernelGGL(plan_tokens, dim3(blocks), dim3(256), 0, stream, q_lens, kv_lens, kv_start, n_req,
                       P, (int)T_glob, n_vrows, (int)T_loc_total, block_table, bt_stride, cu_glob, cu_q,
                       vrow_req, local_gidx,
                       positions, slot, merge_src);
    return hipGetLastError();
}

}  // namespace mla
