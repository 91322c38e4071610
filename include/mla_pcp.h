/*
 * mla_pcp.h — C ABI of the MI355X (gfx950) library for prefill-context-parallel (PCP)
 * MLA prefill attention: DualChunkSwap partition, all-gather stand-in KV insert,
 * rank-local causal (or top-k sparse) partial attention, and the log-sum-exp merge
 * that applies the per-head attention sink once.
 *
 * Conventions for every call below
 *  - Plain pointers and sizes only. "device" pointers are HIP device memory (or
 *    managed memory visible to the GPU); "host" pointers are ordinary host memory.
 *  - Every buffer is owned by the caller. No call allocates, frees or retains memory;
 *    the only library state is a thread-local error string.
 *  - Calls that take `stream` (a hipStream_t; NULL = the null stream) only enqueue
 *    work and return without synchronising. Inputs must stay unchanged until the
 *    stream reaches the work.
 *  - Layouts are row-major and contiguous; integer indices are int32; bf16 is the
 *    IEEE binary32 top half; fp8 is OCP E4M3FN.
 *  - Arguments are validated on the host before any launch. On a non-OK status
 *    nothing was enqueued (except MLA_ERR_HIP, which reports a failed launch) and
 *    mla_pcp_last_error() describes the problem. No call aborts or throws.
 *  - Kernels bound their memory accesses by the sizes passed in. The device index arrays
 *    one call passes to the next (cu_seqlens, vrow_* arrays, positions, local_gidx,
 *    merge_src as pcp_partition writes them) must be consistent with those sizes; within
 *    that, device data that breaks a stated precondition (selected indices out of range,
 *    slots outside [0, N_kv), block-table entries that name no block of the cache, NaN
 *    scores) gives wrong values, never an out-of-bounds access.
 */
#ifndef MLA_PCP_H
#define MLA_PCP_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MLA_PCP_ABI_VERSION 6

typedef enum mla_status {
    MLA_OK = 0,
    MLA_ERR_INVALID_ARG = 1, /* null pointer, bad or inconsistent size, misalignment */
    MLA_ERR_UNSUPPORTED = 2, /* valid request outside what the kernels implement     */
    MLA_ERR_HIP = 3          /* the HIP runtime reported an error                    */
} mla_status;

/* KV element types */
#define MLA_KV_BF16 0
#define MLA_KV_FP8_E4M3 1 /* latent only; rope stays bf16; one fp32 scale per 64 rows */

/* Library ABI version (MLA_PCP_ABI_VERSION of the build). */
int mla_pcp_abi_version(void);

/* Message for the last non-OK status returned on the calling thread ("" if none). */
const char* mla_pcp_last_error(void);

/*
 * pcp_plan_sizes — host-only sizing of a DualChunkSwap plan.
 * Source: "[Core] Add MRV2 virtual-batch PCP for MLA", "PCP algorithm" and
 * "DualChunkSwap partitioning": each prefill is split on its own into 2*P chunks and
 * rank r receives chunks r and 2P-1-r; decode rows are replicated on every rank.
 * A request with q_len < 2P (decode rows, short prefills) is replicated; otherwise it
 * is split with numpy.array_split chunk sizes.
 *
 *  q_lens, kv_lens  host int32 [n_req]: new tokens and total KV rows (new included)
 *                   per request, in batch order; 0 <= q_len <= kv_len.
 *  P                PCP size, 1 <= P <= 64.
 *  T_loc            host out int32 [P]: local rows of each rank.
 *  n_vrows          host out: virtual rows per rank (equal on every rank: 2 per split
 *                   request, 1 per replicated request).
 *  T_glob           host out: sum of q_lens.
 * Errors: INVALID_ARG for null pointers, n_req < 0, P out of range, q_len > kv_len,
 * negative lengths, or totals (sum kv_lens, sum of T_loc) that do not fit int32.
 */
mla_status pcp_plan_sizes(const int32_t* q_lens, const int32_t* kv_lens, int32_t n_req,
                          int32_t P, int32_t* T_loc, int32_t* n_vrows, int64_t* T_glob);

/*
 * pcp_partition — the DualChunkSwap plan on the GPU (integer work, deterministic).
 * Source: as pcp_plan_sizes; the merge map restores global scheduled-token order
 * ("DualChunkSwap partitioning", last paragraph).
 *
 * Inputs (device int32 [n_req]): q_lens, kv_lens, kv_start (first packed KV row of
 * each request). Sizes T_glob, n_vrows, T_loc_total (= sum of T_loc) must be the ones
 * pcp_plan_sizes returned for the same lengths.
 * Paged KV (block_table != NULL): the cache is a pool of 64-row blocks and request b's
 * key at position j lives in row block_table[b * bt_stride + j / 64] * 64 + j % 64
 * ("[Feature][PCP] Add DeepSeek-V4.1-Flash support", "vLLM Launch Arguments": KV cache
 * block size 64); block_table is device int32 [n_req][bt_stride] with ceil(kv_len / 64)
 * entries per request. kv_start is then only copied to vrow_kv_start.
 * Outputs (device int32), ranks concatenated in rank order; rank r's rows start at
 * row_off[r] = T_loc[0] + ... + T_loc[r-1]:
 *  cu_seqlens_glob [n_req+1]           global token offsets of the requests.
 *  cu_seqlens_q    [P][n_vrows+1]      per rank, local token offsets of its virtual
 *                                      rows (each rank starts at 0).
 *  vrow_req        [P][n_vrows]        request of each virtual row.
 *  vrow_kv_start   [P][n_vrows]        kv_start of that request.
 *  vrow_kv_len     [P][n_vrows]        last position of the virtual row + 1.
 *  local_gidx      [T_loc_total]       global token of each local row.
 *  positions       [T_loc_total]       kv_len - q_len + (index of the token among the
 *                                      request's new tokens).
 *  slot            [T_loc_total]       KV row of the token: kv_start + position, or its
 *                                      row through the block table.
 *  merge_src       [T_glob][P]         row (in the rank-concatenated buffers) that rank
 *                                      p contributes to global token t, else -1. Split
 *                                      tokens have one entry (their rank); replicated
 *                                      tokens only rank 0's row.
 * Rank-local order: requests in batch order; a split request gives chunk r then chunk
 * 2P-1-r (two virtual rows); a replicated request one virtual row.
 * Errors: INVALID_ARG for null pointers or sizes out of range; HIP on launch failure.
 */
mla_status pcp_partition(const int32_t* q_lens, const int32_t* kv_lens, const int32_t* kv_start,
                         int32_t n_req, int32_t P, int64_t T_glob, int32_t n_vrows,
                         int64_t T_loc_total, const int32_t* block_table, int32_t bt_stride,
                         int32_t* cu_seqlens_glob, int32_t* cu_seqlens_q,
                         int32_t* vrow_req, int32_t* vrow_kv_start, int32_t* vrow_kv_len,
                         int32_t* local_gidx, int32_t* positions, int32_t* slot,
                         int32_t* merge_src, void* stream);

/*
 * pcp_kv_insert — write a rank's local latent/rope KV rows into the full packed KV at
 * their slots: the single-GPU stand-in for the latent-KV all-gather that gives every
 * rank the full KV for cache insertion and attention ("[Core] Add MRV2 virtual-batch
 * PCP for MLA", "DualChunkSwap partitioning"). A byte copy (bit-exact).
 *
 *  local_latent  device [T_loc][D_latent] bf16, or fp8 codes when kv_dtype is FP8.
 *  local_rope    device [T_loc][D_rope] bf16.
 *  slot          device int32 [T_loc] destination rows; rows outside [0, N_kv) are
 *                skipped.
 *  kv_latent     device [N_kv][D_latent], kv_rope device [N_kv][D_rope] (written).
 * fp8 tile scales are not touched (they are an input of mla_prefill_partial).
 * Errors: INVALID_ARG (null, T_loc < 0, N_kv < 0, 16-byte misalignment);
 * UNSUPPORTED (D_latent not 64/512, D_rope not 16/64, kv_dtype); HIP.
 */
mla_status pcp_kv_insert(const void* local_latent, const void* local_rope, const int32_t* slot,
                         int32_t T_loc, int32_t D_latent, int32_t D_rope, int32_t kv_dtype,
                         int64_t N_kv, void* kv_latent, void* kv_rope, void* stream);

/*
 * pcp_kv_insert_fp8 — write bf16 latent rows into an fp8-e4m3 KV cache at their slots,
 * quantising on insert, and their bf16 rope rows alongside. The cache keeps one fp32
 * scale per 64-row block ("[Feature][PCP] Add DeepSeek-V4.1-Flash support", "vLLM Launch
 * Arguments": fp8 MLA KV cache, block size 64; the scale layout is this library's).
 * A block B is opened by the call that writes its first row (slot % 64 == 0); for it
 *   a = max |x| over the latent elements this call writes into B (as fp32),
 *   kv_scale[B] = the smallest power of two 2^e >= fp32(a / 448) with e >= -126
 *                 (1 when a == 0): a shared power-of-two scale, which makes every decoded
 *                 value code * scale exact in bf16.
 * A block opened by an earlier call keeps its scale (a chunked prefill that continues a
 * block quantises against the scale its first chunk set). Every written element gets
 *   code = e4m3fn_rne(clamp(x / kv_scale[B], -448, 448)) (fp32 division, round to
 *   nearest even, saturating).
 * Writing rows of a block whose first row was never written leaves them against an
 * undefined scale. All-gathered rows go in one call (a block split across two ranks'
 * chunks is then opened once). Calls that run concurrently on one cache race; two rows
 * with the same slot race.
 *  local_latent  device bf16 [T][D_latent]; local_rope device bf16 [T][D_rope].
 *  slot          device int32 [T] destination rows; rows outside [0, N_kv) are skipped.
 *  kv_latent     device uint8 [N_kv][D_latent] (written); kv_rope device bf16 [N_kv][D_rope];
 *  kv_scale      device fp32 [ceil(N_kv / 64)] (the touched blocks' entries written).
 * Errors: INVALID_ARG (null, T < 0, N_kv < 0, 16-byte misalignment); UNSUPPORTED (dims other
 * than 512+64 / 64+16); HIP.
 */
mla_status pcp_kv_insert_fp8(const void* local_latent, const void* local_rope, const int32_t* slot,
                             int32_t T, int32_t D_latent, int32_t D_rope, int64_t N_kv, void* kv_latent,
                             void* kv_rope, float* kv_scale, void* stream);

/*
 * pcp_kv_dequant_fp8 — dequantise listed 64-row blocks of an fp8-e4m3 latent cache into a
 * bf16 workspace with the same row addressing, once per step, for the sparse partial to read
 * bf16 rows (the dequantised-workspace reuse of sparse BF16 CP prefill: "DeepSeek-V4.1: Prefill
 * support CP with multistream forward prepare (4/N)", commit list, "Reuse shared compressed KV
 * dequantization in V4.1 CP prefill").
 * For every listed block B and row r in [64 B, 64 B + 64) with r < N_kv:
 *   ws[r] = bf16_rne(fp32(e4m3(kv_latent[r])) * kv_scale[B])   (bit-identical to the sparse
 *   partial's in-kernel dequantisation).
 *  kv_latent  device uint8 [N_kv][D_latent]; kv_scale device fp32 [ceil(N_kv / 64)];
 *  blocks     device int32 [n_blocks] block ids (ids outside the cache are skipped; a block
 *             listed twice is written twice with the same bytes);
 *  ws         device bf16 [N_kv][D_latent] (rows of unlisted blocks untouched).
 * Errors: INVALID_ARG (null, sizes < 0, N_kv > 2^31 - 1, 16-byte misalignment); UNSUPPORTED
 * (D_latent not 64 / 512); HIP.
 */
mla_status pcp_kv_dequant_fp8(const void* kv_latent, const float* kv_scale, int64_t N_kv, int32_t D_latent,
                              const int32_t* blocks, int32_t n_blocks, void* ws, void* stream);

/*
 * sparse_topk_select — per query row, the k key positions of its causal prefix with the
 * largest index scores: the selected-index input of the sparse partial (the indexer's top-k
 * ahead of sparse MLA, "DeepSeek-V4.1: Prefill support CP with multistream forward prepare
 * (4/N)", "Modifications" and its commit list, "Indexer ... uses topk_v2"). The scores'
 * producer, the indexer, needs trained weights and is not part of this library.
 * Row i has n = min(positions[i] + 1, ld) keys with scores scores[i][0..n):
 *   n <= k: topk_idx[i] = 0, 1, ..., n-1, then -1 pads;
 *   n > k:  the k indices j in [0, n) with the largest scores, equal scores taken by the
 *           smaller index (-0 equals +0), written in increasing order.
 *  scores     device fp32 [T][ld], 16-byte aligned, ld % 4 == 0. NaN is not a score (a row
 *             holding one still gets k distinct in-range indices).
 *  positions  device int32 [T], e.g. the partition's positions of one rank's rows.
 *  topk_idx   device int32 [T][k] (written); with k = mla_partial_args.topk it is that
 *             call's topk_idx.
 * Errors: INVALID_ARG (null, T < 0, ld < 1, ld % 4 != 0, misaligned scores); UNSUPPORTED
 * (k outside 1..2048); HIP.
 */
mla_status sparse_topk_select(const float* scores, int64_t ld, const int32_t* positions, int32_t T, int32_t k,
                              int32_t* topk_idx, void* stream);

/*
 * mla_prefill_partial — one rank's partial MLA attention against the full KV, without
 * the sink. Absorbed MLA: every query head attends one shared latent KV head, key =
 * latent || rope (D_latent + D_rope), value = latent (D_latent). Each PCP rank computes
 * a local partial whose LSE/output are merged later with the sink applied once
 * ("[DeepSeekV4][PCP] Enable context-parallel prefill for hybrid KV and MegaMoE",
 * "Purpose"); the rank attends the full all-gathered latent KV ("[Core] Add MRV2
 * virtual-batch PCP for MLA", "DualChunkSwap partitioning").
 *
 * For local row i (virtual row v, position p = positions[i]) and head h:
 *   dense  (topk_idx == NULL): keys are the request's positions j = 0..p, at KV rows
 *          vrow_kv_start[v] + j, or through block_table as in pcp_partition (request
 *          vrow_req[v]) when block_table != NULL;
 *   sparse (topk_idx != NULL): keys j in {topk_idx[i][*] in [0, p]} union
 *          [max(0, p-window+1), p], counted once (entries -1 or outside [0, p] are
 *          pads; order does not matter).
 *   S_j = scale * <q[i][h], key_j>; O = softmax(S) @ latent (bf16, round to nearest
 *   even); LSE = log(sum_j exp(S_j)) (fp32, natural log). No sink.
 * fp8 latent: element = bf16_rne(fp32(e4m3(code)) * kv_scale[row / 64]) (row = KV row, so
 *   with paging one scale per block), dequantised inside the sparse kernel. Any positive
 *   finite scales are taken; power-of-two scales 2^-117 .. 2^119 (those pcp_kv_insert_fp8
 *   writes) dequantise faster, with the same results. A sparse call with
 *   bf16 latent (for instance the workspace of pcp_kv_dequant_fp8) gathers bf16 rows instead.
 * Split KV (kv_splits = S > 1): the key set of virtual row v is cut by key position into
 *   s_v ranges (s_v = vrow_splits[v], or S for every row when vrow_splits is NULL) and
 *   each range gives its own partial (O, LSE), written at split slice s of the outputs;
 *   merging the slices (pcp_lse_merge with the same S) gives the unsplit result. With
 *   L = vrow_kv_len[v] and n = ceil(L / 64) tiles, range s holds request-relative keys
 *   [64 * floor(s * n / s_v), 64 * floor((s + 1) * n / s_v)), the last one ending at L.
 *   A range with no key of the row gives O = 0, LSE = -inf. Slices s_v .. S-1 of the
 *   row's tokens get LSE = -inf and their O is left as it was (the merge does not read
 *   an output whose weight is zero). The per-rank partial of the "local partial, global
 *   LSE merge" reading ("[DeepSeekV4][PCP] Enable context-parallel prefill for hybrid KV
 *   and MegaMoE", "Purpose") applied to key ranges instead of ranks: long rows, such as
 *   decode rows over a long context, are spread over more workgroups (pcp_plan_splits
 *   picks the per-row counts).
 */
typedef struct mla_partial_args {
    const void* q;               /* device bf16 [T_loc][H][D_latent + D_rope]            */
    const void* latent_kv;       /* device [N_kv][D_latent] bf16, or fp8 codes            */
    const float* kv_scale;       /* device fp32 [ceil(N_kv/64)] (fp8), else NULL          */
    const void* rope_k;          /* device bf16 [N_kv][D_rope]                            */
    const int32_t* cu_seqlens_q; /* device [n_vrows+1] local token offsets (this rank)    */
    const int32_t* vrow_kv_start;/* device [n_vrows] packed KV offset of the row's request */
    const int32_t* positions;    /* device [T_loc] causal position of each local token;
                                    increasing by one inside a virtual row              */
    const int32_t* topk_idx;     /* device [T_loc][topk] request-relative, or NULL       */
    int32_t topk;                /* entries per row of topk_idx (<= 2048), 0 when dense   */
    int32_t window;              /* sliding window added to the sparse set (0 = none)     */
    int32_t n_vrows;
    int32_t T_loc;
    int32_t H;                   /* query heads, 1..128                                    */
    int32_t D_latent;            /* 512 (or 64)                                            */
    int32_t D_rope;              /* 64 (or 16)                                             */
    int32_t kv_dtype;            /* MLA_KV_BF16 or MLA_KV_FP8_E4M3                         */
    int64_t N_kv;                /* rows of latent_kv / rope_k (>= 1 when T_loc > 0; a
                                    multiple of 64 when paged: whole blocks)               */
    float scale;                 /* softmax scale                                          */
    void* o_partial;             /* device bf16 out [T_loc][H][D_latent] (split slice 0)  */
    float* lse;                  /* device fp32 out [T_loc][H] (split slice 0)             */
    int32_t kv_splits;           /* key ranges per row, 1..64 (1 = no split)               */
    int64_t split_stride;        /* rows from one split slice of o_partial / lse to the
                                    next (>= T_loc when kv_splits > 1)                    */
    const int32_t* vrow_kv_len;  /* device [n_vrows] last position of the virtual row + 1,
                                    as pcp_partition writes it (needed when kv_splits > 1) */
    const int32_t* block_table;  /* device [n_req][bt_stride] or NULL (packed KV)          */
    int32_t bt_stride;           /* entries per request row of block_table                 */
    const int32_t* vrow_req;     /* device [n_vrows] request of each virtual row (paged)   */
    const int32_t* vrow_splits;  /* device [n_vrows] key ranges of each virtual row, clamped
                                    into 1..kv_splits, or NULL (every row kv_splits);
                                    ignored when kv_splits == 1                          */
    const int32_t* vrow_order;   /* device [n_vrows] order in which workgroups take the
                                    virtual rows (a permutation; entries are clamped into
                                    [0, n_vrows)), or NULL (last row first). Dense only. */
} mla_partial_args;

/* Errors: INVALID_ARG (null pointers, sizes, 16-byte misalignment, fp8 without scales,
 * kv_splits outside 1..64, split_stride < T_loc or no vrow_kv_len with kv_splits > 1,
 * block_table without vrow_req or with bt_stride < 1, paged N_kv not a multiple of 64,
 * T_loc > 0 with N_kv == 0);
 * UNSUPPORTED (dims other than 512+64 / 64+16, H outside 1..128, topk > 2048, window > 4096,
 * sparse with dims other than 512+64, with fp8 KV of N_kv >= 2^23 rows or bf16 KV of
 * N_kv >= 2^22 rows (32-bit byte offsets), dense with fp8 KV, dtype); HIP.
 * The sparse kernels run one token and a group of up to 64 heads per workgroup, so a head
 * count under 64 (a per-GPU share of the heads under tensor parallelism) leaves the rest of
 * the group's MFMA rows idle: H = 16 or 32 takes the time of H = 64.
 * Sparse preconditions: selected indices of a row are distinct; entries outside [0, p]
 * (including -1) are pads. */
mla_status mla_prefill_partial(const mla_partial_args* args, void* stream);

/*
 * pcp_plan_splits — host-only choice of split KV for the dense partials: the number of key
 * ranges of every virtual row and the order in which the workgroups take the rows, for
 * mla_partial_args.vrow_splits / vrow_order (copied to the device by the caller).
 * Source: the per-rank partials and global LSE merge of "[DeepSeekV4][PCP] Enable
 * context-parallel prefill for hybrid KV and MegaMoE", "Purpose", applied to key ranges, so
 * long rows (decode rows over a long context are replicated on every rank: "[Core] Add MRV2
 * virtual-batch PCP for MLA", "PCP algorithm") are spread over several workgroups.
 * A scheduling heuristic, not part of the method: every (row tile, key range) work item is
 * costed as its key count plus a fixed per-workgroup cost, items are dealt in launch order
 * to n_workers units (each to the first that falls idle), and the plan with the shortest
 * modelled finish time is returned; a plan that splits must beat the unsplit one by 2 %,
 * else every row gets 1 and the default order. Rows never get more than max_splits ranges.
 *
 *  q_lens, kv_lens  host int32 [n_req] as for pcp_plan_sizes; P as there.
 *  H, D_latent      query heads (1..128) and latent width (512 or 64) of the launch.
 *  max_splits       the kv_splits the launch will use (1..64).
 *  n_workers        workgroups resident at once: the GPU's compute units (one dense
 *                   workgroup per unit; 256 on MI355X).
 *  vrow_splits      host out int32 [P][n_vrows]: ranges of each virtual row (1..max_splits).
 *  vrow_order       host out int32 [P][n_vrows]: per rank, a permutation of its rows.
 * Errors: as pcp_plan_sizes; INVALID_ARG (H, max_splits, n_workers, null outputs);
 * UNSUPPORTED (D_latent).
 */
mla_status pcp_plan_splits(const int32_t* q_lens, const int32_t* kv_lens, int32_t n_req, int32_t P,
                           int32_t H, int32_t D_latent, int32_t max_splits, int32_t n_workers,
                           int32_t* vrow_splits, int32_t* vrow_order);

/*
 * pcp_lse_merge — merge per-rank partials into global token order with the sink once.
 * Source: "[DeepSeekV4][PCP] Enable context-parallel prefill for hybrid KV and
 * MegaMoE", "Purpose" and "Main challenges" (merge LSE/output globally, apply attn_sink
 * only once, never per rank); order restore from "[Core] Add MRV2 virtual-batch PCP for
 * MLA", "DualChunkSwap partitioning".
 * For token t, head h, contributors k (rows merge_src[t][k] >= 0, each with kv_splits
 * split slices: rows merge_src[t][k] + s * split_stride, s < kv_splits) and sink s_h:
 *   M = max(s_h, max_k L_k); D = exp(s_h - M) + sum_k exp(L_k - M);
 *   O = sum_k exp(L_k - M) O_k / D (bf16 RNE); LSE = M + log D (fp32).
 *
 *  o_cat     device bf16 [R_total][H][D_v]  partial outputs, ranks concatenated.
 *  lse_cat   device fp32 [R_total][H]       partial LSEs (natural log, no sink).
 *  merge_src device int32 [T_glob][P]       row per contributor or -1; rows outside
 *                                           [0, R_total) are ignored.
 *  sink      device fp32 [H] or NULL (no sink).
 *  o_out     device bf16 out [T_glob][H][D_v]; lse_out device fp32 [T_glob][H] or NULL.
 * A row with no contributor gets O = 0 and LSE = s_h (-inf without a sink). A contributor
 * slice whose weight exp(L_k - M) / D is zero (L_k = -inf: an empty key range, or a slice
 * its row does not use under per-row split KV) is not read, so its O may hold anything.
 * Errors: INVALID_ARG (null, sizes, P out of 1..64, kv_splits < 1, P * kv_splits above
 * 64, split_stride < 0, misalignment); UNSUPPORTED (D_v not a multiple of 8 in 8..1024,
 * H above 128); HIP.
 */
mla_status pcp_lse_merge(const void* o_cat, const float* lse_cat, const int32_t* merge_src,
                         int32_t P, int64_t T_glob, int32_t H, int32_t D_v, int64_t R_total,
                         int32_t kv_splits, int64_t split_stride, const float* sink, void* o_out,
                         float* lse_out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_PCP_H */
