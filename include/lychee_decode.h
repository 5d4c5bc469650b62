/*
 * lychee_decode.h -- C ABI of the MI355X (gfx950) hybrid-head sparse decode step.
 *
 * The method (LycheeDecode; "LycheeDecode: Accelerating Long-Context LLM Inference
 * via Hybrid-Head Sparse Decoding", summary page of arXiv 2602.04541, method
 * paragraph): for one decode token, every attention head of every layer is either a
 * RETRIEVAL head or a SPARSE head (the inference-time split E[z] > 0.5 of method
 * step 7 is supplied by the caller as a bit mask). Every head of layer 0 is a
 * retrieval head (step 1).
 *   - A retrieval head computes full attention softmax(q K^T / sqrt(d_k)) V over its
 *     whole KV cache and hands S = argsTopK(scores, k), a set of k token indices, to
 *     the head at the same position in the next layer (step 3).
 *   - A sparse head attends only to K[S], V[S] of its own layer's cache and forwards
 *     S unchanged (step 4).
 * For HySparse-style stacks ("HySparse: A Hybrid Sparse Attention Architecture
 * with Oracle Token Selection and KV Cache Sharing", section 3) the caller passes the
 * full layer's K/V pointers to the sparse layers.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All tensor pointers are DEVICE pointers owned by the caller; the library never
 *    allocates, frees or synchronises. Every call is asynchronous on `stream`.
 *  - bf16 tensors are 16-byte aligned:
 *      Q   [B][Hq][d]          (one decode token per sequence)
 *      K,V [Hkv][T][d]         (one layer; sequence b owns token rows
 *                               [kv_indptr[b], kv_indptr[b+1]) or [b*N, (b+1)*N))
 *      O   [B][Hq][d]
 *    Query head h reads KV head h / (Hq/Hkv).
 *  - S (int32, indices local to the sequence, in [0, N_b)):
 *      dense: [B][Hq][k];  CSR: row (b,h) = s[s_indptr[b*Hq+h] .. s_indptr[b*Hq+h+1]),
 *      s_indptr is a device int64 array of B*Hq+1 entries and the row length is that
 *      row's k. S rows written by this library are ascending. S rows read by it must
 *      hold distinct in-range entries (any order); entries outside [0, N_b) are
 *      ignored and duplicates count once.
 *  - The head-type mask is a uint64 passed by value: bit h set = retrieval head.
 *  - Top-k order: larger score first; equal scores -> lower index first; -0.0 equals
 *    +0.0; NaN ranks below every number. Scores are the fp32 logits q.k * scale.
 *  - Workspace: caller-owned device memory of at least ld_workspace_size() bytes
 *    (ld_topk_workspace_size() for ld_topk_select), 256-byte aligned. It must be
 *    zeroed once with ld_workspace_init() before its first use; every completed call
 *    leaves it ready for the next one (its counters and flags back at zero, the S
 *    bitmaps that LD_FLAG_S_CHAINED relies on kept). Calls that share a workspace must
 *    be ordered (same stream); concurrent calls need separate workspaces. No launch
 *    relies on all of its workgroups being resident at once: workgroups that wait for
 *    others of the same launch wait only for ones that are running or still to start,
 *    and are kept to a fraction of what the device holds, so other work on the device
 *    (other streams, other processes) can slow a call but not stall it.
 *  - Errors: arguments are validated on the host before any launch; a failing check
 *    returns an error code and launches nothing. Launch failures return LD_ERR_HIP.
 *    Faults inside kernels surface at the caller's next synchronisation. Per-sequence
 *    device-side values (kv_indptr, s_indptr) are preconditions: N_b >= 1 and
 *    1 <= k_{b,h} <= N_b; the kernels clamp k to N_b, clip CSR rows to
 *    ld_shape.s_capacity and never write outside a row.
 */
#ifndef LYCHEE_DECODE_H
#define LYCHEE_DECODE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t ld_status;
enum {
  LD_OK = 0,
  LD_ERR_INVALID_ARGUMENT = 1,  /* null pointer, bad size, misalignment, k out of range */
  LD_ERR_UNSUPPORTED = 2,       /* head_dim not 64/128, group size not 1/2/4/8, Hq > 64 */
  LD_ERR_WORKSPACE = 3,         /* workspace missing or smaller than required */
  LD_ERR_HIP = 4,               /* a HIP launch or copy failed */
  LD_ERR_DEVICE_WAIT = 5,       /* a bounded wait between workgroups gave up (see
                                   ld_workspace_check) */
  LD_ERR_SCRATCH_LIMIT = 6      /* ld_hybrid_layer_noalloc: the shape's scratch exceeds
                                   LD_NOALLOC_SCRATCH_BYTES */
};

/* Flags (bitwise OR). */
enum {
  /* Skip argsTopK for the retrieval heads (e.g. the last layer of a step); S and the
     workspace bitmaps are then left unchanged for those heads. */
  LD_FLAG_SKIP_TOPK = 1u << 0,
  /* The caller promises that s_in is the s_out written by the previous call on this
     workspace with the same shape, so the workspace's per-head membership bitmaps
     already describe s_in and need not be rebuilt. */
  LD_FLAG_S_CHAINED = 1u << 1,
  /* Launch-shape override: merge the split partials by tickets inside the attention
     launch and run argsTopK in launches of their own after it. By default the last
     split of each KV group to arrive merges O (with a few helpers) and the splits that
     arrive just before it select the group's S inside the same launch; the library
     itself takes the separate launches when the retrieval rows are too many for the
     in-launch selectors (e.g. a layer whose every head retrieves over a long context).
     S is the same either way; O may differ by fp32 rounding. */
  LD_FLAG_SEPARATE_SELECT = 1u << 2,
  /* Token-block selection (HySparse, section 3): a retrieval head keeps the k/64 blocks
     of 64 consecutive tokens with the largest block maxima of its logits (ties to the
     lower block, NaN lowest) and S = their tokens in ascending order. Requires k and
     seq_len to be multiples of 64, uniform sequences (kv_indptr NULL) and dense S
     (s_indptr NULL); otherwise the call returns LD_ERR_INVALID_ARGUMENT. In a layer
     without retrieval heads it tells the launch that the sets are whole blocks, which
     only changes how the work is split (any sets give the same result). */
  LD_FLAG_BLOCK_SELECT = 1u << 3
};
/* Optional launch-shape overrides (0 = automatic): rows per attention split =
   256 << (v - 1) for v = 1..5 in bits 8..11, for every KV group (automatic: groups
   serving a retrieval head get smaller splits than groups of sparse heads, so both
   finish together), and waves per attention workgroup in bits 12..13 (1 = 4 waves,
   2 = 8 waves). Results do not depend on them beyond fp32 rounding. */
#define LD_FLAG_SPLIT_ROWS(v) ((uint32_t)(v) << 8)
#define LD_FLAG_WAVES(v) ((uint32_t)(v) << 12)

typedef struct ld_shape {
  int32_t batch;          /* B >= 1 */
  int32_t num_q_heads;    /* Hq, 1..64 */
  int32_t num_kv_heads;   /* Hkv, divides Hq; Hq/Hkv in {1,2,4,8} */
  int32_t head_dim;       /* d in {64, 128} */
  int32_t seq_len;        /* N (uniform) or max_b N_b (ragged), 1..2097152 */
  int32_t page_size;      /* 0: each sequence's K/V rows are contiguous (from kv_indptr[b],
                             or b*seq_len). Else paged KV: a power of two in 16..4096;
                             logical row i of sequence b is pool row
                             block_table[b][i / page_size] * page_size + i % page_size. */
  int64_t total_tokens;   /* T: token rows per KV head in K/V (the head stride, in
                             rows); 0 selects batch*seq_len. Must cover every
                             sequence's rows. Paged: the pool's rows, a multiple of
                             page_size (required). */
  const int64_t* kv_indptr; /* device [B+1] token offsets, or NULL for uniform N. Paged:
                               only the lengths N_b = kv_indptr[b+1] - kv_indptr[b]. */
  float softmax_scale;    /* <= 0 selects 1/sqrt(head_dim) */
  int32_t pages_per_seq;  /* paged: row stride of block_table, >= ceil(seq_len/page_size);
                             else 0 */
  const int32_t* block_table; /* paged: device [B][pages_per_seq] page ids in
                                 0 .. total_tokens/page_size - 1 (ids outside are
                                 clamped); else NULL */
  int32_t kv_dtype;       /* 0: K and V are bf16. 1: K and V are 8-bit E4M3 codes (OCP
                             format: bias 7, no infinities), one byte per element, and
                             the values are k_scale * code and v_scale * code. */
  float k_scale;          /* kv_dtype 1: K dequantisation scale (> 0); else 0 */
  float v_scale;          /* kv_dtype 1: V dequantisation scale (> 0); else 0 */
  int32_t reserved;       /* must be 0 */
  int64_t s_capacity;     /* CSR S (s_indptr given): entries of the S buffers s_in and
                             s_out, required >= 1; every row [s_indptr[r],
                             s_indptr[r+1]) is clipped to [0, s_capacity), so offsets
                             past the buffer are never read or written. Dense S: 0. */
} ld_shape;

/* Human-readable text of a status code (static storage). */
const char* ld_status_string(ld_status status);

/* Bytes of workspace needed by ld_retrieval_decode / ld_sparse_decode /
   ld_hybrid_layer for this shape and a dense/CSR row length of at most k_max.
   Returns 0 for an invalid shape. */
size_t ld_workspace_size(const ld_shape* shape, int32_t k_max);

/* Bytes of workspace needed by ld_topk_select for `rows` rows of `n` scores. */
size_t ld_topk_workspace_size(int32_t rows, int32_t n);

/* Zero a workspace (a fill kernel on `stream`; safe to capture in a HIP graph). */
ld_status ld_workspace_init(void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Report and clear the workspace's wait flag (either kind of workspace). Workgroups
   that meet inside a launch wait for each other with a bounded spin; one that gives up
   sets the flag and carries on, so the results of the calls since the last check are
   then unreliable. Returns LD_ERR_DEVICE_WAIT when the flag was set, LD_OK when not,
   LD_ERR_WORKSPACE for a missing or too small workspace, LD_ERR_HIP when the copy
   fails. Copies 4 bytes to the host on `stream` and synchronises it; not for use
   inside a HIP graph capture. */
ld_status ld_workspace_check(void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Retrieval heads (method step 3): for every head h with bit h of head_mask set,
   O[b][h] = softmax(q K^T * scale) V over all N_b rows of its KV head, and, when
   s_out is non-NULL, S row (b,h) = argsTopK(scores, k) in ascending order (dense
   [B][Hq][k] or CSR through s_indptr). When scores_out is non-NULL the fp32 logits of
   the computed heads are written to scores_out [B][Hq][seq_len] (row-major; entries
   past N_b untouched). Heads outside head_mask are not touched. */
ld_status ld_retrieval_decode(const ld_shape* shape, uint64_t head_mask,
                              const void* q, const void* k_cache, const void* v_cache,
                              int32_t k, int32_t* s_out, const int64_t* s_indptr,
                              float* scores_out, void* out,
                              void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Sparse heads (method step 4): for every head h with bit h of head_mask set,
   O[b][h] = softmax(q K[S]^T * scale) V[S] over the rows of S row (b,h). S is not
   modified. flags: LD_FLAG_S_CHAINED. */
ld_status ld_sparse_decode(const ld_shape* shape, uint64_t head_mask,
                           const void* q, const void* k_cache, const void* v_cache,
                           int32_t k, const int32_t* s_in, const int64_t* s_indptr,
                           void* out, uint32_t flags,
                           void* workspace, size_t workspace_bytes, hipStream_t stream);

/* HySparse sparse layer (HySparse: A Hybrid Sparse Attention Architecture, section 3).
   Every query head h of sequence b combines two branches through a sigmoid gate:
     O_s = softmax(q K[S]^T * scale) V[S] over S row (b,h) of s_in, on k_cache/v_cache
           (the full layer's cache, shared; as ld_sparse_decode, paged or E4M3 allowed),
     O_w = softmax(q Kw^T * scale) Vw over the layer's own window cache: the last
           window_len tokens of the sequence, bf16 [Hkv][B*window_len][d] in
           k_window/v_window (rows of sequence b from b*window_len),
     O   = w * O_s + (1 - w) * O_w with w = 1 / (1 + exp(-gate[b][h])), gate device
           fp32 [B][Hq]; both branches stay fp32 until O is rounded to bf16.
   The window branch runs first (a small launch); the block-sparse attention launch
   mixes it in where it writes O.
   window_len in 1..4096. The workspace must hold ld_hysparse_workspace_size() bytes
   (zeroed once, as for the other entry points). It starts with a layer workspace of
   `shape`, so the same buffer serves ld_hybrid_layer for the full layer, and a sparse
   layer passing LD_FLAG_S_CHAINED reuses the bitmaps that the full layer's selection
   left there. flags: LD_FLAG_S_CHAINED and LD_FLAG_BLOCK_SELECT (as on a layer without
   retrieval heads: the sets are whole 64-token blocks, which only changes how the work
   is split). Errors are found before the first launch. */
size_t ld_hysparse_workspace_size(const ld_shape* shape, int32_t k_max, int32_t window_len);
ld_status ld_hysparse_layer(const ld_shape* shape, const void* q, const void* k_cache,
                            const void* v_cache, int32_t k, const int32_t* s_in,
                            const int64_t* s_indptr, const void* k_window,
                            const void* v_window, int32_t window_len, const float* gate,
                            void* out, uint32_t flags, void* workspace,
                            size_t workspace_bytes, hipStream_t stream);

/* Token Sparse Attention, compress -> dense -> scatter ("Token Sparse Attention:
   Efficient Long-Context Inference", Core Concept and Steps 2-3), over a prefill of T
   tokens per sequence. For every sequence b and query head h (KV head h / (Hq/Hkv)):
     I   = argsTopK(scores[b*Hq + h][0..T), min(k, T)), the order of ld_topk_select,
           written ascending to idx_out[b*Hq + h][0..min(k,T)) (int32, device);
     O_i = softmax_j(q_{I_i} . k_{I_j} * scale) v_{I_j} over the selected tokens only
           (flags & LD_TSA_CAUSAL: only I_j <= I_i);
     out row I_i of (h, b) = O_i (bf16); the other rows are zero with LD_TSA_ZERO_FILL,
           else left as the caller wrote them (the page keeps the residual there).
   Layouts (device, bf16, contiguous): q and out [Hq][B*T][d]; k_cache and v_cache
   [Hkv][B*T][d]; scores fp32 [B*Hq][T]. shape: batch, num_q_heads, num_kv_heads,
   head_dim (64 or 128), seq_len = T (1..2^21), softmax_scale (0 = 1/sqrt(d)),
   total_tokens 0 or B*T; kv_indptr, paging and kv_dtype must be unset
   (LD_ERR_UNSUPPORTED otherwise). The workspace holds ld_tsa_workspace_size(shape, k)
   bytes for a budget k (or any smaller one), zeroed once. Asynchronous on `stream`;
   errors are found before the first launch.
   flags & LD_TSA_GIVEN_IDX: no selection; idx_out already holds the caller's sets
   (ascending distinct positions in 0..T-1, min(k,T) per row; positions outside the
   sequence are clamped to it) and scores may be NULL. */
#define LD_TSA_CAUSAL 1u
#define LD_TSA_ZERO_FILL 2u
#define LD_TSA_GIVEN_IDX 4u
size_t ld_tsa_workspace_size(const ld_shape* shape, int32_t k);
ld_status ld_tsa_attention(const ld_shape* shape, const void* q, const void* k_cache,
                           const void* v_cache, const float* scores, int32_t k, int32_t* idx_out,
                           void* out, uint32_t flags, void* workspace, size_t workspace_bytes,
                           hipStream_t stream);

/* One layer of the recurrence over a causal PREFILL of T prompt tokens per sequence:
   the extension to the prefill stage that the LycheeDecode summary page names in its
   future-work paragraph, with method steps 3 and 4 read for T query rows. Layouts
   (head-major, one contiguous prompt per sequence): Q and O bf16 [Hq][B*T][d], K and V
   bf16 [Hkv][B*T][d], where sequence b owns rows b*T .. b*T + T - 1 (ld_shape:
   seq_len = T, total_tokens 0 or B*T, no kv_indptr, paging or 8-bit codes, else
   LD_ERR_UNSUPPORTED). Prompt row t attends to tokens 0..t of its own sequence.
     - Retrieval heads (bits of retrieval_mask): causal full attention; their S row
       (b,h) of s_out becomes argsTopK of the column sums of their attention matrix A
       (importance_j = sum over rows t >= j of A[t][j], the attention mass token j
       receives; ranked in the top-k order above, ascending indices out).
     - Sparse heads: row t attends to the tokens of S row (b,h) of s_in at positions
       <= t (a row that sees none of them is zero); S^{l+1} = S^{l} (rows copied when
       s_out differs from s_in). Their S rows must be ascending (this library writes
       them so).
   S is dense [B][Hq][k], 1 <= k <= T (the same layout as the decode layers').
   importance_out (nullable): fp32 [B][Hq][T], written for retrieval heads only.
   flags: LD_FLAG_SKIP_TOPK (attention only: no column sums, S and importance left as
   they were). Workspace: ld_prefill_workspace_size(shape, k) bytes, zeroed once with
   ld_workspace_init. */
size_t ld_prefill_workspace_size(const ld_shape* shape, int32_t k);
ld_status ld_prefill_hybrid_layer(const ld_shape* shape, uint64_t retrieval_mask,
                                  const void* q, const void* k_cache, const void* v_cache,
                                  int32_t k, const int32_t* s_in, int32_t* s_out,
                                  float* importance_out, void* out, uint32_t flags,
                                  void* workspace, size_t workspace_bytes, hipStream_t stream);

/* One full layer of the recurrence (method steps 3 and 4) for all Hq heads:
   retrieval heads (bits of retrieval_mask) attend to all rows and write their
   argsTopK rows into s_out; sparse heads attend to S row (b,h) of s_in and S^{l+1} =
   S^{l} for them (s_out may alias s_in; otherwise their rows are copied). s_in may be
   NULL only when every head is a retrieval head (layer 0, method step 1). A KV head
   whose query heads include a retrieval head streams its whole cache once for all of
   them; a KV head serving only sparse heads reads the union of their sets once.
   flags: LD_FLAG_SKIP_TOPK, LD_FLAG_S_CHAINED, LD_FLAG_SEPARATE_SELECT,
   LD_FLAG_BLOCK_SELECT, LD_FLAG_SPLIT_ROWS(), LD_FLAG_WAVES(). scores_out as in
   ld_retrieval_decode (retrieval heads only; may be NULL). */
ld_status ld_hybrid_layer(const ld_shape* shape, uint64_t retrieval_mask,
                          const void* q, const void* k_cache, const void* v_cache,
                          int32_t k, const int32_t* s_in, int32_t* s_out,
                          const int64_t* s_indptr, float* scores_out, void* out,
                          uint32_t flags, void* workspace, size_t workspace_bytes,
                          hipStream_t stream);

/* The launches ld_hybrid_layer makes for the same arguments, decided exactly as it
   decides them, without launching anything or touching any pointer (pointers only
   count as present or absent, so placeholders do; no workspace is needed). It queries
   the current device's compute-unit count and occupancy. Returns what ld_hybrid_layer
   would return for its argument checks (except the workspace check) and fills *plan:
   for launch-shape introspection, tests and per-kernel timing. */
typedef struct ld_layer_plan {
  int32_t launches;             /* kernels the call launches (0 when no head is active) */
  int32_t attention_workgroups; /* workgroups of the attention launch */
  int32_t split_rows_stream;    /* rows per split of KV groups that stream (0: none) */
  int32_t split_rows_gather;    /* rows per split of KV groups of sparse heads (0: none) */
  int32_t waves;                /* waves per attention workgroup */
  int32_t select_in_launch;     /* 1: the retrieval rows' S is selected inside the
                                   attention launch; 0: by launches of their own, or none */
  int32_t selector_parts;       /* in-launch selector workgroups per retrieval row, at most */
  int32_t reserved;
} ld_layer_plan;
ld_status ld_hybrid_layer_plan(const ld_shape* shape, uint64_t retrieval_mask,
                               const void* q, const void* k_cache, const void* v_cache,
                               int32_t k, const int32_t* s_in, int32_t* s_out,
                               const int64_t* s_indptr, float* scores_out, void* out,
                               uint32_t flags, ld_layer_plan* plan);

/* Standalone argsTopK (method step 3) on fp32 scores, row by row. Row r has
   n_r = n_per_row ? min(max(n_per_row[r], 0), n) : n scores starting at
   scores + r*row_stride, and keeps k_r indices: k_r = k_per_row ? k_per_row[r] : k,
   clamped to the row's output capacity and to n_r (the pages' k = min(k, seq_len):
   "Token Sparse Attention" skill page, Step 3; "LycheeDecode: Head-Level KV Cache
   Sharing" skill page, Step 1). Output rows: dense, idx_out + r*k with capacity k
   (k_per_row values above k are clamped to k), or CSR with idx_indptr (device int64,
   rows+1 offsets), idx_out + idx_indptr[r] with capacity idx_indptr[r+1] -
   idx_indptr[r]. The k_r indices are written in ascending order; entries past k_r are
   left as they were, and a row with k_r < 1 is left untouched. val_out (nullable)
   receives their scores at the same positions. n_per_row and k_per_row are device int32
   arrays of `rows` entries (nullable). Bit-exact: the result depends only on the fp32
   values and the order stated above. Requires rows >= 1, 1 <= n <= 2097152, k >= 1,
   row_stride >= n; the workspace holds ld_topk_workspace_size(rows, n) bytes. */
ld_status ld_topk_select(const float* scores, int32_t rows, int32_t n, int64_t row_stride,
                         const int32_t* n_per_row, int32_t k, const int32_t* k_per_row,
                         int32_t* idx_out, const int64_t* idx_indptr, float* val_out,
                         void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ld_hybrid_layer without a workspace, for callers that cannot allocate device memory:
   code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
   Same arguments, results and errors as ld_hybrid_layer, except that the scratch is a
   static buffer inside the library of LD_NOALLOC_SCRATCH_BYTES (128 MiB) per device,
   held from the first call on a device until the process ends. Shapes whose
   ld_workspace_size exceeds it return LD_ERR_SCRATCH_LIMIT before any launch (for
   example B = 1, Hq = 32, d = 128 fits up to about N = 200K). The call allocates and
   frees nothing; it launches a small fill kernel that clears the buffer's counters
   and histograms, then the layer's kernels. Every call on a device shares that
   device's buffer, which keeps the last call's contents: calls that overlap on one
   device (other streams, other threads) race and must be ordered by the caller.
   LD_FLAG_S_CHAINED is valid only when the previous call on the device wrote s_in with
   the same shape. The wait flag of ld_workspace_check is not reported for this buffer. */
#define LD_NOALLOC_SCRATCH_BYTES (128u << 20)
ld_status ld_hybrid_layer_noalloc(const ld_shape* shape, uint64_t retrieval_mask,
                                  const void* q, const void* k_cache, const void* v_cache,
                                  int32_t k, const int32_t* s_in, int32_t* s_out,
                                  const int64_t* s_indptr, float* scores_out, void* out,
                                  uint32_t flags, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* LYCHEE_DECODE_H */
