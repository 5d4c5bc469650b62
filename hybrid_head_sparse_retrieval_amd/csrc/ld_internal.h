// Internal definitions shared by the gfx950 kernels and the host launcher of
// liblychee_decode.so. Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ld {

// ---------------------------------------------------------------- constants

constexpr int kThreads = 256;          // every kernel runs 4 wave64s per workgroup
constexpr int kMaxSplitRows = 4096;    // largest attention split (rows per workgroup)
constexpr int kSelChunk = 512;         // scores per select workgroup (2 per thread)
constexpr int kHist1Bins = 2048;       // digit 1: key bits 31..21
constexpr int kHist2Bins = 2048;       // digit 2: key bits 20..10
constexpr int kHist3Bins = 1024;       // digit 3: key bits 9..0
constexpr int kMaxSeq = 1 << 21;       // seq_len limit
constexpr int kMaxSelChunks = kMaxSeq / kSelChunk;   // 4096
constexpr int kSelSpan = 16384;        // scores per candidate / write workgroup (1024 x 16)
constexpr int kMaxSelSpans = kMaxSeq / kSelSpan;     // 128
constexpr int kMaxSplits = 1024;       // attention splits per sequence
constexpr int kMergeRun = 64;          // splits merged by one first-level merge
constexpr int kBitmapWordsPerBlock = 4096;           // bitmap-build LDS tile (16 KiB)
constexpr int kMaxSpins = 1 << 22;     // bound of a barrier wait (polls with a short sleep)
constexpr int kRep = 8;                // replicas of shared counters and histograms (workgroup id % kRep,
                                       // which is the XCD the workgroup runs on)
constexpr int kMaxParts = 32;          // selector workgroups per retrieval row, at most

// ---------------------------------------------------------------- parameters

// Attention over one layer: workgroup = (sequence b, KV group, split of rows).
struct AttnParams {
  // The workgroup prologue reads the first fields (split decode, sequence bounds, head
  // roles, first loads): they come first, so that its dependent kernel-argument reads
  // share a few scalar-cache lines.
  int B, Hq, Hkv, seq_len;
  // Groups that stream every row (they serve a retrieval head) come first in the grid
  // and use splits of ts_d rows; groups of sparse heads use splits of ts_s rows.
  int ts_d, ts_s;         // rows per split (multiples of 64)
  int nsplit_d, nsplit_s; // splits per sequence at seq_len (grid strides)
  int ngroups;            // KV groups launched
  int ng_dense;           // the first ng_dense of them stream
  int page_shift;         // paged KV (> 0): see block_table
  int W;                  // bitmap words per row
  uint64_t dense_groups;  // bit g: KV group g is launched and streams (ids ascending)
  uint64_t sparse_groups; // bit g: KV group g is launched and gathers (ids ascending, after
                          // the streaming ones)
  uint64_t active;        // heads computed by this launch
  uint64_t retrieval;     // heads attending to every row (subset of active)
  const int64_t* kv_indptr;
  int64_t kv_head_stride; // T*D elements
  int64_t total_tokens;   // T
  const uint16_t* q;      // bf16 [B][Hq][D]
  const void* kc;         // [Hkv][T][D], bf16, or E4M3 codes when kv_fp8
  const void* vc;
  uint32_t* bitmaps;      // [B*Hq][W] membership bits (read: sparse heads; written: selecting heads)
  float* logits;          // [B*Hq][seq_len] scores of retrieval heads, or null
  int do_topk;            // fused first selection digit and in-launch selection
  float scale;            // logit scale
  // paged KV (page_shift > 0): logical row i of sequence b is pool row
  // block_table[b * pages_per_seq + (i >> page_shift)] << page_shift | (i & page - 1)
  const int32_t* block_table;
  int pages_per_seq;
  int kv_fp8;
  int64_t npages;
  float v_scale;          // factor on O (the V dequantisation scale; 1 for bf16)
  int waves;              // waves per workgroup (4 or 8)
  uint16_t* out;          // bf16 [B][Hq][D]
  // HySparse gate (or null): O is written as w * O + (1 - w) * o_win[row] with
  // w = sigmoid(gate[row]), row = b * Hq + h; o_win fp32 [B*Hq][D]
  const float* gate;
  const float* o_win;
  float* part_ml;         // [B*Hq][P][2]  (max in log2 units, sum)
  float* part_acc;        // [B*Hq][P][D]
  int P;                  // partial stride in splits
  int P1;                 // first-level partial stride (ceil(P / kMergeRun))
  uint32_t* tickets;      // [B*Hkv], zero between calls
  uint32_t* tickets_l1;   // [B*Hkv][P1], zero between calls
  float* l1_ml;           // [B*Hq][P1][2]  first-level merged partials
  float* l1_acc;          // [B*Hq][P1][D]
  uint32_t* hist1;        // [B*Hq][kRep][kHist1Bins] (summed over replicas), zero between calls
  int k_dense;
  // finisher mode: the last split of each (b, g) to arrive merges O; with do_topk, up to
  // sel_cap splits that arrive just before it wait for it and then select the group's
  // retrieval rows, one workgroup per row (otherwise the last one selects them)
  int fin;
  const int64_t* s_indptr;
  int64_t s_cap;          // CSR S: entries of the S buffers (rows are clipped to them)
  int merge_w;            // workgroups that merge a KV group's O, at most
  int sel_cap;            // selectors per KV group, at most
  int sel_parts;          // selectors per retrieval row, at most (<= kMaxParts)
  uint32_t* sel_cnt;      // [B*Hq][2]: parts arrived (cleared per call)
  uint32_t* sel_cand;     // [B*Hq][seq_len] candidates (key bits 20..0), part q's from its first row
  uint64_t* sel_pub;      // [B*Hq][kMaxParts] per part: keys above bin b1 | candidates << 32
  uint64_t* gb_rel;       // [B*Hkv][P] release flags of the selectors (1: released; the
                          // selector clears its flag once it has seen it)
  int32_t* s_out;         // S rows written for selecting heads
  uint32_t* err;          // set when a barrier gave up waiting (never expected)
  // token-block sets (the last fields, so that the token path's argument layout is the
  // one it was tuned with): the maxima of each retrieval row's logits over 64-row blocks,
  // [B*nret][seq_len / 64] (row b * nret + the head's rank among the retrieval heads), or
  // null; and the block instance (gather waves own interleaved 64-row steps)
  float* blk_out;
  int gather_blocks;
};

// argsTopK over rows. Row slots index the per-row workspace arrays.
struct SelParams {
  int mode;               // 0: standalone rows, 1: retrieval rows of a layer
  int nrows;              // rows launched
  int C;                  // span-grid stride of the select passes (kSelSpan scores per span)
  int Ch;                 // chunk-grid stride of the standalone histogram (hchunk scores per chunk)
  int hchunk;             // scores per histogram workgroup (a multiple of kSelChunk)
  // standalone: row r has n_r = n_per_row ? clamp(n_per_row[r], 0, n) : n scores and
  // keeps k_r = min(k_per_row ? k_per_row[r] : k, row capacity, n_r) indices; rows are
  // idx_out + r * k (capacity k) or, with idx_indptr, idx_out + idx_indptr[r] (capacity
  // idx_indptr[r + 1] - idx_indptr[r])
  const float* scores; int64_t row_stride; int n; int k; int32_t* idx_out; float* val_out;
  const int32_t* n_per_row; const int32_t* k_per_row; const int64_t* idx_indptr;
  // layer rows: row r -> (b = r / nret, h = heads[r % nret])
  const float* logits; int Hq; int seq_len; const int64_t* kv_indptr;
  int32_t* s_out; const int64_t* s_indptr; int k_dense; int64_t s_cap;
  uint32_t* bitmaps; int W;
  int nret; uint8_t heads[64];
  // workspace (per row slot)
  uint32_t* hist1;        // [slots][kRep][kHist1Bins] (summed over replicas), zero between calls
  uint32_t* hist2;        // [slots][kHist2Bins], zero between calls
  uint32_t* tickets;      // [slots] arrivals, zero between calls
  uint32_t* err;          // the workspace's wait flag (set by the attention launch's bounded waits)
  uint32_t* sel_info;     // [slots][2]: the threshold key T and i_tie, from the row's last span
  uint32_t* span_cnt;     // [slots][C][2]: keys above bin b1, candidates (keys in bin b1)
  uint32_t* span_off;     // [slots][C]: output offset of each span
  uint64_t* cand;         // [slots][ncap]: (index << 32 | key) of the candidates, per span
  int64_t ncap;           // C * kSelSpan
  int hist_reps;          // set by launch_select: digit-1 histogram replicas the rows use
};

// Build membership bitmaps of sparse heads from S rows.
struct BitmapParams {
  const int32_t* s; const int64_t* s_indptr; int k_dense; int64_t s_cap;
  const int64_t* kv_indptr; int seq_len;
  int Hq; int nsp; uint8_t heads[64];   // row r -> (b = r / nsp, h = heads[r % nsp])
  uint32_t* bitmaps; int W;
  int wblocks;                          // word tiles per row
};

struct CopyParams {
  const int32_t* src; int32_t* dst; const int64_t* s_indptr; int k_dense; int64_t s_cap;
  int Hq; int nsp; uint8_t heads[64];
};

// Token-block selection (HySparse): block maxima of retrieval rows' logits, and the
// kept blocks' tokens written as S rows and membership bitmaps.
struct BlockParams {
  float* scores;                          // [rows][nblk] block maxima (written by the attention launch)
  const int32_t* kept;                    // [rows][kblk] kept blocks, ascending
  int rows, nblk, kblk;                   // retrieval rows, blocks per row, blocks kept per row
  int32_t* s_out; int k_dense;            // S rows [B][Hq][k_dense], k_dense = kblk * kBlock
  uint32_t* bitmaps; int W;
  int Hq; int nret; uint8_t heads[64];    // row r -> (b = r / nret, h = heads[r % nret])
};
constexpr int kBlock = 64;                // tokens per block

// ---------------------------------------------------------------- launchers

hipError_t launch_attention(const AttnParams& p, int D, int G, dim3 grid, hipStream_t st);
int64_t attention_capacity(int D, int G, int waves, bool fp8, bool paged);   // workgroups resident at once
// per KV group size G (ld_attention.hip, one compilation per G): occupancy per compute
// unit and the launch
template <int G> int64_t attention_capacity_g(int D, int waves, bool fp8);
template <int G> hipError_t launch_attention_g(const AttnParams& p, int D, dim3 grid, hipStream_t st);
template <int G> hipError_t launch_attention_blk_g(const AttnParams& p, int D, dim3 grid, hipStream_t st);
template <int G> int64_t attention_capacity_pg_g(int D, int waves, bool fp8);
template <int G> hipError_t launch_attention_pg_g(const AttnParams& p, int D, dim3 grid, hipStream_t st);
hipError_t launch_select(const SelParams& p, hipStream_t st, bool with_hist);
// kernels launch_select launches for p (1 to 3)
int select_launches(const SelParams& p, bool with_hist);
hipError_t launch_bitmap_build(const BitmapParams& p, int rows, hipStream_t st);
hipError_t launch_copy_rows(const CopyParams& p, int rows, hipStream_t st);
hipError_t launch_zero(void* ptr, size_t bytes, hipStream_t st);
// Sliding-window branch of a HySparse sparse layer: o[b*Hq+h] = softmax(q kw^T * scale) vw
// over the W rows of sequence b in kw/vw [Hkv][B*W][D] (bf16), fp32 out.
struct WindowParams {
  const uint16_t* q;
  const uint16_t* kw;
  const uint16_t* vw;
  float* o;
  int B, Hq, Hkv, D, W;
  float scale;
};
hipError_t launch_window(const WindowParams& p, hipStream_t st);

// Token Sparse Attention dense stage: for row b * Hq + h with selected positions
// idx[row][0..kk) (ascending), out[h][b*T + idx[i]] = softmax_j(q_i . k_j * scale) v_j
// over the selected rows (j <= i when causal). q, out [Hq][B*T][D]; k, v [Hkv][B*T][D].
struct TsaParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* idx;
  uint16_t* out;
  int B, Hq, Hkv, D, T, kk;
  int qtiles;             // ceil(kk / tsa_queries_per_block())
  float scale;
  int causal;
  // key splits: workgroup (row, query block, split s) takes selected keys
  // [s * split_keys, (s + 1) * split_keys); with nsplit > 1 the partials go to
  // part_ml [rows][qtiles][nsplit][queries per block][2] and part_o [..][D], merged by a
  // second launch
  int nsplit, split_keys;
  float* part_ml;
  float* part_o;
};
hipError_t launch_tsa(const TsaParams& p, hipStream_t st);
int tsa_queries_per_block();
// Key splits for kk selected keys of `rows` rows, and the bytes of their partials.
void tsa_splits(int64_t rows, int kk, int D, int* nsplit, int* split_keys, size_t* part_bytes);
hipError_t launch_block_expand(const BlockParams& p, int rows, hipStream_t st);
// Hybrid-head layer over a causal prefill: Q [Hq][B*T][D], K/V [Hkv][B*T][D], O like Q.
struct PrefillParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* out;
  int B, Hq, Hkv, D, T;
  int qtiles;             // ceil(T / prefill_rows_per_block()): row blocks, and key blocks of the sums
  uint64_t retrieval;     // bit h: query head h attends to every earlier token
  const int32_t* s_in;    // [B][Hq][kk] ascending token sets of the sparse heads
  int kk;
  float scale;
  float* lse;             // [B*Hq][T] log2-sum-exp2 of the retrieval rows' scaled scores
  float* imp;             // [B*Hq][T] column sums of the retrieval rows' attention matrices
  int nret;               // retrieval heads (column-sum launch: rows b * nret + i)
  uint8_t heads[64];      // their ids, ascending
};
int prefill_rows_per_block();
hipError_t launch_prefill_attention(const PrefillParams& p, hipStream_t st);
hipError_t launch_prefill_colsum(const PrefillParams& p, hipStream_t st);


}  // namespace ld
