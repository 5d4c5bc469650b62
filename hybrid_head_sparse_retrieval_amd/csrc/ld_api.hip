// Host side of liblychee_decode.so: argument validation, workspace layout and the
// launch sequence of one layer (declared in include/lychee_decode.h).

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstring>
#include <mutex>

#include "lychee_decode.h"
#include "ld_internal.h"

namespace {

using namespace ld;

constexpr size_t kAlign = 256;
inline size_t align_up(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }


struct SelArrays {
  size_t tickets, hist1, hist2, err;                  // zero between calls
  size_t sel_info, span_cnt, span_off, cand;
  int C;
  int64_t ncap;
};

struct LayerLayout {
  int slots, P, P1, W;
  size_t attn_tickets, attn_tickets_l1;               // zero between calls
  SelArrays sel;
  size_t logits, part_ml, part_acc, l1_ml, l1_acc, bitmaps;
  size_t gb_rel;                                      // selectors' release flags
  size_t sel_cnt, sel_cand, sel_pub;                  // in-launch selection
  size_t blk_scores, blk_idx;                         // token-block selection
  size_t ctrl_end;                                    // end of the arrays that start at zero
  size_t total;
};

struct SelLayout {
  SelArrays sel;
  size_t total;
};

// Every workspace starts with a header line whose first word is the wait flag that
// kernels set when a bounded wait gives up (read and cleared by ld_workspace_check).
constexpr size_t kHeaderBytes = 256;
constexpr size_t kErrOffset = 0;

// Per-row selection scratch for `rows` rows of at most n scores: first the arrays that
// must be zero when a call starts (sel_ctrl), then the others (sel_data).
template <typename Take>
void sel_ctrl(SelArrays& a, int rows, Take take) {
  a.err = kErrOffset;
  a.tickets = take((size_t)rows * 4);
  a.hist1 = take((size_t)rows * kRep * kHist1Bins * 4);
  a.hist2 = take((size_t)rows * kHist2Bins * 4);
}
template <typename Take>
void sel_data(SelArrays& a, int rows, int n, Take take) {
  a.C = (n + kSelSpan - 1) / kSelSpan;
  a.ncap = (int64_t)a.C * kSelSpan;
  a.sel_info = take((size_t)rows * 8);
  a.span_cnt = take((size_t)rows * a.C * 8);
  a.span_off = take((size_t)rows * a.C * 4);
  a.cand = take((size_t)rows * a.ncap * 8);
}
template <typename Take>
SelArrays sel_arrays(int rows, int n, Take take) {
  SelArrays a{};
  sel_ctrl(a, rows, take);
  sel_data(a, rows, n, take);
  return a;
}

template <typename T>
T* at(void* ws, size_t off) { return reinterpret_cast<T*>(reinterpret_cast<uintptr_t>(ws) + off); }

// Scores per workgroup of the standalone digit-1 histogram: 512, doubled while the
// grid would exceed about 256 workgroups (long rows), at most 16384, so that each
// workgroup's fixed work (clearing and flushing 2048 bins) is spread over many scores
// (for 32 rows of 131072 scores, 256 workgroups measured faster than 128 or 512).
void set_hist_chunks(SelParams& sp, int64_t rows, int n) {
  int c = kSelChunk;
  while (c < 16384 && rows * ((n + c - 1) / c) > 256) c <<= 1;
  sp.hchunk = c;
  sp.Ch = (n + c - 1) / c;
}

void fill_sel(SelParams& sp, const SelArrays& a, void* ws) {
  sp.C = a.C;
  sp.hist1 = at<uint32_t>(ws, a.hist1);
  sp.hist2 = at<uint32_t>(ws, a.hist2);
  sp.tickets = at<uint32_t>(ws, a.tickets);
  sp.err = at<uint32_t>(ws, a.err);
  sp.sel_info = at<uint32_t>(ws, a.sel_info);
  sp.span_cnt = at<uint32_t>(ws, a.span_cnt);
  sp.span_off = at<uint32_t>(ws, a.span_off);
  sp.cand = at<uint64_t>(ws, a.cand);
  sp.ncap = a.ncap;
}

bool shape_ok(const ld_shape* s, ld_status* why) {
  *why = LD_ERR_INVALID_ARGUMENT;
  if (!s) return false;
  if (s->batch < 1 || s->num_q_heads < 1 || s->num_kv_heads < 1 || s->seq_len < 1) return false;
  if (s->total_tokens < 0) return false;
  if (s->page_size != 0) {
    // paged KV: a power-of-two page of 16..4096 rows, a block table that covers seq_len,
    // and a pool of whole pages
    const int ps = s->page_size;
    if (ps < 16 || ps > 4096 || (ps & (ps - 1)) != 0 || !s->block_table) return false;
    if ((int64_t)s->pages_per_seq * ps < s->seq_len || s->total_tokens <= 0 || s->total_tokens % ps != 0)
      return false;
  } else if (s->pages_per_seq != 0 || s->block_table) {
    return false;
  }
  if (s->reserved != 0 || s->s_capacity < 0) return false;
  if (s->kv_dtype == 1) {
    if (!(s->k_scale > 0.f) || !(s->v_scale > 0.f) || !std::isfinite(s->k_scale) || !std::isfinite(s->v_scale))
      return false;
  } else if (s->kv_dtype != 0 || s->k_scale != 0.f || s->v_scale != 0.f) {
    return false;
  }
  if (s->seq_len > kMaxSeq) { *why = LD_ERR_UNSUPPORTED; return false; }
  if (s->num_q_heads > 64) { *why = LD_ERR_UNSUPPORTED; return false; }
  if (s->num_q_heads % s->num_kv_heads != 0) return false;
  const int G = s->num_q_heads / s->num_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8) { *why = LD_ERR_UNSUPPORTED; return false; }
  if (s->head_dim != 64 && s->head_dim != 128) { *why = LD_ERR_UNSUPPORTED; return false; }
  if (!s->kv_indptr && s->page_size == 0 && s->total_tokens != 0 &&
      s->total_tokens < (int64_t)s->batch * s->seq_len)
    return false;
  if (!(std::isfinite(s->softmax_scale))) return false;
  return true;
}

LayerLayout layer_layout(const ld_shape* s) {
  LayerLayout L{};
  const int N = s->seq_len;
  L.slots = s->batch * s->num_q_heads;
  L.P = (N + 63) / 64;
  if (L.P > kMaxSplits) L.P = kMaxSplits;
  L.W = (N + 31) / 32;
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t at = o; o = align_up(o + bytes); return at; };
  L.P1 = (L.P + kMergeRun - 1) / kMergeRun;
  take(kHeaderBytes);
  // arrays that hold zero when a call starts (every call leaves them so); they come first
  // so that one fill over [kHeaderBytes, ctrl_end) restores them
  L.attn_tickets = take((size_t)s->batch * s->num_kv_heads * 4);
  L.attn_tickets_l1 = take((size_t)s->batch * s->num_kv_heads * L.P1 * 4);
  sel_ctrl(L.sel, L.slots, take);
  L.gb_rel = take((size_t)s->batch * s->num_kv_heads * L.P * 128);
  L.sel_cnt = take((size_t)L.slots * 2 * 4);
  L.ctrl_end = o;
  sel_data(L.sel, L.slots, N, take);
  L.logits = take((size_t)L.slots * N * 4);
  L.part_ml = take((size_t)L.slots * L.P * 8);
  L.part_acc = take((size_t)L.slots * L.P * s->head_dim * 4);
  L.l1_ml = take((size_t)L.slots * L.P1 * 8);
  L.l1_acc = take((size_t)L.slots * L.P1 * s->head_dim * 4);
  L.bitmaps = take((size_t)L.slots * L.W * 4);
  L.sel_cand = take((size_t)L.slots * N * 4);
  L.sel_pub = take((size_t)L.slots * kMaxParts * 8);
  L.blk_scores = take((size_t)L.slots * ((N + kBlock - 1) / kBlock) * 4);
  L.blk_idx = take((size_t)L.slots * ((N + kBlock - 1) / kBlock) * 4);
  L.total = o;
  return L;
}

SelLayout sel_layout(int rows, int n) {
  SelLayout L{};
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t at = o; o = align_up(o + bytes); return at; };
  take(kHeaderBytes);
  L.sel = sel_arrays(rows, n, take);
  L.total = o;
  return L;
}

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Compute units of the current device (cached per device).
int cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int c = cache[dev].load(std::memory_order_relaxed);
  if (c > 0) return c;
  if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c <= 0) c = 256;
  cache[dev].store(c, std::memory_order_relaxed);
  return c;
}

}  // namespace

namespace ld {

int64_t attention_capacity(int D, int G, int waves, bool fp8, bool paged) {
  // cached per device and (D, G, waves, KV format, paged)
  static std::atomic<int64_t> cache[64][2][4][2][2][2];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  const int di = D == 128 ? 1 : 0;
  const int gi = G == 1 ? 0 : G == 2 ? 1 : G == 4 ? 2 : 3;
  const int wi = waves == 8 ? 1 : 0;
  const int fi = fp8 ? 1 : 0;
  const int pi = paged ? 1 : 0;
  int64_t c = cache[dev][di][gi][wi][fi][pi].load(std::memory_order_relaxed);
  if (c > 0) return c;
  int64_t per_cu = 0;
  switch (G) {
    case 1: per_cu = paged ? attention_capacity_pg_g<1>(D, waves, fp8) : attention_capacity_g<1>(D, waves, fp8); break;
    case 2: per_cu = paged ? attention_capacity_pg_g<2>(D, waves, fp8) : attention_capacity_g<2>(D, waves, fp8); break;
    case 4: per_cu = paged ? attention_capacity_pg_g<4>(D, waves, fp8) : attention_capacity_g<4>(D, waves, fp8); break;
    case 8: per_cu = paged ? attention_capacity_pg_g<8>(D, waves, fp8) : attention_capacity_g<8>(D, waves, fp8); break;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  c = per_cu * cus;
  cache[dev][di][gi][wi][fi][pi].store(c, std::memory_order_relaxed);
  return c;
}

hipError_t launch_attention(const AttnParams& p, int D, int G, dim3 grid, hipStream_t st) {
  if (p.gather_blocks) {
    switch (G) {
      case 1: return launch_attention_blk_g<1>(p, D, grid, st);
      case 2: return launch_attention_blk_g<2>(p, D, grid, st);
      case 4: return launch_attention_blk_g<4>(p, D, grid, st);
      case 8: return launch_attention_blk_g<8>(p, D, grid, st);
    }
    return hipErrorInvalidValue;
  }
  if (p.page_shift) {
    switch (G) {
      case 1: return launch_attention_pg_g<1>(p, D, grid, st);
      case 2: return launch_attention_pg_g<2>(p, D, grid, st);
      case 4: return launch_attention_pg_g<4>(p, D, grid, st);
      case 8: return launch_attention_pg_g<8>(p, D, grid, st);
    }
    return hipErrorInvalidValue;
  }
  switch (G) {
    case 1: return launch_attention_g<1>(p, D, grid, st);
    case 2: return launch_attention_g<2>(p, D, grid, st);
    case 4: return launch_attention_g<4>(p, D, grid, st);
    case 8: return launch_attention_g<8>(p, D, grid, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace ld

namespace {

using namespace ld;

// Waves per attention workgroup: flag bits 12..13 = 1 or 2 force 4 or 8; otherwise 4
// (two workgroups per compute unit: with the group's last arrivals finishing it, the
// 32K step measured 1.24 ms with 4 waves against 1.30 ms with 8).
int choose_waves(uint32_t flags) {
  const uint32_t v = (flags >> 12) & 0x3u;
  return v == 2u ? 8 : 4;
}

// Rows per split for the groups that stream every row (ts_d) and for the groups of
// sparse heads, which visit only the union of their rows (ts_s). Flag bits 8..11 = v
// (1..5) force 256 << (v-1) rows for both. Otherwise both finish together and the grid
// fits in one round of resident workgroups (`capacity`): a streaming split of ts_d rows
// costs as much as a gathering split of ts_s rows of estimated union density rho, plus,
// when the group selects inside the launch, the selection's fixed latency counted as
// `sel_rows` rows of streaming. The smallest ts_s that fits gives the most parallelism.
// Returns false when no choice fits (the caller then takes one uniform size).
// (sel_rows = 256 rows measured best: 32K steps 1.184 / 1.179 / 1.190 / 1.191 / 1.237 ms and
// 128K steps 3.210 / 3.206 / 3.211 / 3.284 / 3.328 ms for 128 / 256 / 384 / 512 / 768)
constexpr int kSelRows = 256;
// A streamed row of a group that serves a retrieval head costs about 1.12 visited rows of
// a gathering group: it also writes the row's logits and counts them in the fused
// histogram (measured per workgroup at 128K rows: 21.9 against 24.5 rows per us).
constexpr double kStreamRowCost = 1.12;
bool choose_splits(int N, int B, int ng_dense, int ng_sparse, double rho, int sel_rows, int64_t capacity,
                   uint32_t flags, int* ts_d, int* ts_s) {
  const int v = (int)((flags >> 8) & 0xfu);
  auto nsp = [&](int ts) { return (int64_t)((N + ts - 1) / ts); };
  if (v >= 1 && v <= 5) {
    *ts_d = *ts_s = 256 << (v - 1);
    return true;
  }
  // Every split of the launch runs at once. A streaming split of d rows visits d rows (at
  // kStreamRowCost each), a gathering split of s rows about rho * s, and a streaming
  // group's selection adds about sel_rows rows' time after its last split; the launch
  // ends with the slower of the two. For each gather split size, the streaming groups get the smallest split
  // (a multiple of 64, at least 192 rows) whose grid still fits next to the gathering
  // groups', and the pair that ends first wins (ties: the smaller splits).
  double best = 1e300;
  int bd = 0, bs = 0;
  for (int s = 256; s <= kMaxSplitRows; s += 64) {
    if (ng_sparse && nsp(s) > kMaxSplits) continue;
    const int64_t used = ng_sparse ? (int64_t)B * ng_sparse * nsp(s) : 0;
    if (used > capacity) continue;
    int d = s;
    if (ng_dense) {
      const int64_t room = (capacity - used) / ((int64_t)B * ng_dense);   // splits per streaming group
      if (room < 1) continue;
      d = (int)std::max<int64_t>(192, ((N + room - 1) / room + 63) / 64 * 64);
      if (d > kMaxSplitRows || nsp(d) > kMaxSplits) continue;
    }
    const double cost = std::max(ng_dense ? (double)(kStreamRowCost * d + sel_rows) : 0.0, ng_sparse ? rho * s : 0.0);
    if (cost < best) {
      best = cost;
      bd = d;
      bs = ng_sparse ? s : d;
    }
    if (!ng_sparse) break;                     // only streaming groups: s plays no part
  }
  if (!bd) return false;
  *ts_d = bd;
  *ts_s = bs;
  return true;
}

// Uniform split size when the grid cannot fit one round: the smallest power of two
// from 256 rows that keeps each sequence within kMaxSplits splits and, if possible,
// the grid within `capacity`.
int uniform_split(int N, int64_t groups_total, int64_t capacity) {
  int ts = 256;
  while (ts < kMaxSplitRows && groups_total * (int64_t)((N + ts - 1) / ts) > capacity) ts <<= 1;
  while ((N + ts - 1) / ts > kMaxSplits && ts < kMaxSplitRows) ts <<= 1;
  return ts;
}

// Core of the three layer entry points.
// active: heads computed; retrieval: heads attending to all rows (subset of active).
ld_status run_layer(const ld_shape* shape, uint64_t active, uint64_t retrieval, const void* q,
                    const void* kc, const void* vc, int32_t k, const int32_t* s_in,
                    int32_t* s_out, const int64_t* s_indptr, float* scores_out, void* out,
                    uint32_t flags, bool want_topk, void* ws, size_t ws_bytes, hipStream_t st,
                    const float* gate = nullptr, const float* o_win = nullptr, bool clear_ctrl = false,
                    ld_layer_plan* plan = nullptr) {
  // plan != null: validate and decide as for a launch, count the kernels instead of
  // launching them, and describe the attention launch in *plan
  if (plan) *plan = ld_layer_plan{};
#define LD_LAUNCH(expr, count)                                  \
  do {                                                          \
    if (plan) plan->launches += (count);                        \
    else if ((expr) != hipSuccess) return LD_ERR_HIP;           \
  } while (0)
  ld_status why;
  if (!shape_ok(shape, &why)) return why;
  const int B = shape->batch, Hq = shape->num_q_heads, Hkv = shape->num_kv_heads;
  const int D = shape->head_dim, G = Hq / Hkv, N = shape->seq_len;
  const uint64_t all = (Hq == 64) ? ~0ull : ((1ull << Hq) - 1ull);
  if ((active & ~all) || (retrieval & ~active)) return LD_ERR_INVALID_ARGUMENT;
  if (!q || !kc || !vc || !out) return LD_ERR_INVALID_ARGUMENT;
  if (!aligned16(q) || !aligned16(kc) || !aligned16(vc) || !aligned16(out)) return LD_ERR_INVALID_ARGUMENT;
  if (k < 1 || k > N) return LD_ERR_INVALID_ARGUMENT;
  const uint64_t sparse = active & ~retrieval;
  const bool do_topk = want_topk && retrieval != 0;
  const bool block = do_topk && (flags & LD_FLAG_BLOCK_SELECT);
  if (block && (k % kBlock != 0 || N % kBlock != 0 || shape->kv_indptr || s_indptr)) return LD_ERR_INVALID_ARGUMENT;
  if (sparse && !s_in) return LD_ERR_INVALID_ARGUMENT;
  if (s_indptr && ((uintptr_t)s_indptr & 7u || shape->s_capacity < 1)) return LD_ERR_INVALID_ARGUMENT;
  const int64_t s_cap = s_indptr ? shape->s_capacity : (int64_t)B * Hq * k;
  if (do_topk && !s_out) return LD_ERR_INVALID_ARGUMENT;
  if ((s_in && ((uintptr_t)s_in & 3u)) || (s_out && ((uintptr_t)s_out & 3u))) return LD_ERR_INVALID_ARGUMENT;
  if (scores_out && ((uintptr_t)scores_out & 3u)) return LD_ERR_INVALID_ARGUMENT;
  const LayerLayout L = layer_layout(shape);
  if (!plan && (!ws || ws_bytes < L.total || ((uintptr_t)ws & 15u))) return LD_ERR_WORKSPACE;
  if (active == 0) return LD_OK;

  int64_t T = shape->total_tokens;
  if (T == 0) T = (int64_t)B * N;
  const float scale = shape->softmax_scale > 0.f ? shape->softmax_scale : 1.0f / std::sqrt((float)D);

  // heads lists
  uint8_t sp_heads[64], ret_heads[64];
  int nsp = 0, nret = 0;
  for (int h = 0; h < Hq; ++h) {
    if (sparse >> h & 1ull) sp_heads[nsp++] = (uint8_t)h;
    if (retrieval >> h & 1ull) ret_heads[nret++] = (uint8_t)h;
  }
  uint32_t* bitmaps = at<uint32_t>(ws, L.bitmaps);

  // 0. a buffer that other shapes' calls may have used: its counters, histograms and
  // release words start from zero (a fill kernel, so the call stays capturable)
  if (clear_ctrl) LD_LAUNCH(launch_zero(at<char>(ws, kHeaderBytes), L.ctrl_end - kHeaderBytes, st), 1);

  // 1. membership bitmaps of the sparse heads (unless the caller chains them)
  if (nsp && !(flags & LD_FLAG_S_CHAINED)) {
    BitmapParams bp{};
    bp.s = s_in; bp.s_indptr = s_indptr; bp.k_dense = k; bp.s_cap = s_cap;
    bp.kv_indptr = shape->kv_indptr; bp.seq_len = N;
    bp.Hq = Hq; bp.nsp = nsp;
    std::memcpy(bp.heads, sp_heads, sizeof(sp_heads));
    bp.bitmaps = bitmaps; bp.W = L.W;
    bp.wblocks = (L.W + kBitmapWordsPerBlock - 1) / kBitmapWordsPerBlock;
    LD_LAUNCH(launch_bitmap_build(bp, B * nsp, st), 1);
  }
  // 2. S^{l+1} = S^{l} for sparse heads when the output buffer is a different one
  if (nsp && s_out && s_out != s_in) {
    CopyParams cp{};
    cp.src = s_in; cp.dst = s_out; cp.s_indptr = s_indptr; cp.k_dense = k; cp.s_cap = s_cap;
    cp.Hq = Hq; cp.nsp = nsp;
    std::memcpy(cp.heads, sp_heads, sizeof(sp_heads));
    LD_LAUNCH(launch_copy_rows(cp, B * nsp, st), 1);
  }
  // 3. attention (+ fused first selection digit)
  AttnParams ap{};
  ap.q = static_cast<const uint16_t*>(q);
  ap.kc = kc;
  ap.vc = vc;
  ap.kv_fp8 = shape->kv_dtype == 1 ? 1 : 0;
  ap.v_scale = ap.kv_fp8 ? shape->v_scale : 1.f;
  ap.out = static_cast<uint16_t*>(out);
  ap.gate = gate;
  ap.o_win = o_win;
  ap.kv_indptr = shape->kv_indptr;
  ap.kv_head_stride = T * D;
  ap.total_tokens = T;
  if (shape->page_size) {
    ap.block_table = shape->block_table;
    ap.page_shift = __builtin_ctz((unsigned)shape->page_size);
    ap.pages_per_seq = shape->pages_per_seq;
    ap.npages = T >> ap.page_shift;
  }
  ap.B = B; ap.Hq = Hq; ap.Hkv = Hkv; ap.seq_len = N;
  ap.scale = ap.kv_fp8 ? scale * shape->k_scale : scale;
  ap.active = active; ap.retrieval = retrieval;
  // groups that stream (they serve a retrieval head) first, then groups of sparse heads
  int ng = 0, ng_dense = 0, ret_per_group = 0, sp_per_group = 0;
  for (int pass = 0; pass < 2; ++pass) {
    for (int g = 0; g < Hkv; ++g) {
      const uint64_t gm = ((G == 64) ? ~0ull : ((1ull << G) - 1ull)) << (g * G);
      if (!(active & gm)) continue;
      const bool streams = (retrieval & gm) != 0;
      if (streams != (pass == 0)) continue;
      ++ng;
      (streams ? ap.dense_groups : ap.sparse_groups) |= 1ull << g;
      ret_per_group = std::max(ret_per_group, __builtin_popcountll(retrieval & gm));
      sp_per_group = std::max(sp_per_group, __builtin_popcountll(active & ~retrieval & gm));
    }
    if (pass == 0) ng_dense = ng;
  }
  ap.ngroups = ng;
  ap.ng_dense = ng_dense;
  ap.gather_blocks = (flags & LD_FLAG_BLOCK_SELECT) ? 1 : 0;   // the sets are whole 64-token blocks
  ap.waves = ap.gather_blocks ? 4 : choose_waves(flags);
  // Finisher mode (default): the last split of each KV group to arrive merges O, and
  // the retrieval rows are selected inside the launch by the splits that arrive just
  // before it. At most a quarter of the resident capacity may wait for its group's last
  // arrival at once, so every wait ends. Separate mode (LD_FLAG_SEPARATE_SELECT, or
  // chosen here when the in-launch selectors would be too few for the rows): ticket
  // merge inside the launch and the selection in launches of their own.
  const int64_t capacity = attention_capacity(D, G, ap.waves, ap.kv_fp8 != 0, ap.page_shift != 0);
  bool fin = !(flags & LD_FLAG_SEPARATE_SELECT);
  bool in_select = fin && do_topk && !block;
  const int sel_groups = B * ng_dense;
  // Merge helpers and selectors wait for their group's last split: up to 8 workgroups
  // (4 in a launch that selects) per group merge O (half the budget at most); of the
  // rest, few rows share up to
  // kMaxParts selectors each (enough for one pass of 16 keys per thread), many rows get
  // one selector each (sel_cap per group; 0: the last arrival selects every row).
  {
    const int64_t budget = capacity / 4;
    const int64_t rows = (int64_t)B * nret;
    const int64_t groups_total = std::max<int64_t>(1, (int64_t)B * ng);
    // (4 mergers per group when the launch also selects: its retrieval layers took 102.4
    // against 104.5 us at 128K rows, the merge itself no longer)
    ap.merge_w = (int)std::max<int64_t>(1, std::min<int64_t>(in_select ? 4 : 8, 1 + budget / 2 / groups_total));
    const int64_t sel_budget = budget - (int64_t)(ap.merge_w - 1) * groups_total;
    const int64_t pass = 16LL * 64 * ap.waves;
    const int64_t want = std::max<int64_t>(2, (N + pass - 1) / pass);
    if (rows > 0 && 2 * rows <= sel_budget) {
      // parts <= threads / 8, so that each part's sub-list has 8 readers when they gather
      ap.sel_parts = (int)std::min<int64_t>({(int64_t)kMaxParts, sel_budget / rows, want, 64LL * ap.waves / 8});
      ap.sel_cap = G * ap.sel_parts;
    } else {
      ap.sel_parts = 1;
      ap.sel_cap = (int)std::min<int64_t>(G, std::max<int64_t>(0, sel_budget) / std::max(1, sel_groups));
    }
    // Rows that would get under half the parts one pass needs (a full-attention layer's
    // 32 heads at 32K rows get 2 of 8): the selection launches, with many workgroups per
    // row, finish sooner (measured at 32K and 128K rows: 82 vs 90 and 170 vs 285 us).
    if (in_select && rows > 0 && 2 * (int64_t)ap.sel_parts < want) {
      fin = false;
      in_select = false;
    }
  }
  ap.fin = fin ? 1 : 0;
  // union density of a sparse group's rows if its heads' sets were independent
  const double kf = std::min(1.0, (double)k / (double)N);
  const double rho = 1.0 - std::pow(1.0 - kf, (double)std::max(1, sp_per_group));
  // the selection's latency after a streaming group's last split, in streamed rows
  const int sel_rows = in_select ? kSelRows : 0;
  if (!choose_splits(N, B, ng_dense, ng - ng_dense, rho, sel_rows, capacity, flags, &ap.ts_d, &ap.ts_s))
    ap.ts_d = ap.ts_s = uniform_split(N, (int64_t)B * ng, capacity);
  ap.nsplit_d = (N + ap.ts_d - 1) / ap.ts_d;
  ap.nsplit_s = (N + ap.ts_s - 1) / ap.ts_s;
  ap.bitmaps = bitmaps; ap.W = L.W;
  // token selection reads the logits from the workspace (or scores_out); block selection
  // takes the launch's block maxima instead
  ap.logits = scores_out ? scores_out : ((do_topk && !block) ? at<float>(ws, L.logits) : nullptr);
  ap.blk_out = block ? at<float>(ws, L.blk_scores) : nullptr;
  ap.part_ml = at<float>(ws, L.part_ml);
  ap.part_acc = at<float>(ws, L.part_acc);
  ap.P = L.P;
  ap.tickets = at<uint32_t>(ws, L.attn_tickets);
  ap.tickets_l1 = at<uint32_t>(ws, L.attn_tickets_l1);
  ap.l1_ml = at<float>(ws, L.l1_ml);
  ap.l1_acc = at<float>(ws, L.l1_acc);
  ap.P1 = L.P1;
  ap.do_topk = (do_topk && !block) ? 1 : 0;     // block selection needs the logits only
  ap.hist1 = at<uint32_t>(ws, L.sel.hist1);
  ap.k_dense = k;
  ap.s_indptr = s_indptr;
  ap.s_cap = s_cap;
  ap.s_out = s_out;
  ap.gb_rel = at<uint64_t>(ws, L.gb_rel);
  ap.sel_cnt = at<uint32_t>(ws, L.sel_cnt);
  ap.sel_cand = at<uint32_t>(ws, L.sel_cand);
  ap.sel_pub = at<uint64_t>(ws, L.sel_pub);
  ap.err = at<uint32_t>(ws, L.sel.err);
  const int64_t nwg = (int64_t)B * ((int64_t)ng_dense * ap.nsplit_d + (int64_t)(ng - ng_dense) * ap.nsplit_s);
  if (plan) {
    plan->attention_workgroups = (int32_t)nwg;
    plan->split_rows_stream = ng_dense ? ap.ts_d : 0;
    plan->split_rows_gather = ng > ng_dense ? ap.ts_s : 0;
    plan->waves = ap.waves;
    plan->select_in_launch = in_select && nret > 0 ? 1 : 0;
    plan->selector_parts = plan->select_in_launch ? ap.sel_parts : 0;
  }
  LD_LAUNCH(launch_attention(ap, D, G, dim3((unsigned)nwg), st), 1);

  // 4. argsTopK of the retrieval rows: by token blocks (block maxima, then the same
  // radix select over the block scores, then the kept blocks' tokens), or by tokens
  if (block) {
    BlockParams bk{};
    bk.scores = at<float>(ws, L.blk_scores);
    bk.kept = at<int32_t>(ws, L.blk_idx);
    bk.rows = B * nret; bk.nblk = N / kBlock; bk.kblk = k / kBlock;
    bk.s_out = s_out; bk.k_dense = k;
    bk.bitmaps = bitmaps; bk.W = L.W;
    bk.Hq = Hq; bk.nret = nret;
    std::memcpy(bk.heads, ret_heads, sizeof(ret_heads));
    SelParams sp{};
    sp.mode = 0;
    sp.nrows = bk.rows;
    set_hist_chunks(sp, B * nret, bk.nblk);
    sp.scores = bk.scores; sp.row_stride = bk.nblk; sp.n = bk.nblk; sp.k = bk.kblk;
    sp.idx_out = at<int32_t>(ws, L.blk_idx); sp.val_out = nullptr;
    fill_sel(sp, L.sel, ws);
    sp.C = (bk.nblk + kSelSpan - 1) / kSelSpan;    // spans of this row length
    LD_LAUNCH(launch_select(sp, st, true), select_launches(sp, true));
    LD_LAUNCH(launch_block_expand(bk, bk.rows, st), 1);
  } else if (do_topk && !in_select) {
    SelParams sp{};
    sp.mode = 1;
    sp.nrows = B * nret;
    sp.logits = ap.logits; sp.Hq = Hq; sp.seq_len = N; sp.kv_indptr = shape->kv_indptr;
    sp.s_out = s_out; sp.s_indptr = s_indptr; sp.k_dense = k; sp.s_cap = s_cap;
    sp.bitmaps = bitmaps; sp.W = L.W;
    sp.nret = nret;
    std::memcpy(sp.heads, ret_heads, sizeof(ret_heads));
    fill_sel(sp, L.sel, ws);
    LD_LAUNCH(launch_select(sp, st, false), select_launches(sp, false));
  }
  return LD_OK;
#undef LD_LAUNCH
}

}  // namespace

extern "C" {

const char* ld_status_string(ld_status status) {
  switch (status) {
    case LD_OK: return "ok";
    case LD_ERR_INVALID_ARGUMENT: return "invalid argument";
    case LD_ERR_UNSUPPORTED: return "unsupported shape";
    case LD_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case LD_ERR_HIP: return "HIP launch or copy failed";
    case LD_ERR_DEVICE_WAIT: return "a bounded wait between workgroups gave up";
    case LD_ERR_SCRATCH_LIMIT: return "the shape needs more scratch than the library's static buffer holds";
  }
  return "unknown status";
}

size_t ld_workspace_size(const ld_shape* shape, int32_t k_max) {
  ld_status why;
  if (!shape_ok(shape, &why) || k_max < 1 || k_max > shape->seq_len) return 0;
  return layer_layout(shape).total;
}

}  // extern "C"

namespace {

// The HySparse layer's workspace: a layer workspace of the shared cache, then the
// window branch's fp32 output.
struct HysLayout {
  size_t main, o_w, total;
};
bool hys_layout(const ld_shape* s, int32_t window_len, HysLayout* H) {
  ld_status why;
  if (!shape_ok(s, &why) || window_len < 1 || window_len > 4096) return false;
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t at = o; o = align_up(o + bytes); return at; };
  H->main = take(layer_layout(s).total);
  H->o_w = take((size_t)s->batch * s->num_q_heads * s->head_dim * 4);
  H->total = o;
  return true;
}

}  // namespace

extern "C" {

size_t ld_hysparse_workspace_size(const ld_shape* shape, int32_t k_max, int32_t window_len) {
  HysLayout H;
  if (!shape || k_max < 1 || k_max > shape->seq_len || !hys_layout(shape, window_len, &H)) return 0;
  return H.total;
}

ld_status ld_hysparse_layer(const ld_shape* shape, const void* q, const void* k_cache,
                            const void* v_cache, int32_t k, const int32_t* s_in,
                            const int64_t* s_indptr, const void* k_window,
                            const void* v_window, int32_t window_len, const float* gate,
                            void* out, uint32_t flags, void* workspace,
                            size_t workspace_bytes, hipStream_t stream) {
  HysLayout H;
  ld_status why;
  if (!shape) return LD_ERR_INVALID_ARGUMENT;
  if (!shape_ok(shape, &why)) return why;
  if (!hys_layout(shape, window_len, &H)) return LD_ERR_INVALID_ARGUMENT;
  // every check is made before the first launch
  if (!q || !aligned16(q) || !s_in || ((uintptr_t)s_in & 3u) || !k_window || !v_window || !gate || !out ||
      ((uintptr_t)gate & 3u))
    return LD_ERR_INVALID_ARGUMENT;
  if (!k_cache || !v_cache || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out))
    return LD_ERR_INVALID_ARGUMENT;
  if (!aligned16(k_window) || !aligned16(v_window)) return LD_ERR_INVALID_ARGUMENT;
  if (flags & ~(uint32_t)(LD_FLAG_S_CHAINED | LD_FLAG_BLOCK_SELECT)) return LD_ERR_INVALID_ARGUMENT;
  if (k < 1 || k > shape->seq_len) return LD_ERR_INVALID_ARGUMENT;
  if (!workspace || workspace_bytes < H.total || ((uintptr_t)workspace & 15u)) return LD_ERR_WORKSPACE;
  char* ws = static_cast<char*>(workspace);
  const int Hq = shape->num_q_heads;
  const uint64_t all = (Hq == 64) ? ~0ull : ((1ull << Hq) - 1ull);
  float* o_w = reinterpret_cast<float*>(ws + H.o_w);
  // window branch first; the block-sparse launch mixes it in when it writes O
  WindowParams wp{};
  wp.q = static_cast<const uint16_t*>(q);
  wp.kw = static_cast<const uint16_t*>(k_window);
  wp.vw = static_cast<const uint16_t*>(v_window);
  wp.o = o_w;
  wp.B = shape->batch; wp.Hq = Hq; wp.Hkv = shape->num_kv_heads; wp.D = shape->head_dim;
  wp.W = window_len;
  wp.scale = shape->softmax_scale > 0.f ? shape->softmax_scale : 1.0f / std::sqrt((float)shape->head_dim);
  if (launch_window(wp, stream) != hipSuccess) return LD_ERR_HIP;
  return run_layer(shape, all, 0ull, q, k_cache, v_cache, k, s_in, nullptr, s_indptr, nullptr, out, flags,
                   false, ws + H.main, H.o_w - H.main, stream, gate, o_w);
}

}  // extern "C"

namespace {

// The TSA workspace: the selection's arrays, then the key splits' partials.
struct TsaLayout {
  size_t ml, o, total;
  int nsplit, split_keys;
};
TsaLayout tsa_layout(const ld_shape* s, int k) {
  TsaLayout L{};
  const int rows = s->batch * s->num_q_heads, kk = std::min(k, s->seq_len);
  size_t o = align_up(sel_layout(rows, s->seq_len).total);
  size_t part = 0;
  tsa_splits(rows, kk, s->head_dim, &L.nsplit, &L.split_keys, &part);
  const size_t ml_bytes = part / (size_t)(s->head_dim + 2) * 2;   // the (max, sum) pairs
  L.ml = o;
  o = align_up(o + ml_bytes);
  L.o = o;
  o = align_up(o + (part - ml_bytes));
  L.total = o;
  return L;
}

// Prefill layer workspace: the selection arrays of B*Hq rows of T scores, then the
// retrieval rows' log-sum-exp and column sums ([B*Hq][T] fp32 each).
struct PrefillLayout {
  SelLayout sel;
  size_t lse, imp, total;
};
PrefillLayout prefill_layout(const ld_shape* s) {
  PrefillLayout L{};
  const size_t rows = (size_t)s->batch * s->num_q_heads, T = (size_t)s->seq_len;
  L.sel = sel_layout((int)rows, s->seq_len);
  size_t o = align_up(L.sel.total);
  L.lse = o;
  o = align_up(o + rows * T * 4);
  L.imp = o;
  o = align_up(o + rows * T * 4);
  L.total = o;
  return L;
}

bool prefill_shape_ok(const ld_shape* s, ld_status* why) {
  if (!s) { *why = LD_ERR_INVALID_ARGUMENT; return false; }
  if (!shape_ok(s, why)) return false;
  // one contiguous bf16 layout of the prompt: no ragged batch, paging or 8-bit codes
  if (s->kv_indptr || s->page_size || s->kv_dtype) { *why = LD_ERR_UNSUPPORTED; return false; }
  if (s->total_tokens != 0 && s->total_tokens != (int64_t)s->batch * s->seq_len) {
    *why = LD_ERR_INVALID_ARGUMENT;
    return false;
  }
  return true;
}

}  // namespace

extern "C" {

size_t ld_prefill_workspace_size(const ld_shape* shape, int32_t k) {
  ld_status why;
  if (!prefill_shape_ok(shape, &why) || k < 1 || k > shape->seq_len) return 0;
  return prefill_layout(shape).total;
}

ld_status ld_prefill_hybrid_layer(const ld_shape* shape, uint64_t retrieval_mask, const void* q,
                                  const void* k_cache, const void* v_cache, int32_t k,
                                  const int32_t* s_in, int32_t* s_out, float* importance_out,
                                  void* out, uint32_t flags, void* workspace, size_t workspace_bytes,
                                  hipStream_t stream) {
  ld_status why;
  if (!prefill_shape_ok(shape, &why)) return why;
  const int B = shape->batch, Hq = shape->num_q_heads, D = shape->head_dim, T = shape->seq_len;
  const uint64_t all = (Hq == 64) ? ~0ull : ((1ull << Hq) - 1ull);
  if (retrieval_mask & ~all) return LD_ERR_INVALID_ARGUMENT;
  if (flags & ~(uint32_t)LD_FLAG_SKIP_TOPK) return LD_ERR_INVALID_ARGUMENT;
  if (!q || !k_cache || !v_cache || !out || k < 1 || k > T) return LD_ERR_INVALID_ARGUMENT;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out)) return LD_ERR_INVALID_ARGUMENT;
  if (((uintptr_t)s_in & 3u) || ((uintptr_t)s_out & 3u) || ((uintptr_t)importance_out & 3u))
    return LD_ERR_INVALID_ARGUMENT;
  const uint64_t sparse = all & ~retrieval_mask;
  const bool select = retrieval_mask && !(flags & LD_FLAG_SKIP_TOPK);
  if (sparse && !s_in) return LD_ERR_INVALID_ARGUMENT;
  if (select && !s_out) return LD_ERR_INVALID_ARGUMENT;
  const PrefillLayout L = prefill_layout(shape);
  if (!workspace || workspace_bytes < L.total || ((uintptr_t)workspace & 15u)) return LD_ERR_WORKSPACE;

  uint8_t sp_heads[64], ret_heads[64];
  int nsp = 0, nret = 0;
  for (int h = 0; h < Hq; ++h) {
    if (sparse >> h & 1ull) sp_heads[nsp++] = (uint8_t)h;
    if (retrieval_mask >> h & 1ull) ret_heads[nret++] = (uint8_t)h;
  }
  // 1. S^{l+1} = S^{l} for sparse heads when the output buffer is a different one
  if (nsp && s_out && s_out != s_in) {
    CopyParams cp{};
    cp.src = s_in; cp.dst = s_out; cp.s_indptr = nullptr; cp.k_dense = k; cp.s_cap = (int64_t)B * Hq * k;
    cp.Hq = Hq; cp.nsp = nsp;
    std::memcpy(cp.heads, sp_heads, sizeof(sp_heads));
    if (launch_copy_rows(cp, B * nsp, stream) != hipSuccess) return LD_ERR_HIP;
  }
  // 2. causal attention of every head (retrieval rows also leave their log-sum-exp)
  PrefillParams pp{};
  pp.q = static_cast<const uint16_t*>(q);
  pp.k = static_cast<const uint16_t*>(k_cache);
  pp.v = static_cast<const uint16_t*>(v_cache);
  pp.out = static_cast<uint16_t*>(out);
  pp.B = B; pp.Hq = Hq; pp.Hkv = shape->num_kv_heads; pp.D = D; pp.T = T;
  pp.qtiles = (T + prefill_rows_per_block() - 1) / prefill_rows_per_block();
  pp.retrieval = retrieval_mask;
  pp.s_in = s_in;
  pp.kk = k;
  pp.scale = shape->softmax_scale > 0.f ? shape->softmax_scale : 1.0f / std::sqrt((float)D);
  pp.lse = select ? at<float>(workspace, L.lse) : nullptr;
  pp.imp = importance_out ? importance_out : at<float>(workspace, L.imp);
  pp.nret = nret;
  std::memcpy(pp.heads, ret_heads, sizeof(ret_heads));
  if (launch_prefill_attention(pp, stream) != hipSuccess) return LD_ERR_HIP;
  if (!select) return LD_OK;
  // 3. column sums of the retrieval heads' attention matrices, then S = argsTopK of them
  if (launch_prefill_colsum(pp, stream) != hipSuccess) return LD_ERR_HIP;
  SelParams sp{};
  sp.mode = 1;
  sp.nrows = B * nret;
  set_hist_chunks(sp, sp.nrows, T);
  sp.logits = pp.imp; sp.Hq = Hq; sp.seq_len = T; sp.kv_indptr = nullptr;
  sp.s_out = s_out; sp.s_indptr = nullptr; sp.k_dense = k; sp.s_cap = (int64_t)B * Hq * k;
  sp.bitmaps = nullptr; sp.W = 0;
  sp.nret = nret;
  std::memcpy(sp.heads, ret_heads, sizeof(ret_heads));
  fill_sel(sp, L.sel.sel, workspace);
  return launch_select(sp, stream, true) == hipSuccess ? LD_OK : LD_ERR_HIP;
}

size_t ld_tsa_workspace_size(const ld_shape* shape, int32_t k) {
  ld_status why;
  if (!shape || !shape_ok(shape, &why) || shape->kv_indptr || shape->page_size || shape->kv_dtype || k < 1) return 0;
  return tsa_layout(shape, k).total;
}

ld_status ld_tsa_attention(const ld_shape* shape, const void* q, const void* k_cache,
                           const void* v_cache, const float* scores, int32_t k, int32_t* idx_out,
                           void* out, uint32_t flags, void* workspace, size_t workspace_bytes,
                           hipStream_t stream) {
  ld_status why;
  if (!shape) return LD_ERR_INVALID_ARGUMENT;
  if (!shape_ok(shape, &why)) return why;
  // one contiguous bf16 layout of the prefill: no ragged batch, paging or 8-bit codes
  if (shape->kv_indptr || shape->page_size || shape->kv_dtype) return LD_ERR_UNSUPPORTED;
  const int B = shape->batch, Hq = shape->num_q_heads, D = shape->head_dim, T = shape->seq_len;
  if (shape->total_tokens != 0 && shape->total_tokens != (int64_t)B * T) return LD_ERR_INVALID_ARGUMENT;
  const bool given = (flags & LD_TSA_GIVEN_IDX) != 0;
  if (!q || !k_cache || !v_cache || (!scores && !given) || !idx_out || !out || k < 1) return LD_ERR_INVALID_ARGUMENT;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out) ||
      ((uintptr_t)scores & 3u) || ((uintptr_t)idx_out & 3u))
    return LD_ERR_INVALID_ARGUMENT;
  if (flags & ~(uint32_t)(LD_TSA_CAUSAL | LD_TSA_ZERO_FILL | LD_TSA_GIVEN_IDX)) return LD_ERR_INVALID_ARGUMENT;
  const int rows = B * Hq;
  const SelLayout L = sel_layout(rows, T);
  const TsaLayout TL = tsa_layout(shape, k);
  if (!workspace || workspace_bytes < TL.total || ((uintptr_t)workspace & 15u)) return LD_ERR_WORKSPACE;
  const int kk = std::min(k, T);
  // 1. rows that receive no output are zero when asked for
  if ((flags & LD_TSA_ZERO_FILL) &&
      launch_zero(out, (size_t)Hq * B * T * D * 2, stream) != hipSuccess)
    return LD_ERR_HIP;
  // 2. compress: argsTopK of every head's scores (unless the caller gives the sets)
  if (!given) {
    SelParams sp{};
    sp.mode = 0;
    sp.nrows = rows;
    set_hist_chunks(sp, rows, T);
    sp.scores = scores; sp.row_stride = T; sp.n = T; sp.k = kk;
    sp.idx_out = idx_out; sp.val_out = nullptr;
    fill_sel(sp, L.sel, workspace);
    if (launch_select(sp, stream, true) != hipSuccess) return LD_ERR_HIP;
  }
  // 3. dense attention among the selected tokens, scattered to their rows
  TsaParams tp{};
  tp.q = static_cast<const uint16_t*>(q);
  tp.k = static_cast<const uint16_t*>(k_cache);
  tp.v = static_cast<const uint16_t*>(v_cache);
  tp.idx = idx_out;
  tp.out = static_cast<uint16_t*>(out);
  tp.B = B; tp.Hq = Hq; tp.Hkv = shape->num_kv_heads; tp.D = D; tp.T = T; tp.kk = kk;
  tp.qtiles = (kk + tsa_queries_per_block() - 1) / tsa_queries_per_block();
  tp.scale = shape->softmax_scale > 0.f ? shape->softmax_scale : 1.0f / std::sqrt((float)D);
  tp.causal = (flags & LD_TSA_CAUSAL) ? 1 : 0;
  tp.nsplit = TL.nsplit;
  tp.split_keys = TL.split_keys;
  tp.part_ml = at<float>(workspace, TL.ml);
  tp.part_o = at<float>(workspace, TL.o);
  return launch_tsa(tp, stream) == hipSuccess ? LD_OK : LD_ERR_HIP;
}

size_t ld_topk_workspace_size(int32_t rows, int32_t n) {
  if (rows < 1 || n < 1 || n > kMaxSeq) return 0;
  return sel_layout(rows, n).total;
}

ld_status ld_workspace_init(void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!workspace || workspace_bytes == 0) return LD_ERR_WORKSPACE;
  return launch_zero(workspace, workspace_bytes, stream) == hipSuccess ? LD_OK : LD_ERR_HIP;
}

ld_status ld_workspace_check(void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!workspace || workspace_bytes < kHeaderBytes || ((uintptr_t)workspace & 15u)) return LD_ERR_WORKSPACE;
  uint32_t flag = 0;
  if (hipMemcpyAsync(&flag, static_cast<char*>(workspace) + kErrOffset, sizeof(flag), hipMemcpyDeviceToHost,
                     stream) != hipSuccess)
    return LD_ERR_HIP;
  if (hipStreamSynchronize(stream) != hipSuccess) return LD_ERR_HIP;
  if (flag == 0) return LD_OK;
  if (launch_zero(workspace, 16, stream) != hipSuccess) return LD_ERR_HIP;
  return LD_ERR_DEVICE_WAIT;
}

ld_status ld_retrieval_decode(const ld_shape* shape, uint64_t head_mask, const void* q,
                              const void* k_cache, const void* v_cache, int32_t k,
                              int32_t* s_out, const int64_t* s_indptr, float* scores_out,
                              void* out, void* workspace, size_t workspace_bytes,
                              hipStream_t stream) {
  return run_layer(shape, head_mask, head_mask, q, k_cache, v_cache, k, nullptr, s_out, s_indptr,
                   scores_out, out, 0u, s_out != nullptr, workspace, workspace_bytes, stream);
}

ld_status ld_sparse_decode(const ld_shape* shape, uint64_t head_mask, const void* q,
                           const void* k_cache, const void* v_cache, int32_t k,
                           const int32_t* s_in, const int64_t* s_indptr, void* out,
                           uint32_t flags, void* workspace, size_t workspace_bytes,
                           hipStream_t stream) {
  if (head_mask && !s_in) return LD_ERR_INVALID_ARGUMENT;
  return run_layer(shape, head_mask, 0ull, q, k_cache, v_cache, k, s_in, nullptr, s_indptr,
                   nullptr, out, flags, false, workspace, workspace_bytes, stream);
}

ld_status ld_hybrid_layer(const ld_shape* shape, uint64_t retrieval_mask, const void* q,
                          const void* k_cache, const void* v_cache, int32_t k,
                          const int32_t* s_in, int32_t* s_out, const int64_t* s_indptr,
                          float* scores_out, void* out, uint32_t flags, void* workspace,
                          size_t workspace_bytes, hipStream_t stream) {
  ld_status why;
  if (!shape_ok(shape, &why)) return why;
  const int Hq = shape->num_q_heads;
  const uint64_t all = (Hq == 64) ? ~0ull : ((1ull << Hq) - 1ull);
  if (retrieval_mask & ~all) return LD_ERR_INVALID_ARGUMENT;
  return run_layer(shape, all, retrieval_mask, q, k_cache, v_cache, k, s_in, s_out, s_indptr,
                   scores_out, out, flags, !(flags & LD_FLAG_SKIP_TOPK), workspace,
                   workspace_bytes, stream);
}

ld_status ld_hybrid_layer_plan(const ld_shape* shape, uint64_t retrieval_mask, const void* q,
                               const void* k_cache, const void* v_cache, int32_t k,
                               const int32_t* s_in, int32_t* s_out, const int64_t* s_indptr,
                               float* scores_out, void* out, uint32_t flags, ld_layer_plan* plan) {
  if (!plan) return LD_ERR_INVALID_ARGUMENT;
  ld_status why;
  if (!shape_ok(shape, &why)) return why;
  const int Hq = shape->num_q_heads;
  const uint64_t all = (Hq == 64) ? ~0ull : ((1ull << Hq) - 1ull);
  if (retrieval_mask & ~all) return LD_ERR_INVALID_ARGUMENT;
  return run_layer(shape, all, retrieval_mask, q, k_cache, v_cache, k, s_in, s_out, s_indptr,
                   scores_out, out, flags, !(flags & LD_FLAG_SKIP_TOPK), nullptr, 0, nullptr,
                   nullptr, nullptr, false, plan);
}

ld_status ld_topk_select(const float* scores, int32_t rows, int32_t n, int64_t row_stride,
                         const int32_t* n_per_row, int32_t k, const int32_t* k_per_row, int32_t* idx_out,
                         const int64_t* idx_indptr, float* val_out, void* workspace,
                         size_t workspace_bytes, hipStream_t stream) {
  if (!scores || !idx_out || rows < 1 || n < 1 || n > kMaxSeq || k < 1 || row_stride < n)
    return LD_ERR_INVALID_ARGUMENT;
  if (((uintptr_t)scores & 3u) || ((uintptr_t)idx_out & 3u) || (val_out && ((uintptr_t)val_out & 3u)) ||
      ((uintptr_t)n_per_row & 3u) || ((uintptr_t)k_per_row & 3u) || ((uintptr_t)idx_indptr & 7u))
    return LD_ERR_INVALID_ARGUMENT;
  const SelLayout L = sel_layout(rows, n);
  if (!workspace || workspace_bytes < L.total || ((uintptr_t)workspace & 15u)) return LD_ERR_WORKSPACE;
  SelParams sp{};
  sp.mode = 0;
  sp.nrows = rows;
  set_hist_chunks(sp, rows, n);
  sp.scores = scores; sp.row_stride = row_stride; sp.n = n; sp.k = k;
  sp.idx_out = idx_out; sp.val_out = val_out;
  sp.n_per_row = n_per_row; sp.k_per_row = k_per_row; sp.idx_indptr = idx_indptr;
  fill_sel(sp, L.sel, workspace);
  return launch_select(sp, stream, true) == hipSuccess ? LD_OK : LD_ERR_HIP;
}

}  // extern "C"

// ---------------------------------------------------------------- allocation-free entry

namespace {

// Scratch of ld_hybrid_layer_noalloc: one copy per device, held until the process ends.
// Host code never uses the array's name as an address: each device's address comes
// from hipGetSymbolAddress (scratch_on_device).
static __device__ __align__(256) unsigned char scratch[LD_NOALLOC_SCRATCH_BYTES];

std::mutex g_scratch_mu;
void* g_scratch_ptr[64];

// Device address of the current device's scratch, looked up once per device.
ld_status scratch_on_device(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return LD_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return LD_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return LD_OK;
}

}  // namespace

extern "C" {

ld_status ld_hybrid_layer_noalloc(const ld_shape* shape, uint64_t retrieval_mask, const void* q,
                                  const void* k_cache, const void* v_cache, int32_t k,
                                  const int32_t* s_in, int32_t* s_out, const int64_t* s_indptr,
                                  float* scores_out, void* out, uint32_t flags, hipStream_t stream) {
  ld_status why;
  if (!shape_ok(shape, &why)) return why;
  const int Hq = shape->num_q_heads;
  const uint64_t all = (Hq == 64) ? ~0ull : ((1ull << Hq) - 1ull);
  if (retrieval_mask & ~all) return LD_ERR_INVALID_ARGUMENT;
  if (layer_layout(shape).total > (size_t)LD_NOALLOC_SCRATCH_BYTES) return LD_ERR_SCRATCH_LIMIT;
  void* ws = nullptr;
  if ((why = scratch_on_device(&ws)) != LD_OK) return why;
  return run_layer(shape, all, retrieval_mask, q, k_cache, v_cache, k, s_in, s_out, s_indptr, scores_out, out,
                   flags, !(flags & LD_FLAG_SKIP_TOPK), ws, (size_t)LD_NOALLOC_SCRATCH_BYTES, stream, nullptr,
                   nullptr, true);
}

}  // extern "C"
