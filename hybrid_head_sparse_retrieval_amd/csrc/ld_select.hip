// argsTopK on fp32 scores (LycheeDecode summary page, method step 3), plus the
// small helper kernels of the layer call (S -> membership bitmaps, S row copies,
// workspace fill).
//
// Selection is an exact three-digit radix select on order-preserving 32-bit keys
// (digit 1 = bits 31..21, digit 2 = bits 20..10, digit 3 = bits 9..0), over spans
// of 16384 scores, one 1024-thread workgroup per span:
//   1. digit-1 histogram of the row (fused into the attention kernel for retrieval
//      heads, or k_sel_hist over 512-score chunks for standalone rows);
//   2. k_sel_cand: each span sums the row's digit-1 histogram while its scores load and
//      picks the bin b1 holding the k-th largest key (the last span of the row clears
//      the histogram); it counts its keys above bin b1 and stores its keys of bin
//      b1 (the candidates) with their digit-2 histogram; the last span of the row
//      finds digit 2, then from the candidates digit 3 (threshold key T), the highest
//      kept index i_tie among the keys equal to T (ties go to lower indices) and the
//      number of kept keys of every span, hence each span's output offset;
//   3. k_sel_write: each span writes its kept indices (key > T, or key == T and
//      index <= i_tie) in ascending order at its offset, plus its membership bitmap
//      words.
// Only integer atomics are used, so the result is deterministic.

#include <atomic>

#include "ld_device.h"

namespace ld {

namespace {

struct RowView {
  const float* sc;
  int n, k;
  int32_t* out;
  float* vout;
  uint32_t* bm;
  int slot;
};

__device__ __forceinline__ RowView row_view(const SelParams& p, int r) {
  RowView v;
  if (p.mode == 0) {
    v.sc = p.scores + (int64_t)r * p.row_stride;
    v.n = p.n_per_row ? max(0, min(p.n_per_row[r], p.n)) : p.n;
    int k = p.k_per_row ? p.k_per_row[r] : p.k;
    int64_t o;
    if (p.idx_indptr) {
      o = p.idx_indptr[r];
      const int64_t cap = p.idx_indptr[r + 1] - o;
      k = (int)max((int64_t)0, min((int64_t)k, cap));
    } else {
      o = (int64_t)r * p.k;
      k = min(k, p.k);
    }
    v.k = max(0, min(k, v.n));              // the pages' clamp k = min(k, n)
    v.out = p.idx_out + o;
    v.vout = p.val_out ? p.val_out + o : nullptr;
    v.bm = nullptr;
    v.slot = r;
  } else {
    const int b = r / p.nret, h = p.heads[r % p.nret];
    const int slot = b * p.Hq + h;
    int n = p.kv_indptr ? (int)(p.kv_indptr[b + 1] - p.kv_indptr[b]) : p.seq_len;
    n = max(0, min(n, p.seq_len));
    int64_t so;
    int k;
    s_row(p.s_indptr, p.k_dense, p.s_cap, slot, &so, &k);
    v.sc = p.logits + (size_t)slot * p.seq_len;
    v.n = n;
    v.k = min(k, n);
    v.out = p.s_out + so;
    v.vout = nullptr;
    v.bm = p.bitmaps ? p.bitmaps + (size_t)slot * p.W : nullptr;
    v.slot = slot;
  }
  return v;
}

// ------------------------------------------------------------- digit-1 histogram

// Digit-1 counts of NB * 4 * kThreads scores from s (16-byte aligned): every load is
// issued before the first count, so the chunk waits for memory once.
template <int NB>
__device__ __forceinline__ void hist1_whole(const float* __restrict__ s, uint32_t* hist, int tid) {
  float4 x[NB];
#pragma unroll
  for (int u = 0; u < NB; ++u) x[u] = reinterpret_cast<const float4*>(s)[u * kThreads + tid];
#pragma unroll
  for (int u = 0; u < NB; ++u) {
    atomicAdd(&hist[score_key(x[u].x) >> 21], 1u);
    atomicAdd(&hist[score_key(x[u].y) >> 21], 1u);
    atomicAdd(&hist[score_key(x[u].z) >> 21], 1u);
    atomicAdd(&hist[score_key(x[u].w) >> 21], 1u);
  }
}

__global__ __launch_bounds__(kThreads) void k_sel_hist(const SelParams p) {
  __shared__ uint32_t hist[kHist1Bins];
  const int r = blockIdx.x / p.C, c = blockIdx.x % p.C;
  const RowView v = row_view(p, r);
  const int hc = p.hchunk;
  if (c * hc >= v.n || v.k < 1) return;
  const int tid = threadIdx.x;
  for (int i = tid; i < kHist1Bins; i += kThreads) hist[i] = 0;
  __syncthreads();
  const int lo = c * hc, hi = min(v.n, lo + hc);
  const float* s = v.sc + lo;
  constexpr int kVec = 4 * kThreads;   // scores per round of float4 loads
  if (hi - lo == hc && hc % kVec == 0 && (reinterpret_cast<uintptr_t>(s) & 15u) == 0) {
    // a whole chunk (hc is a power of two): rounds of up to 8 float4 loads per thread
    for (int j = 0; j < hc / kVec;) {
      const int left = hc / kVec - j;
      if (left >= 8) { hist1_whole<8>(s + j * kVec, hist, tid); j += 8; }
      else if (left >= 4) { hist1_whole<4>(s + j * kVec, hist, tid); j += 4; }
      else if (left >= 2) { hist1_whole<2>(s + j * kVec, hist, tid); j += 2; }
      else { hist1_whole<1>(s + j * kVec, hist, tid); j += 1; }
    }
  } else {
#pragma unroll 4
    for (int i = lo + tid; i < hi; i += kThreads) atomicAdd(&hist[score_key(v.sc[i]) >> 21], 1u);
  }
  __syncthreads();
  uint32_t* gh = hist1_mine(p.hist1, v.slot, p.hist_reps);
  for (int i = tid; i < kHist1Bins; i += kThreads)
    if (hist[i]) atomicAdd(gh + i, hist[i]);
}

// ------------------------------------------------ short standalone rows

// A standalone row of at most kSmallRow scores in one workgroup: the keys stay in
// registers (kSmallPer contiguous ones per thread), three digit histograms in LDS give
// the threshold key T and the number k3 of keys equal to T to keep (the lowest
// indices), and two workgroup scans place the kept indices in ascending order.
constexpr int kSmallThreads = 1024;
constexpr int kSmallPer = 4;
constexpr int kSmallRow = kSmallThreads * kSmallPer;

// Exclusive prefix of x over the workgroup (thread order); wsum: __shared__ int[16].
__device__ __forceinline__ int block_excl_scan(int x, int* wsum) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int wt;
  const int before = wave_excl_scan(x, wt);
  if (lane == 0) wsum[wave] = wt;
  __syncthreads();
  int off = 0;
#pragma unroll
  for (int w = 0; w < kSmallThreads / 64; ++w) off += (w < wave) ? wsum[w] : 0;
  __syncthreads();
  return off + before;
}

__global__ __launch_bounds__(kSmallThreads) void k_sel_small(const SelParams p) {
  __shared__ uint32_t hist[kHist1Bins];
  __shared__ int tmp[kSmallThreads / 64];
  __shared__ int wsum[kSmallThreads / 64];
  __shared__ uint32_t res[2];
  const int tid = threadIdx.x;
  const RowView v = row_view(p, blockIdx.x);
  if (v.n < 1 || v.k < 1) return;
  const int n = v.n;
  const uint32_t k = (uint32_t)v.k;
  uint32_t key[kSmallPer];
  bool in[kSmallPer];
#pragma unroll
  for (int e = 0; e < kSmallPer; ++e) {
    const int i = tid * kSmallPer + e;
    in[e] = i < n;
    key[e] = in[e] ? score_key(v.sc[i]) : 0u;
  }
  // digit i: the histogram of the keys that match the digits above, and the bin that
  // holds the k-th largest of them
  auto digit = [&](int nb, int shift, uint32_t mask, int pshift, uint32_t prefix, uint32_t kk, uint32_t* bin,
                   uint32_t* left) {
    for (int i = tid; i < nb; i += kSmallThreads) hist[i] = 0u;
    if (tid == 0) { res[0] = 0u; res[1] = 0u; }
    __syncthreads();
#pragma unroll
    for (int e = 0; e < kSmallPer; ++e)
      if (in[e] && (pshift >= 32 || (key[e] >> pshift) == prefix)) atomicAdd(&hist[(key[e] >> shift) & mask], 1u);
    __syncthreads();
    if (nb == kHist1Bins)
      find_bin_from_top<kHist1Bins, kSmallThreads>([&](int i) { return hist[i]; }, kk, tmp, res);
    else
      find_bin_from_top<kHist3Bins, kSmallThreads>([&](int i) { return hist[i]; }, kk, tmp, res);
    *bin = res[0];
    *left = kk - res[1];
    __syncthreads();
  };
  uint32_t b1, k1, b2, k2, b3, k3;
  digit(kHist1Bins, 21, 0x7ffu, 32, 0u, k, &b1, &k1);
  digit(kHist2Bins, 10, 0x7ffu, 21, b1, k1, &b2, &k2);
  digit(kHist3Bins, 0, 0x3ffu, 10, (b1 << 11) | b2, k2, &b3, &k3);
  const uint32_t T = (b1 << 21) | (b2 << 10) | b3;
  // keys equal to T before this thread's, then the kept keys before this thread's
  int eq = 0;
#pragma unroll
  for (int e = 0; e < kSmallPer; ++e) eq += (in[e] && key[e] == T) ? 1 : 0;
  int eq_before = block_excl_scan(eq, wsum);
  bool kf[kSmallPer];
  int kc = 0;
#pragma unroll
  for (int e = 0; e < kSmallPer; ++e) {
    const bool tie = in[e] && key[e] == T;
    kf[e] = in[e] && (key[e] > T || (tie && (uint32_t)eq_before < k3));
    eq_before += tie ? 1 : 0;
    kc += kf[e] ? 1 : 0;
  }
  int q = block_excl_scan(kc, wsum);
#pragma unroll
  for (int e = 0; e < kSmallPer; ++e) {
    if (kf[e]) {
      const int i = tid * kSmallPer + e;
      v.out[q] = i;
      if (v.vout) v.vout[q] = v.sc[i];
      ++q;
    }
  }
}

// ------------------------------------------------ spans of kSelSpan scores

constexpr int kSpanThreads = 1024;
constexpr int kSpanWaves = kSpanThreads / 64;
constexpr int kSpanRounds = kSelSpan / (4 * kSpanThreads);   // float4 loads per thread
constexpr int kFineCap = 4096;                                // fine candidates kept in LDS
constexpr int kSpecSlots = 4;                                 // candidates fetched early per thread
static_assert(kSpanRounds == 4, "one 16-bit lane mask per span");

// Keys of this thread's scores of span `base`: round r holds indices
// base + r*4096 + tid*4 + e; positions at or past n get key 0 (masked by index).
__device__ __forceinline__ void load_span(const float* __restrict__ sc, int n, int base, int tid,
                                          uint32_t (&key)[kSpanRounds][4]) {
  // workgroup-uniform test, so that the fast path issues every load before any wait
  const bool whole = base + kSelSpan <= n && (reinterpret_cast<uintptr_t>(sc + base) & 15u) == 0;
  if (whole) {
    float4 x[kSpanRounds];
#pragma unroll
    for (int r = 0; r < kSpanRounds; ++r)
      x[r] = *reinterpret_cast<const float4*>(sc + base + r * 4 * kSpanThreads + tid * 4);
#pragma unroll
    for (int r = 0; r < kSpanRounds; ++r) {
      key[r][0] = score_key(x[r].x); key[r][1] = score_key(x[r].y);
      key[r][2] = score_key(x[r].z); key[r][3] = score_key(x[r].w);
    }
  } else {
#pragma unroll
    for (int r = 0; r < kSpanRounds; ++r)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = base + r * 4 * kSpanThreads + tid * 4 + e;
        key[r][e] = (i < n) ? score_key(sc[i]) : 0u;
      }
  }
}

__device__ __forceinline__ int span_index(int base, int tid, int bit) {
  return base + (bit >> 2) * 4 * kSpanThreads + tid * 4 + (bit & 3);
}

__device__ __forceinline__ uint32_t span_key(const uint32_t (&key)[kSpanRounds][4], int bit) {
  uint32_t v = 0;
#pragma unroll
  for (int r = 0; r < kSpanRounds; ++r)
#pragma unroll
    for (int e = 0; e < 4; ++e) v = (bit == 4 * r + e) ? key[r][e] : v;
  return v;
}

__device__ __forceinline__ int wave_sum(int x) { return wave_total(x); }

struct SpanSmem {
  uint32_t hist[2048];
  uint64_t fine[kFineCap];           // (index << 32 | key) of keys in bins (b1, b2)
  uint32_t above[kMaxSelSpans];      // per span: keys above bin b1
  uint32_t ncd[kMaxSelSpans];        // per span: candidates
  uint32_t cnt2[kMaxSelSpans];       // per span: candidates above bin b2
  uint32_t cnt3[kMaxSelSpans];       // per span: kept keys of bin (b1, b2)
  int tmp[kSpanWaves];
  uint32_t res[2];
  uint32_t misc[4];                  // candidate count, above count, fine count
  uint64_t wtot[kSpanWaves];
  int flag;
};

// Pass over the candidates of a row (keys of bin b1 stored per span) from position
// `start` of each span on, spread over the 16 waves: f(key, index) per candidate, then
// done(span, wave total) once per wave and span with the wave-wide sum of what f
// returned.
template <typename F, typename Done>
__device__ __forceinline__ void for_candidates(const uint64_t* __restrict__ cand, const uint32_t* ncd, int nsp,
                                               int start, int lane, int wave, F f, Done done) {
  const int wpc = nsp >= kSpanWaves ? 1 : kSpanWaves / nsp;   // waves per span
  const int first = wave / wpc, slice = wave % wpc;
  for (int c = first; c < nsp; c += kSpanWaves / wpc) {
    const int cnt = (int)ncd[c];
    const uint64_t* cp = cand + (size_t)c * kSelSpan;
    int acc = 0;
    int q = start + slice * 64 + lane;
    for (; q + 3 * wpc * 64 < cnt; q += 4 * wpc * 64) {
      uint64_t x[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) x[u] = ld_dev(cp + q + u * wpc * 64);
#pragma unroll
      for (int u = 0; u < 4; ++u) acc += f((uint32_t)x[u], (uint32_t)(x[u] >> 32));
    }
    for (; q < cnt; q += wpc * 64) {
      const uint64_t x = ld_dev(cp + q);
      acc += f((uint32_t)x, (uint32_t)(x >> 32));
    }
    done(c, wave_sum(acc));
  }
}

// Phase 1 of a span: count its keys above bin b1, store its keys of bin b1 (the
// candidates, device-coherent) and add their digit-2 histogram to gh2; the span's
// two counts go to span_cnt. Every thread of the workgroup calls it.
__device__ __forceinline__ void span_candidates(const SelParams& p, int slot, int c, int n, uint32_t b1,
                                                const uint32_t (&key)[kSpanRounds][4], uint64_t* cand,
                                                uint32_t* gh2, SpanSmem& sm) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int base = c * kSelSpan;
  for (int i = tid; i < 2048; i += kSpanThreads) sm.hist[i] = 0;
  if (tid == 0) { sm.misc[0] = 0; sm.misc[1] = 0; }
  uint32_t cm = 0;
  int na = 0;
#pragma unroll
  for (int rr = 0; rr < kSpanRounds; ++rr)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bool in = base + rr * 4 * kSpanThreads + tid * 4 + e < n;
      const uint32_t d1 = key[rr][e] >> 21;
      na += (in && d1 > b1) ? 1 : 0;
      cm |= (uint32_t)(in && d1 == b1) << (4 * rr + e);
    }
  __syncthreads();
  int wtot;
  const int before = wave_excl_scan(__popc(cm), wtot);
  na = wave_sum(na);
  if (lane == 0) atomicAdd(&sm.misc[1], (uint32_t)na);
  if (wtot) {
    uint32_t wb = 0;
    if (lane == 0) wb = atomicAdd(&sm.misc[0], (uint32_t)wtot);
    uint32_t q = (uint32_t)__builtin_amdgcn_readlane((int)wb, 0) + (uint32_t)before;
    while (cm) {
      const int bit = __builtin_ctz(cm);
      cm &= cm - 1u;
      const uint32_t kv = span_key(key, bit);
      st_dev(cand + base + q, ((uint64_t)(uint32_t)span_index(base, tid, bit) << 32) | kv);
      ++q;
      atomicAdd(&sm.hist[(kv >> 10) & 0x7ffu], 1u);
    }
  }
  __syncthreads();
  for (int i = tid; i < 2048; i += kSpanThreads)
    if (sm.hist[i]) atomicAdd(gh2 + i, sm.hist[i]);
  if (tid == 0) {
    st_dev(p.span_cnt + ((size_t)slot * p.C + c) * 2 + 0, sm.misc[1]);
    st_dev(p.span_cnt + ((size_t)slot * p.C + c) * 2 + 1, sm.misc[0]);
  }
}

// Phase 2, once phase 1 of every span of the row is complete: digits 2 and 3 give
// the threshold key T; i_tie is the highest kept index among the keys equal to T
// (ties go to lower indices); sm.above/cnt2/cnt3 then hold the parts of each span's
// kept count. zero_hist: clear gh2 once read. Every thread of the workgroup calls it.
__device__ __forceinline__ void row_threshold(const SelParams& p, int slot, int nsp, uint32_t b1, uint32_t k1,
                                              uint32_t* gh2, bool zero_hist, const uint64_t* cand,
                                              SpanSmem& sm, uint32_t& T_out, uint32_t& i_tie_out) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) { sm.res[0] = 0; sm.res[1] = 0; sm.misc[2] = 0; }
  for (int i = tid; i < nsp; i += kSpanThreads) {
    sm.above[i] = ld_dev(p.span_cnt + ((size_t)slot * p.C + i) * 2 + 0);
    sm.ncd[i] = ld_dev(p.span_cnt + ((size_t)slot * p.C + i) * 2 + 1);
    sm.cnt2[i] = 0;
    sm.cnt3[i] = 0;
  }
  // digit-2 bins of this thread (the two that find_bin_from_top asks it for)
  const uint32_t h0 = ld_dev(gh2 + 2 * tid), h1 = ld_dev(gh2 + 2 * tid + 1);
  // the first `per` stored candidates of every span, fetched before their counts are
  // known (entries past a span's count are ignored); per is a multiple of 64, so the
  // lanes of a wave share one span
  const int per = nsp <= 64 ? ((kSpecSlots * kSpanThreads / nsp) / 64) * 64 : 0;
  uint64_t spec[kSpecSlots];
#pragma unroll
  for (int u = 0; u < kSpecSlots; ++u) {
    const int f = u * kSpanThreads + tid;
    const int c = per ? f / per : nsp;
    spec[u] = (c < nsp) ? ld_dev(cand + (size_t)c * kSelSpan + (f - c * per)) : 0ull;
  }
  __syncthreads();
  find_bin_from_top<2048, kSpanThreads>([&](int i) { return (i & 1) ? h1 : h0; }, k1, sm.tmp, sm.res);
  const uint32_t b2 = sm.res[0];
  const uint32_t k2 = k1 - sm.res[1];
  for (int i = tid; i < 2048; i += kSpanThreads) {
    if (zero_hist) gh2[i] = 0u;
    sm.hist[i] = 0u;
  }
  __syncthreads();

  // ---- candidates above bin b2 per span; digit-3 histogram and list of bin (b1, b2)
  auto visit = [&](uint32_t kv, uint32_t ix) -> int {
    const uint32_t d2 = (kv >> 10) & 0x7ffu;
    if (d2 == b2) {
      atomicAdd(&sm.hist[kv & 0x3ffu], 1u);
      const uint32_t f = atomicAdd(&sm.misc[2], 1u);
      if (f < (uint32_t)kFineCap) sm.fine[f] = ((uint64_t)ix << 32) | kv;
    }
    return d2 > b2 ? 1 : 0;
  };
#pragma unroll
  for (int u = 0; u < kSpecSlots; ++u) {
    const int f = u * kSpanThreads + tid;
    const int c = per ? f / per : nsp;            // wave-uniform
    if (c < nsp) {
      const int a = (f - c * per < (int)sm.ncd[c]) ? visit((uint32_t)spec[u], (uint32_t)(spec[u] >> 32)) : 0;
      const int tot = wave_sum(a);
      if (lane == 0 && tot) atomicAdd(&sm.cnt2[c], (uint32_t)tot);
    }
  }
  for_candidates(cand, sm.ncd, nsp, per, lane, wave, visit,
      [&](int cc, int tot) { if (lane == 0 && tot) atomicAdd(&sm.cnt2[cc], (uint32_t)tot); });
  if (tid == 0) { sm.res[0] = 0; sm.res[1] = 0; }
  __syncthreads();
  const uint32_t nfine = sm.misc[2];
  const bool fine_lds = nfine <= (uint32_t)kFineCap;
  find_bin_from_top<1024, kSpanThreads>([&](int i) { return sm.hist[i]; }, k2, sm.tmp, sm.res);
  const uint32_t b3 = sm.res[0];
  const uint32_t e_take = k2 - sm.res[1];         // keys equal to T that are kept
  const uint32_t nties = sm.hist[b3];
  const uint32_t T = (b1 << 21) | (b2 << 10) | b3;
  const uint32_t pre22 = T >> 10;
  __syncthreads();

  // every key of bin (b1, b2): from the LDS list, else from the stored candidates
  auto for_fine = [&](auto f) {
    if (fine_lds) {
      for (uint32_t q = tid; q < nfine; q += kSpanThreads) {
        const uint64_t x = sm.fine[q];
        f((uint32_t)x, (uint32_t)(x >> 32));
      }
    } else {
      for_candidates(cand, sm.ncd, nsp, 0, lane, wave,
          [&](uint32_t kv, uint32_t ix) -> int { if ((kv >> 10) == pre22) f(kv, ix); return 0; },
          [&](int, int) {});
    }
  };

  // ---- highest kept tie index: the e_take-th smallest index among keys == T
  uint32_t i_tie = 0x7fffffffu;
  if (e_take < nties) {
    // indices are < 2^21: digit A = bits 20..11 (1024 bins), digit B = bits 10..0
    for (int i = tid; i < 2048; i += kSpanThreads) sm.hist[i] = 0u;
    if (tid == 0) { sm.res[0] = 0; sm.res[1] = 0; }
    __syncthreads();
    for_fine([&](uint32_t kv, uint32_t ix) { if (kv == T) atomicAdd(&sm.hist[ix >> 11], 1u); });
    __syncthreads();
    find_bin_from_top<1024, kSpanThreads>([&](int i) { return sm.hist[1023 - i]; }, e_take, sm.tmp, sm.res);
    const uint32_t binA = 1023u - sm.res[0];
    const uint32_t eB = e_take - sm.res[1];
    __syncthreads();    // every wave has read the result before it is cleared
    for (int i = tid; i < 2048; i += kSpanThreads) sm.hist[i] = 0u;
    if (tid == 0) { sm.res[0] = 0; sm.res[1] = 0; }
    __syncthreads();
    for_fine([&](uint32_t kv, uint32_t ix) {
      if (kv == T && (ix >> 11) == binA) atomicAdd(&sm.hist[ix & 0x7ffu], 1u);
    });
    __syncthreads();
    find_bin_from_top<2048, kSpanThreads>([&](int i) { return sm.hist[2047 - i]; }, eB, sm.tmp, sm.res);
    i_tie = (binA << 11) | (2047u - sm.res[0]);
  }

  // ---- kept keys of bin (b1, b2) per span
  for_fine([&](uint32_t kv, uint32_t ix) {
    if (kv > T || (kv == T && ix <= i_tie)) atomicAdd(&sm.cnt3[ix / kSelSpan], 1u);
  });
  __syncthreads();
  T_out = T;
  i_tie_out = i_tie;
}

// Phase 3 of a span: its kept indices (key > T, or key == T and index <= i_tie) in
// ascending order from `off`, plus its membership bitmap words.
__device__ __forceinline__ void span_write(const SelParams& p, const RowView& v, int c, uint32_t T, uint32_t i_tie,
                                           int off, const uint32_t (&key)[kSpanRounds][4], SpanSmem& sm) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = v.n, kk = v.k;
  const int base = c * kSelSpan;
  uint32_t fm = 0;
#pragma unroll
  for (int rr = 0; rr < kSpanRounds; ++rr)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t ix = (uint32_t)(base + rr * 4 * kSpanThreads + tid * 4 + e);
      const uint32_t kv = key[rr][e];
      fm |= (uint32_t)(ix < (uint32_t)n && (kv > T || (kv == T && ix <= i_tie))) << (4 * rr + e);
    }
  // per-round counts packed in 16-bit fields (rounds 0, 1 and rounds 2, 3); inclusive
  // scans over the wave
  uint32_t c01 = 0, c23 = 0;
  c01 = (uint32_t)__popc(fm & 0xfu) | ((uint32_t)__popc((fm >> 4) & 0xfu) << 16);
  c23 = (uint32_t)__popc((fm >> 8) & 0xfu) | ((uint32_t)__popc((fm >> 12) & 0xfu) << 16);
  const uint32_t i01 = (uint32_t)wave_incl_sum((int)c01), i23 = (uint32_t)wave_incl_sum((int)c23);
  const uint64_t cnt = (uint64_t)c01 | ((uint64_t)c23 << 32);
  const uint64_t inc = (uint64_t)i01 | ((uint64_t)i23 << 32);
  if (lane == 63) sm.wtot[wave] = inc;
  __syncthreads();
  uint64_t below = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kSpanWaves; ++w) {
    const uint64_t t = sm.wtot[w];
    below += (w < wave) ? t : 0ull;
    all += t;
  }
  const uint64_t mine = below + inc - cnt;        // exclusive prefix, per round
  int run = off;
#pragma unroll
  for (int rr = 0; rr < kSpanRounds; ++rr) {
    const uint32_t nib = (fm >> (4 * rr)) & 0xfu;
    int j = run + (int)((mine >> (16 * rr)) & 0xffffu);
    const int i0 = base + rr * 4 * kSpanThreads + tid * 4;
    uint32_t m = nib;
    while (m) {
      const int e = __builtin_ctz(m);
      m &= m - 1u;
      if (j < kk) {
        v.out[j] = i0 + e;
        if (v.vout) v.vout[j] = v.sc[i0 + e];
      }
      ++j;
    }
    run += (int)((all >> (16 * rr)) & 0xffffu);
    if (v.bm) {                                  // 8 lanes x 4 bits = one 32-bit word
      // the 8 lanes' bits are disjoint, so their sum is their union
      const uint32_t w = (uint32_t)sum8_i((int)(nib << ((lane & 7) * 4)));
      const int wi = i0 >> 5;
      if ((lane & 7) == 0 && i0 < n && wi < p.W) v.bm[wi] = w;
    }
  }
}

// Output offset of span c from the per-span kept counts in sm (wave 0 scans them).
__device__ __forceinline__ int span_offsets(int nsp, SpanSmem& sm, uint32_t* off_out, int c_want) {
  const int tid = threadIdx.x, lane = tid & 63;
  if (tid < 64) {
    // lane l owns spans 2l and 2l+1 (at most 128 spans)
    int s0 = 0, s1 = 0;
    const int c0 = 2 * lane, c1 = 2 * lane + 1;
    if (c0 < nsp) s0 = (int)(sm.above[c0] + sm.cnt2[c0] + sm.cnt3[c0]);
    if (c1 < nsp) s1 = (int)(sm.above[c1] + sm.cnt2[c1] + sm.cnt3[c1]);
    int tot;
    const int pre = wave_excl_scan(s0 + s1, tot);
    if (off_out) {
      if (c0 < nsp) off_out[c0] = (uint32_t)pre;
      if (c1 < nsp) off_out[c1] = (uint32_t)(pre + s0);
    }
    if (c0 == c_want) sm.misc[3] = (uint32_t)pre;
    if (c1 == c_want) sm.misc[3] = (uint32_t)(pre + s0);
  }
  __syncthreads();
  return (int)sm.misc[3];
}

// Selection in two launches, which assumes nothing about how many of its workgroups the
// device holds at once: k_sel_cand, whose last span of a row runs phase 2 and stores T,
// i_tie and the span offsets, then k_sel_write.
__global__ __launch_bounds__(kSpanThreads) void k_sel_cand(const SelParams p) {
  __shared__ SpanSmem sm;
  const int r = blockIdx.x / p.C, c = blockIdx.x % p.C;
  const RowView v = row_view(p, r);
  const int n = v.n, kk = v.k;
  if (n < 1) return;
  if (kk < 1) {                                 // an empty row of a CSR S: nothing to keep,
    if (c == 0) hist1_clear(p.hist1, v.slot, p.hist_reps);   // but its histogram may hold counts
    return;
  }
  const int nsp = (n + kSelSpan - 1) / kSelSpan;
  if (c >= nsp) return;
  const int tid = threadIdx.x;
  const int slot = v.slot;
  uint64_t* cand = p.cand + (size_t)slot * p.ncap;
  uint32_t* gh2 = p.hist2 + (size_t)slot * kHist2Bins;
  uint32_t key[kSpanRounds][4];
  load_span(v.sc, n, c * kSelSpan, tid, key);
  // digit 1 from the row's histogram (the sum of its replicas), while the scores load
  hist1_sum<kSpanThreads>(sm.hist, p.hist1, slot, p.hist_reps);
  if (tid == 0) { sm.res[0] = 0; sm.res[1] = 0; }
  __syncthreads();
  find_bin_from_top<kHist1Bins, kSpanThreads>([&](int i) { return sm.hist[i]; }, (uint32_t)kk, sm.tmp, sm.res);
  const uint32_t b1 = sm.res[0];
  const uint32_t k1 = (uint32_t)kk - sm.res[1];
  span_candidates(p, slot, c, n, b1, key, cand, gh2, sm);   // (find_bin ends with a barrier)
  if (!arrive_last(p.tickets + slot, (uint32_t)nsp, &sm.flag)) return;
  if (tid == 0) p.tickets[slot] = 0u;
  hist1_clear(p.hist1, slot, p.hist_reps);      // every span has read it
  uint32_t T, i_tie;
  row_threshold(p, slot, nsp, b1, k1, gh2, true, cand, sm, T, i_tie);
  (void)span_offsets(nsp, sm, p.span_off + (size_t)slot * p.C, -1);
  if (tid == 0) {
    p.sel_info[slot * 2 + 0] = T;
    p.sel_info[slot * 2 + 1] = i_tie;
  }
}

__global__ __launch_bounds__(kSpanThreads) void k_sel_write(const SelParams p) {
  __shared__ SpanSmem sm;
  const int r = blockIdx.x / p.C, c = blockIdx.x % p.C;
  const RowView v = row_view(p, r);
  if (v.n < 1 || v.k < 1) return;
  const int nsp = (v.n + kSelSpan - 1) / kSelSpan;
  if (c >= nsp) return;
  const int slot = v.slot;
  const uint32_t T = p.sel_info[slot * 2 + 0];
  const uint32_t i_tie = p.sel_info[slot * 2 + 1];
  const int off = (int)p.span_off[(size_t)slot * p.C + c];
  uint32_t key[kSpanRounds][4];
  load_span(v.sc, v.n, c * kSelSpan, threadIdx.x, key);
  span_write(p, v, c, T, i_tie, off, key, sm);
}

// ---------------------------------------------------- S rows -> bitmaps

__global__ __launch_bounds__(kThreads) void k_bitmap_build(const BitmapParams p) {
  __shared__ uint32_t bits[kBitmapWordsPerBlock];
  const int r = blockIdx.x / p.wblocks, wb = blockIdx.x % p.wblocks;
  const int b = r / p.nsp, h = p.heads[r % p.nsp];
  const int slot = b * p.Hq + h;
  int n = p.kv_indptr ? (int)(p.kv_indptr[b + 1] - p.kv_indptr[b]) : p.seq_len;
  n = max(0, min(n, p.seq_len));
  const int nw = min(p.W, (n + 31) >> 5);
  const int w0 = wb * kBitmapWordsPerBlock;
  if (w0 >= nw) return;
  const int w1 = min(nw, w0 + kBitmapWordsPerBlock);
  int64_t so;
  int kk;
  s_row(p.s_indptr, p.k_dense, p.s_cap, slot, &so, &kk);
  const int tid = threadIdx.x;
  for (int i = tid; i < w1 - w0; i += kThreads) bits[i] = 0;
  __syncthreads();
  const int32_t* s = p.s + so;
  for (int i = tid; i < kk; i += kThreads) {
    const int x = s[i];
    if (x >= 0 && x < n) {
      const int w = x >> 5;
      if (w >= w0 && w < w1) atomicOr(&bits[w - w0], 1u << (x & 31));
    }
  }
  __syncthreads();
  uint32_t* out = p.bitmaps + (size_t)slot * p.W;
  for (int i = tid; i < w1 - w0; i += kThreads) out[w0 + i] = bits[i];
}

__global__ __launch_bounds__(kThreads) void k_copy_rows(const CopyParams p) {
  const int r = blockIdx.x;
  const int b = r / p.nsp, h = p.heads[r % p.nsp];
  const int slot = b * p.Hq + h;
  int64_t so;
  int kk;
  s_row(p.s_indptr, p.k_dense, p.s_cap, slot, &so, &kk);
  for (int i = threadIdx.x; i < kk; i += kThreads) p.dst[so + i] = p.src[so + i];
}

__global__ __launch_bounds__(kThreads) void k_zero(uint4* p16, size_t n16, uint8_t* tail, int ntail) {
  const size_t stride = (size_t)gridDim.x * kThreads;
  for (size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x; i < n16; i += stride)
    p16[i] = make_uint4(0, 0, 0, 0);
  if (blockIdx.x == 0 && (int)threadIdx.x < ntail) tail[threadIdx.x] = 0;
}

// ------------------------------------------------------- token-block selection

// One workgroup per retrieval row: S = the tokens of the kept blocks in ascending
// order, and the row's membership bitmap = exactly those tokens.
__global__ __launch_bounds__(kThreads) void k_block_expand(const BlockParams p) {
  const int r = blockIdx.x;
  const int b = r / p.nret, h = p.heads[r % p.nret];
  const int slot = b * p.Hq + h;
  const int32_t* kept = p.kept + (size_t)r * p.kblk;
  int32_t* out = p.s_out + (size_t)slot * p.k_dense;
  for (int i = threadIdx.x; i < p.kblk * kBlock; i += kThreads) out[i] = kept[i / kBlock] * kBlock + (i % kBlock);
  if (p.bitmaps) {
    uint32_t* bm = p.bitmaps + (size_t)slot * p.W;
    for (int w = threadIdx.x; w < p.W; w += kThreads) bm[w] = 0u;
    __syncthreads();
    for (int i = threadIdx.x; i < p.kblk; i += kThreads) {
      const int w0 = kept[i] * (kBlock / 32);
#pragma unroll
      for (int q = 0; q < kBlock / 32; ++q)
        if (w0 + q < p.W) bm[w0 + q] = 0xffffffffu;
    }
  }
}

}  // namespace

hipError_t launch_block_expand(const BlockParams& p, int rows, hipStream_t st) {
  hipLaunchKernelGGL(k_block_expand, dim3((unsigned)rows), dim3(kThreads), 0, st, p);
  return hipGetLastError();
}

constexpr int kHistOneRepChunks = 16;   // histogram workgroups per row that share one replica

int select_launches(const SelParams& p, bool with_hist) {
  if (with_hist && p.mode == 0 && p.n <= kSmallRow) return 1;
  return (with_hist ? 1 : 0) + 2;
}

hipError_t launch_select(const SelParams& p, hipStream_t st, bool with_hist) {
  if (with_hist && p.mode == 0 && p.n <= kSmallRow) {
    hipLaunchKernelGGL(k_sel_small, dim3((unsigned)p.nrows), dim3(kSmallThreads), 0, st, p);
    return hipGetLastError();
  }
  // The histogram launch spreads a row's counts over replicas only when many of its
  // workgroups share the row (their atomics would meet on the same bins); with a few, one
  // replica is enough, and the candidate launch then sums one instead of kRep. The
  // attention launch's fused histogram always uses kRep.
  SelParams q = p;
  q.hist_reps = (with_hist && p.Ch <= kHistOneRepChunks) ? 1 : kRep;
  if (with_hist) {
    SelParams ph = q;
    ph.C = p.Ch;
    hipLaunchKernelGGL(k_sel_hist, dim3((unsigned)p.nrows * (unsigned)p.Ch), dim3(kThreads), 0, st, ph);
  }
  const dim3 grid((unsigned)p.nrows * (unsigned)p.C);
  hipLaunchKernelGGL(k_sel_cand, grid, dim3(kSpanThreads), 0, st, q);
  hipLaunchKernelGGL(k_sel_write, grid, dim3(kSpanThreads), 0, st, q);
  return hipGetLastError();
}

hipError_t launch_bitmap_build(const BitmapParams& p, int rows, hipStream_t st) {
  hipLaunchKernelGGL(k_bitmap_build, dim3((unsigned)(rows * p.wblocks)), dim3(kThreads), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_copy_rows(const CopyParams& p, int rows, hipStream_t st) {
  hipLaunchKernelGGL(k_copy_rows, dim3((unsigned)rows), dim3(kThreads), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_zero(void* ptr, size_t bytes, hipStream_t st) {
  const size_t n16 = bytes / 16;
  const int ntail = (int)(bytes - n16 * 16);
  size_t blocks = (n16 + kThreads - 1) / kThreads;
  if (blocks > 4096) blocks = 4096;
  if (blocks == 0) blocks = 1;
  hipLaunchKernelGGL(k_zero, dim3((unsigned)blocks), dim3(kThreads), 0, st,
                     reinterpret_cast<uint4*>(ptr), n16, reinterpret_cast<uint8_t*>(ptr) + n16 * 16, ntail);
  return hipGetLastError();
}

}  // namespace ld
