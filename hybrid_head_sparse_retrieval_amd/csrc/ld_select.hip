// argsTopK on fp32 scores (LycheeDecode summary page, method step 3), plus the
// small helper kernels of the layer call (S -> membership bitmaps, S row copies,
// workspace fill).
//
// Selection is an exact three-digit radix select on order-preserving 32-bit keys
// (digit 1 = bits 31..21, digit 2 = bits 20..10, digit 3 = bits 9..0):
//   1. digit-1 histogram of the row (fused into the attention kernel for retrieval
//      heads, or k_sel_hist over 512-score chunks for standalone rows); the last
//      workgroup of the row picks the bin b1 holding the k-th largest key;
//   2. k_topk_row, one 1024-thread workgroup per row: the keys of bin b1 (the
//      candidates) go to LDS with their digit-2 histogram; digits 2 and 3 give the
//      exact threshold key T and the highest index i_tie among the keys equal to T
//      that are kept (ties go to lower indices); every wave then writes its selected
//      indices (key > T, or key == T and index <= i_tie) in ascending order at its
//      offset from one scan over the wave totals, plus the membership bitmap words.
// Each wave reads 2048 consecutive scores per 32768-score segment in coalesced 1 KB
// loads; a row of one segment stays in registers between the passes, longer rows
// are re-read. Only integer atomics are used, so the result is deterministic.

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
    v.n = p.n;
    v.k = p.k;
    v.out = p.idx_out + (int64_t)r * p.k;
    v.vout = p.val_out ? p.val_out + (int64_t)r * p.k : nullptr;
    v.bm = nullptr;
    v.slot = r;
  } else {
    const int b = r / p.nret, h = p.heads[r % p.nret];
    const int slot = b * p.Hq + h;
    int n = p.kv_indptr ? (int)(p.kv_indptr[b + 1] - p.kv_indptr[b]) : p.seq_len;
    n = max(0, min(n, p.seq_len));
    int64_t so;
    int k;
    if (p.s_indptr) {
      so = p.s_indptr[slot];
      k = (int)(p.s_indptr[slot + 1] - so);
    } else {
      so = (int64_t)slot * p.k_dense;
      k = p.k_dense;
    }
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

__global__ __launch_bounds__(kThreads) void k_sel_hist(const SelParams p) {
  __shared__ uint32_t hist[kHist1Bins];
  __shared__ int tmp[4];
  __shared__ uint32_t res[2];
  __shared__ int flag;
  const int r = blockIdx.x / p.C, c = blockIdx.x % p.C;
  const RowView v = row_view(p, r);
  if (c * kSelChunk >= v.n || v.k < 1) return;
  const int tid = threadIdx.x;
  for (int i = tid; i < kHist1Bins; i += kThreads) hist[i] = 0;
  __syncthreads();
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int i = c * kSelChunk + h * kThreads + tid;
    if (i < v.n) atomicAdd(&hist[score_key(v.sc[i]) >> 21], 1u);
  }
  __syncthreads();
  uint32_t* gh = p.hist1 + (size_t)v.slot * kHist1Bins;
  for (int i = tid; i < kHist1Bins; i += kThreads)
    if (hist[i]) atomicAdd(gh + i, hist[i]);
  const uint32_t nch = (uint32_t)((v.n + kSelChunk - 1) / kSelChunk);
  if (!arrive_last(p.tickets + v.slot, nch, &flag)) return;
  if (tid == 0) { res[0] = 0; res[1] = 0; p.tickets[v.slot] = 0; }
  __syncthreads();
  find_bin_from_top<kHist1Bins, kThreads>([&](int i) { return ld_dev(gh + i); }, (uint32_t)v.k, tmp, res);
  if (tid == 0) {
    p.sel_info[v.slot * 4 + 0] = res[0];
    p.sel_info[v.slot * 4 + 1] = (uint32_t)v.k - res[1];
  }
  for (int i = tid; i < kHist1Bins; i += kThreads) gh[i] = 0u;
}

// ------------------------------------------------- one workgroup per row

constexpr int kRowThreads = 1024;
constexpr int kRowWaves = kRowThreads / 64;
constexpr int kRounds = 8;                      // 256-score rounds per wave per segment
constexpr int kWaveSpan = kRounds * 256;        // 2048 scores per wave per segment
constexpr int kSeg = kRowWaves * kWaveSpan;     // 32768 scores per segment
constexpr int kCandCap = 8192;                  // candidates kept in LDS

// Keys of this lane's scores of one segment: round r holds indices
// wbase + r*256 + lane*4 + e; positions past the row end get key 0 (masked by index).
__device__ __forceinline__ void load_keys(const float* __restrict__ sc, int n, int wbase, int lane,
                                          uint32_t (&key)[kRounds][4]) {
  // wave-uniform test, so that the fast path issues every load before any wait
  const bool whole = wbase + kWaveSpan <= n && (reinterpret_cast<uintptr_t>(sc + wbase) & 15u) == 0;
  if (whole) {
    float4 x[kRounds];
#pragma unroll
    for (int r = 0; r < kRounds; ++r) x[r] = *reinterpret_cast<const float4*>(sc + wbase + r * 256 + lane * 4);
#pragma unroll
    for (int r = 0; r < kRounds; ++r) {
      key[r][0] = score_key(x[r].x); key[r][1] = score_key(x[r].y);
      key[r][2] = score_key(x[r].z); key[r][3] = score_key(x[r].w);
    }
  } else {
#pragma unroll
    for (int r = 0; r < kRounds; ++r)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = wbase + r * 256 + lane * 4 + e;
        key[r][e] = (i < n) ? score_key(sc[i]) : 0u;
      }
  }
}

// Bit (4r + e) set for the keys of this lane that satisfy the predicate.
template <typename P>
__device__ __forceinline__ uint32_t key_mask(const uint32_t (&key)[kRounds][4], int wbase, int lane, int n,
                                             P pred) {
  uint32_t m = 0;
#pragma unroll
  for (int r = 0; r < kRounds; ++r)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = wbase + r * 256 + lane * 4 + e;
      m |= (uint32_t)(i < n && pred(key[r][e], (uint32_t)i)) << (4 * r + e);
    }
  return m;
}

__device__ __forceinline__ uint32_t key_at(const uint32_t (&key)[kRounds][4], int bit) {
  uint32_t v = 0;
#pragma unroll
  for (int r = 0; r < kRounds; ++r)
#pragma unroll
    for (int e = 0; e < 4; ++e) v = (bit == 4 * r + e) ? key[r][e] : v;
  return v;
}

__device__ __forceinline__ int wave_excl_scan(int x, int lane, int& total) {
  int v = x;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(v, o, 64);
    if (lane >= o) v += y;
  }
  total = __shfl(v, 63, 64);
  return v - x;
}

struct RowSmem {
  uint32_t hist[2048];
  uint32_t ckey[kCandCap];
  uint32_t cidx[kCandCap];
  int tmp[kRowWaves];
  uint32_t res[2];
  uint32_t ncand;
};

__global__ __launch_bounds__(kRowThreads) void k_topk_row(const SelParams p) {
  __shared__ RowSmem sm;
  const RowView v = row_view(p, blockIdx.x);
  const int n = v.n, kk = v.k;
  if (n < 1 || kk < 1) return;
  const float* __restrict__ sc = v.sc;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int slot = v.slot;
  const uint32_t b1 = p.sel_info[slot * 4 + 0];
  const uint32_t k1 = p.sel_info[slot * 4 + 1];
  const int nseg = (n + kSeg - 1) / kSeg;

  uint32_t key[kRounds][4];

  // ---- pass 1: candidates of bin b1 (LDS) and their digit-2 histogram
  for (int i = tid; i < 2048; i += kRowThreads) sm.hist[i] = 0;
  if (tid == 0) sm.ncand = 0;
  __syncthreads();
  for (int sg = 0; sg < nseg; ++sg) {
    const int wbase = sg * kSeg + wave * kWaveSpan;
    load_keys(sc, n, wbase, lane, key);
    uint32_t cm = key_mask(key, wbase, lane, n, [&](uint32_t kv, uint32_t) { return (kv >> 21) == b1; });
    int wtot;
    const int before = wave_excl_scan(__popc(cm), lane, wtot);
    if (wtot) {
      uint32_t wb = 0;
      if (lane == 0) wb = atomicAdd(&sm.ncand, (uint32_t)wtot);
      uint32_t q = __shfl(wb, 0, 64) + (uint32_t)before;
      while (cm) {
        const int bit = __builtin_ctz(cm);
        cm &= cm - 1u;
        const uint32_t kv = key_at(key, bit);
        if (q < (uint32_t)kCandCap) {
          sm.ckey[q] = kv;
          sm.cidx[q] = (uint32_t)(wbase + (bit >> 2) * 256 + lane * 4 + (bit & 3));
        }
        ++q;
        atomicAdd(&sm.hist[(kv >> 10) & 0x7ffu], 1u);
      }
    }
  }
  if (tid == 0) { sm.res[0] = 0; sm.res[1] = 0; }
  __syncthreads();
  const uint32_t ncand = sm.ncand;
  const bool in_lds = ncand <= (uint32_t)kCandCap;
  find_bin_from_top<2048, kRowThreads>([&](int i) { return sm.hist[i]; }, k1, sm.tmp, sm.res);
  const uint32_t b2 = sm.res[0];
  const uint32_t k2 = k1 - sm.res[1];

  // candidate histograms: mode 0 digit 3 of bin (b1, b2); 1 index bits 20..11 of keys
  // == T; 2 index bits 10..0 of keys == T in index bin binA
  auto cand_hist = [&](int mode, uint32_t T, uint32_t binA) {
    for (int i = tid; i < 2048; i += kRowThreads) sm.hist[i] = 0;
    if (tid == 0) { sm.res[0] = 0; sm.res[1] = 0; }
    __syncthreads();
    auto one = [&](uint32_t kv, uint32_t ix) {
      if (mode == 0) { if (((kv >> 10) & 0x7ffu) == b2) atomicAdd(&sm.hist[kv & 0x3ffu], 1u); }
      else if (mode == 1) { if (kv == T) atomicAdd(&sm.hist[ix >> 11], 1u); }
      else { if (kv == T && (ix >> 11) == binA) atomicAdd(&sm.hist[ix & 0x7ffu], 1u); }
    };
    if (in_lds) {
      for (uint32_t q = tid; q < ncand; q += kRowThreads) one(sm.ckey[q], sm.cidx[q]);
    } else {
      // a one-segment row is still in registers; longer rows are re-read
      for (int sg = 0; sg < nseg; ++sg) {
        const int wbase = sg * kSeg + wave * kWaveSpan;
        if (nseg > 1) load_keys(sc, n, wbase, lane, key);
        uint32_t cm = key_mask(key, wbase, lane, n, [&](uint32_t kv, uint32_t) { return (kv >> 21) == b1; });
        while (cm) {
          const int bit = __builtin_ctz(cm);
          cm &= cm - 1u;
          one(key_at(key, bit), (uint32_t)(wbase + (bit >> 2) * 256 + lane * 4 + (bit & 3)));
        }
      }
    }
    __syncthreads();
  };

  // ---- digit 3
  __syncthreads();
  cand_hist(0, 0u, 0u);
  find_bin_from_top<1024, kRowThreads>([&](int i) { return sm.hist[i]; }, k2, sm.tmp, sm.res);
  const uint32_t b3 = sm.res[0];
  const uint32_t e_take = k2 - sm.res[1];       // keys equal to T that are kept
  const uint32_t nties = sm.hist[b3];
  const uint32_t T = (b1 << 21) | (b2 << 10) | b3;
  __syncthreads();

  // ---- highest kept tie index: the e_take-th smallest index among keys == T
  uint32_t i_tie = 0x7fffffffu;
  if (e_take < nties) {
    // indices are < 2^21: digit A = bits 20..11 (1024 bins), digit B = bits 10..0
    cand_hist(1, T, 0u);
    find_bin_from_top<1024, kRowThreads>([&](int i) { return sm.hist[1023 - i]; }, e_take, sm.tmp, sm.res);
    const uint32_t binA = 1023u - sm.res[0];
    const uint32_t eB = e_take - sm.res[1];
    __syncthreads();
    cand_hist(2, T, binA);
    find_bin_from_top<2048, kRowThreads>([&](int i) { return sm.hist[2047 - i]; }, eB, sm.tmp, sm.res);
    i_tie = (binA << 11) | (2047u - sm.res[0]);
    __syncthreads();
  }

  // ---- pass 3: ascending write of the selected indices and the bitmap words
  int run = 0;
  for (int sg = 0; sg < nseg; ++sg) {
    const int wbase = sg * kSeg + wave * kWaveSpan;
    if (nseg > 1) load_keys(sc, n, wbase, lane, key);
    const uint32_t fm = key_mask(key, wbase, lane, n, [&](uint32_t kv, uint32_t ix) {
      return kv > T || (kv == T && ix <= i_tie);
    });
    // waves hold consecutive index blocks: exclusive scan of the wave totals
    int wtot;
    (void)wave_excl_scan(__popc(fm), lane, wtot);
    if (lane == 0) sm.tmp[wave] = wtot;
    __syncthreads();
    int woff = 0, stot = 0;
#pragma unroll
    for (int w = 0; w < kRowWaves; ++w) {
      woff += (w < wave) ? sm.tmp[w] : 0;
      stot += sm.tmp[w];
    }
    __syncthreads();
    int pos = run + woff;
#pragma unroll
    for (int r = 0; r < kRounds; ++r) {
      const uint32_t nib = (fm >> (4 * r)) & 0xfu;
      int rtot;
      const int before = wave_excl_scan(__popc(nib), lane, rtot);
      int j = pos + before;
      const int i0 = wbase + r * 256 + lane * 4;
      uint32_t m = nib;
      while (m) {
        const int e = __builtin_ctz(m);
        m &= m - 1u;
        if (j < kk) {
          v.out[j] = i0 + e;
          if (v.vout) v.vout[j] = sc[i0 + e];
        }
        ++j;
      }
      pos += rtot;
      if (v.bm) {                               // 8 lanes x 4 bits = one 32-bit word
        uint32_t w = nib << ((lane & 7) * 4);
        w |= __shfl_xor(w, 1, 64);
        w |= __shfl_xor(w, 2, 64);
        w |= __shfl_xor(w, 4, 64);
        const int wi = i0 >> 5;
        if ((lane & 7) == 0 && i0 < n && wi < p.W) v.bm[wi] = w;
      }
    }
    run += stot;
  }
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
  if (p.s_indptr) {
    so = p.s_indptr[slot];
    kk = (int)(p.s_indptr[slot + 1] - so);
  } else {
    so = (int64_t)slot * p.k_dense;
    kk = p.k_dense;
  }
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
  if (p.s_indptr) {
    so = p.s_indptr[slot];
    kk = (int)(p.s_indptr[slot + 1] - so);
  } else {
    so = (int64_t)slot * p.k_dense;
    kk = p.k_dense;
  }
  for (int i = threadIdx.x; i < kk; i += kThreads) p.dst[so + i] = p.src[so + i];
}

__global__ __launch_bounds__(kThreads) void k_zero(uint4* p16, size_t n16, uint8_t* tail, int ntail) {
  const size_t stride = (size_t)gridDim.x * kThreads;
  for (size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x; i < n16; i += stride)
    p16[i] = make_uint4(0, 0, 0, 0);
  if (blockIdx.x == 0 && (int)threadIdx.x < ntail) tail[threadIdx.x] = 0;
}

}  // namespace

hipError_t launch_select(const SelParams& p, hipStream_t st, bool with_hist) {
  if (with_hist) {
    SelParams ph = p;
    ph.C = p.Ch;
    hipLaunchKernelGGL(k_sel_hist, dim3((unsigned)p.nrows * (unsigned)p.Ch), dim3(kThreads), 0, st, ph);
  }
  hipLaunchKernelGGL(k_topk_row, dim3((unsigned)p.nrows), dim3(kRowThreads), 0, st, p);
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
