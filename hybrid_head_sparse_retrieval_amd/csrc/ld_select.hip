// argsTopK on fp32 scores (LycheeDecode summary page, method step 3), plus the
// small helper kernels of the layer call (S -> membership bitmaps, S row copies,
// workspace fill).
//
// Selection is an exact three-digit radix select on order-preserving 32-bit keys
// (digit 1 = bits 31..21, digit 2 = bits 20..10, digit 3 = bits 9..0) spread over
// many workgroups, one per 512-score chunk of a row:
//   1. digit-1 histogram of the row (fused into the attention kernel for retrieval
//      heads, or k_sel_hist for standalone rows); the last workgroup of the row picks
//      the bin b1 holding the k-th largest key;
//   2. k_sel_cand: every chunk counts its keys above bin b1 and appends the keys of
//      bin b1 (the candidates) to a per-row list, plus a digit-2 histogram of them;
//      the last chunk workgroup of the row resolves digits 2 and 3 on the candidates,
//      giving the exact threshold key T, and the highest index i_tie among the keys
//      equal to T that are kept (ties go to lower indices), then the output offset of
//      every chunk;
//   3. k_sel_write: every chunk writes its selected indices (key > T, or key == T and
//      index <= i_tie) in ascending order at its offset, and its membership bitmap.
// Only integer atomics are used, so the result is deterministic.

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

// Arrive at the row's ticket; returns true in every thread of the last workgroup.
__device__ __forceinline__ bool arrive_last(uint32_t* ticket, uint32_t target, int* flag) {
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t old = __hip_atomic_fetch_add(ticket, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    *flag = (old == target - 1u);
  }
  __syncthreads();
  const bool last = *flag != 0;
  if (last) __threadfence();
  return last;
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
  find_bin_from_top<kHist1Bins / kThreads>([&](int i) { return gh[i]; }, (uint32_t)v.k, tmp, res);
  if (tid == 0) {
    p.sel_info[v.slot * 4 + 0] = res[0];
    p.sel_info[v.slot * 4 + 1] = (uint32_t)v.k - res[1];
  }
  for (int i = tid; i < kHist1Bins; i += kThreads) gh[i] = 0u;
}

// ------------------------------------------------- candidates + exact threshold

constexpr int kResolveLds = kMaxSelChunks;   // 4096 words, reused by every phase

__global__ __launch_bounds__(kThreads) void k_sel_cand(const SelParams p) {
  __shared__ uint32_t buf[kResolveLds];
  __shared__ int tmp[4];
  __shared__ uint32_t res[2];
  __shared__ int flag;
  __shared__ uint32_t base_s;
  const int r = blockIdx.x / p.C, c = blockIdx.x % p.C;
  const RowView v = row_view(p, r);
  if (c * kSelChunk >= v.n || v.k < 1) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int slot = v.slot;
  const uint32_t b1 = p.sel_info[slot * 4 + 0];

  uint32_t key[2];
  bool gt[2], cand[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int i = c * kSelChunk + h * kThreads + tid;
    const bool valid = i < v.n;
    key[h] = valid ? score_key(v.sc[i]) : 0u;
    gt[h] = valid && (key[h] >> 21) > b1;
    cand[h] = valid && (key[h] >> 21) == b1;
  }
  int ngt_total;
  block_excl_scan((int)gt[0] + (int)gt[1], tmp, ngt_total);
  int ncand_total;
  const int cpos = block_excl_scan((int)cand[0] + (int)cand[1], tmp, ncand_total);
  if (tid == 0) {
    base_s = ncand_total ? atomicAdd(p.cand_count + slot, (uint32_t)ncand_total) : 0u;
    p.chunk_cnt[((size_t)slot * p.C + c) * 2 + 0] = (uint32_t)ngt_total;
  }
  __syncthreads();
  {
    int q = (int)base_s + cpos;
    uint32_t* ck = p.cand_key + (size_t)slot * p.ncap;
    int32_t* ci = p.cand_idx + (size_t)slot * p.ncap;
    uint32_t* h2 = p.hist2 + (size_t)slot * kHist2Bins;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (cand[h] && q < p.ncap) {
        ck[q] = key[h];
        ci[q] = c * kSelChunk + h * kThreads + tid;
        atomicAdd(h2 + ((key[h] >> 10) & 0x7ffu), 1u);
        ++q;
      }
    }
  }
  (void)lane;
  const uint32_t nch = (uint32_t)((v.n + kSelChunk - 1) / kSelChunk);
  if (!arrive_last(p.tickets + slot, nch, &flag)) return;

  // ---------------- last chunk workgroup of the row: resolve the threshold
  const int M = (int)min((int64_t)p.cand_count[slot], p.ncap);
  const uint32_t k1 = p.sel_info[slot * 4 + 1];
  const uint32_t* ck = p.cand_key + (size_t)slot * p.ncap;
  const int32_t* ci = p.cand_idx + (size_t)slot * p.ncap;
  uint32_t* h2 = p.hist2 + (size_t)slot * kHist2Bins;
  if (tid == 0) { res[0] = 0; res[1] = 0; p.tickets[slot] = 0; }
  __syncthreads();
  find_bin_from_top<kHist2Bins / kThreads>([&](int i) { return h2[i]; }, k1, tmp, res);
  const uint32_t b2 = res[0];
  const uint32_t k2 = k1 - res[1];
  for (int i = tid; i < kHist2Bins; i += kThreads) h2[i] = 0u;
  // digit 3 over candidates in bin (b1, b2)
  for (int i = tid; i < kHist3Bins; i += kThreads) buf[i] = 0;
  __syncthreads();
  for (int q = tid; q < M; q += kThreads) {
    const uint32_t kk = ck[q];
    if (((kk >> 10) & 0x7ffu) == b2) atomicAdd(&buf[kk & 0x3ffu], 1u);
  }
  __syncthreads();
  if (tid == 0) { res[0] = 0; res[1] = 0; }
  __syncthreads();
  find_bin_from_top<kHist3Bins / kThreads>([&](int i) { return buf[i]; }, k2, tmp, res);
  const uint32_t b3 = res[0];
  const uint32_t e_take = k2 - res[1];          // keys equal to T that are kept
  const uint32_t nties = buf[b3];
  const uint32_t T = (b1 << 21) | (b2 << 10) | b3;
  __syncthreads();
  // highest kept tie index: the e_take-th smallest index among keys == T
  uint32_t i_tie = 0x7fffffffu;
  if (e_take < nties) {
    // indices are < 2^22: digit A = bits 21..11, digit B = bits 10..0
    for (int i = tid; i < 2048; i += kThreads) buf[i] = 0;
    __syncthreads();
    for (int q = tid; q < M; q += kThreads)
      if (ck[q] == T) atomicAdd(&buf[(uint32_t)ci[q] >> 11], 1u);
    __syncthreads();
    if (tid == 0) { res[0] = 0; res[1] = 0; }
    __syncthreads();
    // smallest-index side: search the reversed histogram from its top
    find_bin_from_top<2048 / kThreads>([&](int i) { return buf[2047 - i]; }, e_take, tmp, res);
    const uint32_t binA = 2047u - res[0];
    const uint32_t eB = e_take - res[1];
    __syncthreads();
    for (int i = tid; i < 2048; i += kThreads) buf[i] = 0;
    __syncthreads();
    for (int q = tid; q < M; q += kThreads)
      if (ck[q] == T && ((uint32_t)ci[q] >> 11) == binA) atomicAdd(&buf[(uint32_t)ci[q] & 0x7ffu], 1u);
    __syncthreads();
    if (tid == 0) { res[0] = 0; res[1] = 0; }
    __syncthreads();
    find_bin_from_top<2048 / kThreads>([&](int i) { return buf[2047 - i]; }, eB, tmp, res);
    i_tie = (binA << 11) | (2047u - res[0]);
    __syncthreads();
  }
  // selected candidates per chunk, then the chunk output offsets
  const int nchi = (int)nch;
  for (int i = tid; i < nchi; i += kThreads) buf[i] = 0;
  __syncthreads();
  for (int q = tid; q < M; q += kThreads) {
    const uint32_t kk = ck[q];
    const uint32_t ix = (uint32_t)ci[q];
    if (kk > T || (kk == T && ix <= i_tie)) atomicAdd(&buf[ix / kSelChunk], 1u);
  }
  __syncthreads();
  {
    const int per = (nchi + kThreads - 1) / kThreads;
    const int c0 = tid * per;
    int local = 0;
    for (int i = 0; i < per; ++i) {
      const int cc = c0 + i;
      if (cc < nchi) local += (int)(p.chunk_cnt[((size_t)slot * p.C + cc) * 2 + 0] + buf[cc]);
    }
    int total;
    int run = block_excl_scan(local, tmp, total);
    for (int i = 0; i < per; ++i) {
      const int cc = c0 + i;
      if (cc < nchi) {
        const int cnt = (int)(p.chunk_cnt[((size_t)slot * p.C + cc) * 2 + 0] + buf[cc]);
        p.chunk_cnt[((size_t)slot * p.C + cc) * 2 + 1] = (uint32_t)run;
        run += cnt;
      }
    }
  }
  if (tid == 0) {
    p.sel_info[slot * 4 + 2] = T;
    p.sel_info[slot * 4 + 3] = i_tie;
    p.cand_count[slot] = 0u;
  }
}

// ------------------------------------------------------------- ordered write

__global__ __launch_bounds__(kThreads) void k_sel_write(const SelParams p) {
  __shared__ int tmp[4];
  const int r = blockIdx.x / p.C, c = blockIdx.x % p.C;
  const RowView v = row_view(p, r);
  if (c * kSelChunk >= v.n || v.k < 1) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int slot = v.slot;
  const uint32_t T = p.sel_info[slot * 4 + 2];
  const uint32_t i_tie = p.sel_info[slot * 4 + 3];
  int run = (int)p.chunk_cnt[((size_t)slot * p.C + c) * 2 + 1];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int i = c * kSelChunk + h * kThreads + tid;
    const bool valid = i < v.n;
    float s = 0.f;
    bool f = false;
    if (valid) {
      s = v.sc[i];
      const uint32_t kk = score_key(s);
      f = kk > T || (kk == T && (uint32_t)i <= i_tie);
    }
    int total;
    const int pos = block_excl_scan((int)f, tmp, total);
    if (f && run + pos < v.k) {
      v.out[run + pos] = i;
      if (v.vout) v.vout[run + pos] = s;
    }
    run += total;
    if (v.bm) {
      const uint64_t bal = __ballot(f);
      const int w0 = (c * kSelChunk + h * kThreads + wave * 64) >> 5;
      if (lane == 0 && w0 < p.W) v.bm[w0] = (uint32_t)bal;
      if (lane == 32 && w0 + 1 < p.W) v.bm[w0 + 1] = (uint32_t)(bal >> 32);
    }
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
  const dim3 grid((unsigned)p.nrows * (unsigned)p.C);
  if (with_hist) hipLaunchKernelGGL(k_sel_hist, grid, dim3(kThreads), 0, st, p);
  hipLaunchKernelGGL(k_sel_cand, grid, dim3(kThreads), 0, st, p);
  hipLaunchKernelGGL(k_sel_write, grid, dim3(kThreads), 0, st, p);
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
