// Device-side helpers for the gfx950 kernels (wave64, CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ld_internal.h"

namespace ld {

#define LD_INF __builtin_huge_valf()

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// bf16 pair in one dword -> the two floats (bf16 is the top half of a binary32).
// E4M3 codes (four per word, lowest byte first) to fp32, exactly, by the hardware
// conversion of the OCP 8-bit format.
__device__ __forceinline__ void fp8x4_to_f32(uint32_t w, float* f) {
  const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
  const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
  f[0] = lo[0]; f[1] = lo[1]; f[2] = hi[0]; f[3] = hi[1];
}
// Eight E4M3 codes to eight bf16 (exact: every E4M3 value has at most 4 significant
// bits and an exponent inside bf16's range, so the fp32 value's upper half is it).
__device__ __forceinline__ uint4 fp8x8_to_bf16x8(uint32_t w0, uint32_t w1) {
  float f[8];
  fp8x4_to_f32(w0, f);
  fp8x4_to_f32(w1, f + 4);
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = (__float_as_uint(f[2 * i + 1]) & 0xffff0000u) | (__float_as_uint(f[2 * i]) >> 16);
  return make_uint4(o[0], o[1], o[2], o[3]);
}

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// v_dot2c_f32_bf16: acc + a.lo*b.lo + a.hi*b.hi, bf16 operands, fp32 accumulate.
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), acc, false);
}

// Round-to-nearest-even fp32 -> bf16 (NaN stays a quiet NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x0040u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Order-preserving unsigned key of an fp32 score: a larger key is a better score.
// -0.0 maps to the key of +0.0 and every NaN maps to 0, below -inf.
__device__ __forceinline__ uint32_t score_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0u;
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// The fp32 value of an order-preserving key (the inverse of score_key; key 0 is NaN,
// and -0.0 comes back as +0.0, which the top-k order does not tell apart).
__device__ __forceinline__ float key_score(uint32_t k) {
  if (k == 0u) return __uint_as_float(0x7fc00000u);
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// S row of query-head slot `slot`: dense [slot * k_dense, +k_dense), or the CSR row
// [s_indptr[slot], s_indptr[slot + 1]) clipped to the s_cap entries of the S buffer, so
// that malformed offsets never reach outside it.
__device__ __forceinline__ void s_row(const int64_t* s_indptr, int k_dense, int64_t s_cap, int slot, int64_t* so,
                                      int* len) {
  if (!s_indptr) {
    *so = (int64_t)slot * k_dense;
    *len = k_dense;
    return;
  }
  const int64_t a = min(max(s_indptr[slot], (int64_t)0), s_cap);
  const int64_t e = min(max(s_indptr[slot + 1], a), s_cap);
  *so = a;
  *len = (int)min(e - a, (int64_t)0x7fffffff);
}

// Device-coherent accesses for data handed between workgroups of one launch: stores
// write through to the device coherence point and loads read from it (sc1), so no
// L2 writeback/invalidate fence is needed around the hand-off.
template <typename T>
__device__ __forceinline__ void st_dev(T* p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ __forceinline__ T ld_dev(const T* p) {
  return __hip_atomic_load(const_cast<T*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ float4 ld_dev4(const float* p) {
  return make_float4(ld_dev(p), ld_dev(p + 1), ld_dev(p + 2), ld_dev(p + 3));
}

// Count this workgroup in `ticket` once all of its device-coherent stores have
// completed; true in every thread of the workgroup that arrives last (of `target`).
// Every thread must call it.
__device__ __forceinline__ bool arrive_last(uint32_t* ticket, uint32_t target, int* flag) {
  __builtin_amdgcn_s_waitcnt(0);   // this wave's stores are acknowledged
  __syncthreads();                 // ... and every other wave's
  if (threadIdx.x == 0) {
    const uint32_t old = __hip_atomic_fetch_add(ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *flag = (old == target - 1u);
  }
  __syncthreads();
  return *flag != 0;
}

// ---- cross-lane steps without the LDS crossbar: DPP moves inside rows of 16 lanes,
// row broadcasts, and the gfx950 row-pair / half-wave swaps.

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
template <int CTRL, int ROWS = 0xf, bool ZERO = false>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, ROWS, 0xf, ZERO);
}

// Sum over each aligned group of 8 lanes; every lane of the group receives the same
// (bitwise identical) total: xor-1, xor-2 quad permutes, then the half-row mirror.
__device__ __forceinline__ float sum8(float v) {
  v += dpp_f<0xB1>(v);    // quad_perm [1,0,3,2]
  v += dpp_f<0x4E>(v);    // quad_perm [2,3,0,1]
  v += dpp_f<0x141>(v);   // row_half_mirror
  return v;
}
__device__ __forceinline__ int sum8_i(int v) {
  v += dpp_i<0xB1>(v);
  v += dpp_i<0x4E>(v);
  v += dpp_i<0x141>(v);
  return v;
}

// Partner 8 lanes away inside the row of 16 (row_ror:8 is lane ^ 8 there).
__device__ __forceinline__ float xor8_f(float v) { return dpp_f<0x128>(v); }

// Values of a lane and of its partner 16 (32) lanes away: v_permlane16_swap
// (v_permlane32_swap) of v with itself leaves the even-row (lower-half) value in the
// first result and the odd-row (upper-half) value in the second, in both lanes of the
// pair, so an operation on the two is bitwise the same in both.
__device__ __forceinline__ float add_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float add_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float max_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Max / sum over the 64 lanes, the same value in every lane.
__device__ __forceinline__ float wave_max_f(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v));
  v = fmaxf(v, dpp_f<0x4E>(v));
  v = fmaxf(v, dpp_f<0x141>(v));
  v = fmaxf(v, xor8_f(v));
  v = max_xor16(v);
  return max_xor32(v);
}
__device__ __forceinline__ float wave_sum_f(float v) {
  v = sum8(v);
  v += xor8_f(v);
  v = add_xor16(v);
  return add_xor32(v);
}

// Inclusive prefix sum over the 64 lanes: shifts by 1, 2, 4, 8 inside each row of 16
// (zero fill), then lane 15 of a row added to rows 1 and 3 and lane 31 to rows 2, 3.
__device__ __forceinline__ int wave_incl_sum(int v) {
  v += dpp_i<0x111, 0xf, true>(v);   // row_shr:1
  v += dpp_i<0x112, 0xf, true>(v);   // row_shr:2
  v += dpp_i<0x114, 0xf, true>(v);   // row_shr:4
  v += dpp_i<0x118, 0xf, true>(v);   // row_shr:8
  v += dpp_i<0x142, 0xa>(v);         // row_bcast:15
  v += dpp_i<0x143, 0xc>(v);         // row_bcast:31
  return v;
}
__device__ __forceinline__ int wave_total(int v) {
  return __builtin_amdgcn_readlane(wave_incl_sum(v), 63);
}
// Exclusive prefix sum over the wave; `total` receives the wave's sum.
__device__ __forceinline__ int wave_excl_scan(int x, int& total) {
  const int inc = wave_incl_sum(x);
  total = __builtin_amdgcn_readlane(inc, 63);
  return inc - x;
}

// Find the digit bin that holds the k-th largest key, with all NT threads of the
// workgroup. `cnt(i)` gives the count of bin i (i < NB). On return (in every thread):
// res[0] = bin, res[1] = number of keys in bins above it. Requires 1 <= k <= total.
// `tmp` is __shared__ int[NT/64].
template <int NB, int NT, typename F>
__device__ __forceinline__ void find_bin_from_top(F cnt, uint32_t k, int* tmp, uint32_t* res) {
  constexpr int PER = NB / NT;
  constexpr int NWV = NT / 64;
  const int t = threadIdx.x;
  uint32_t c[PER];
  uint32_t s = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) { c[i] = cnt(t * PER + i); s += c[i]; }
  // keys in the bins of higher threads: exclusive suffix sum (totals stay below 2^31)
  const int lane = t & 63, wave = t >> 6;
  // keys in this lane's bins and the bins of higher lanes of the wave
  const int inc = wave_incl_sum((int)s);
  const int wtot = __builtin_amdgcn_readlane(inc, 63);
  const int x = wtot - inc + (int)s;
  if (lane == 0) tmp[wave] = x;
  __syncthreads();
  int above_waves = 0;
#pragma unroll
  for (int i = 0; i < NWV; ++i) above_waves += (i > wave) ? tmp[i] : 0;
  __syncthreads();
  uint32_t run = (uint32_t)(above_waves + x - (int)s);
  if (run < k && run + s >= k) {
#pragma unroll
    for (int i = PER - 1; i >= 0; --i) {
      if (run + c[i] >= k) { res[0] = (uint32_t)(t * PER + i); res[1] = run; break; }
      run += c[i];
    }
  }
  __syncthreads();
}

// find_bin_from_top over counts held by the threads themselves: thread t holds the
// counts of bins t*PER .. t*PER+PER-1 in c[].
template <int NB, int NT>
__device__ __forceinline__ void find_bin_regs(const uint32_t (&c)[NB / NT], uint32_t k, int* tmp, uint32_t* res) {
  constexpr int PER = NB / NT;
  constexpr int NWV = NT / 64;
  const int t = threadIdx.x;
  uint32_t s = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) s += c[i];
  const int lane = t & 63, wave = t >> 6;
  const int inc = wave_incl_sum((int)s);
  const int wtot = __builtin_amdgcn_readlane(inc, 63);
  const int x = wtot - inc + (int)s;
  if (lane == 0) tmp[wave] = x;
  __syncthreads();
  int above_waves = 0;
#pragma unroll
  for (int i = 0; i < NWV; ++i) above_waves += (i > wave) ? tmp[i] : 0;
  __syncthreads();
  uint32_t run = (uint32_t)(above_waves + x - (int)s);
  if (run < k && run + s >= k) {
#pragma unroll
    for (int i = PER - 1; i >= 0; --i) {
      if (run + c[i] >= k) { res[0] = (uint32_t)(t * PER + i); res[1] = run; break; }
      run += c[i];
    }
  }
  __syncthreads();
}

// Sum over the NT threads of a workgroup, returned to every thread. tmp: __shared__
// int[NT / 64].
template <int NT>
__device__ __forceinline__ int block_sum(int v, int* tmp) {
  const int w = wave_total(v);
  if ((threadIdx.x & 63) == 0) tmp[threadIdx.x >> 6] = w;
  __syncthreads();
  int s = 0;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) s += tmp[i];
  __syncthreads();
  return s;
}

// The kRep replicas of a shared counter or histogram are indexed by workgroup id % kRep
// (the XCD it runs on), so that the atomics of the workgroups of one XCD meet in one
// replica and no address sees more than its share.
__device__ __forceinline__ int rep_of_block() { return (int)(blockIdx.x % kRep); }

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// 128-bit device-coherent (sc1) access through a buffer resource over `base`.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0x7fffffff, 0x00020000);
}
constexpr int kSc1 = 16;   // cache-policy bit of sc1 for buffer instructions
constexpr int kNt = 2;     // cache-policy bit of nt (streaming: read once) for buffer instructions

// bf16 KV rows are read once per launch: loads with the nontemporal hint, which keeps them
// from displacing the lines that are reused (partials, membership words, Q). (E4M3 rows
// keep plain loads: there four loads of a wave share each 128-byte line of K, and with the
// hint the later ones fetched it again, 32K steps 1.20 against 1.12 ms.)
__device__ __forceinline__ uint4 ld_stream16(const char* p) {
  const u32x4_t x = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(x.x, x.y, x.z, x.w);
}
// The same over `bytes` bytes from `base`: loads past them return 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_n(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}

// Digit-1 histogram rows: writers add to their replica; hist1_sum (every thread of the
// workgroup) writes the sum of the kRep replicas of row `slot` to lds[kHist1Bins],
// with 128-bit loads that are contiguous across the lanes. The caller synchronises
// before reading lds.
// reps: the replicas the row's writers use (at most kRep; the others stay zero).
__device__ __forceinline__ uint32_t* hist1_mine(uint32_t* h1, int slot, int reps = kRep) {
  return h1 + ((size_t)slot * kRep + (int)(blockIdx.x % (unsigned)reps)) * kHist1Bins;
}
// Clears the kRep replicas of row `slot` (every thread of the workgroup).
__device__ __forceinline__ void hist1_clear(uint32_t* h1, int slot, int reps = kRep) {
  uint4* r = reinterpret_cast<uint4*>(h1 + (size_t)slot * kRep * kHist1Bins);
  for (int i = threadIdx.x; i < reps * kHist1Bins / 4; i += (int)blockDim.x) r[i] = make_uint4(0u, 0u, 0u, 0u);
}
// NT: the workgroup's thread count (it sizes the thread's register columns).
template <int NT>
__device__ __forceinline__ void hist1_sum(uint32_t* lds, const uint32_t* h1, int slot, int reps = kRep) {
  const __amdgpu_buffer_rsrc_t r = rsrc(h1 + (size_t)slot * kRep * kHist1Bins);
  // every load of the thread's columns is issued before the first sum
  constexpr int kMaxCols = (kHist1Bins / 4 + NT - 1) / NT;   // column groups per thread
  constexpr int nt = NT;
  u32x4_t a[kMaxCols][kRep];
#pragma unroll
  for (int c = 0; c < kMaxCols; ++c) {
    const int i = threadIdx.x + c * nt;
#pragma unroll
    for (int q = 0; q < kRep; ++q)
      a[c][q] = (i < kHist1Bins / 4 && q < reps)
                    ? __builtin_amdgcn_raw_buffer_load_b128(r, (q * kHist1Bins + 4 * i) * 4, 0, kSc1)
                    : u32x4_t{0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int c = 0; c < kMaxCols; ++c) {
    const int i = threadIdx.x + c * nt;
    if (i < kHist1Bins / 4) {
      u32x4_t t = a[c][0];
#pragma unroll
      for (int q = 1; q < kRep; ++q) t += a[c][q];
      lds[4 * i + 0] = t.x;
      lds[4 * i + 1] = t.y;
      lds[4 * i + 2] = t.z;
      lds[4 * i + 3] = t.w;
    }
  }
}

// Release flags of a KV group's selectors: one 64-bit word per selector, on a 128-byte
// line of its own (rel[s * kRelStride]), so pollers never share a line.
constexpr int kRelStride = 16;

// Every member's release word := w (each by thread s % blockDim.x).
__device__ __forceinline__ void group_publish(uint64_t* rel, int ns, uint64_t w) {
  for (int s = threadIdx.x; s < ns; s += (int)blockDim.x) st_dev(rel + (size_t)s * kRelStride, w);
}

// Waits until this member's release word reaches w. Thread 0 polls with a
// read-modify-write, performed where the release lands and never on a stale copy. The
// wait is bounded; giving up sets *err.
__device__ __forceinline__ void group_wait(uint64_t* rel, int me, uint64_t w, uint32_t* err) {
  if (threadIdx.x == 0) {
    uint64_t* mine = rel + (size_t)me * kRelStride;
    int spins = 0;
    while (__hip_atomic_fetch_or(mine, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < w) {
      __builtin_amdgcn_s_sleep(2);
      if (++spins > kMaxSpins) {
        st_dev(err, 1u);
        break;
      }
    }
  }
  __syncthreads();
}

}  // namespace ld
