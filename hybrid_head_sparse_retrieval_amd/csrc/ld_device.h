// Device-side helpers for the gfx950 kernels (wave64, CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ld_internal.h"

namespace ld {

#define LD_INF __builtin_huge_valf()

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// bf16 pair in one dword -> the two floats (bf16 is the top half of a binary32).
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

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

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

// DPP lane moves inside a row of 16 lanes.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
// Sum over each aligned group of 8 lanes; every lane of the group receives the same
// (bitwise identical) total: xor-1, xor-2 quad permutes, then the half-row mirror.
__device__ __forceinline__ float sum8(float v) {
  v += dpp_f<0xB1>(v);    // quad_perm [1,0,3,2]
  v += dpp_f<0x4E>(v);    // quad_perm [2,3,0,1]
  v += dpp_f<0x141>(v);   // row_half_mirror
  return v;
}

__device__ __forceinline__ float shfl_xor_f(float v, int m) { return __shfl_xor(v, m, 64); }

// Exclusive scan over the 256 threads of a workgroup (thread order). `tmp` is
// __shared__ int[4]. Returns the exclusive prefix; `total` receives the sum.
__device__ __forceinline__ int block_excl_scan(int v, int* tmp, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) tmp[wave] = x;
  __syncthreads();
  int w0 = tmp[0], w1 = tmp[1], w2 = tmp[2], w3 = tmp[3];
  __syncthreads();
  int off = (wave > 0 ? w0 : 0) + (wave > 1 ? w1 : 0) + (wave > 2 ? w2 : 0);
  total = w0 + w1 + w2 + w3;
  return off + x - v;
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
  int x = (int)s;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int y = __shfl_down(x, o, 64);
    if (lane + o < 64) x += y;
  }
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

}  // namespace ld
