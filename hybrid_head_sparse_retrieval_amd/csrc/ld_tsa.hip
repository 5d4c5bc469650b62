// Token Sparse Attention, dense stage (Token Sparse Attention: Efficient Long-Context
// Inference, "Core Concept" and Steps 2-3): each query head keeps its top-k tokens (a
// selection launch writes their ascending positions I), attends densely among them
// only, and scatters the result back to the tokens' own rows of the output.
//
// This is a dense contraction, so both products run on the matrix cores
// (v_mfma_f32_16x16x32_bf16). A workgroup takes 64 selected queries of one head, 16 per
// wave; it walks the head's selected keys in tiles of 32 gathered rows staged in LDS
// (K row-major for the q.k product, V transposed so that the P.V product reads 8
// consecutive keys of one dimension per lane). The softmax runs online in log2 units;
// P goes through LDS (bf16) from the product's output layout to the operand layout.
// With the causal mask a key is allowed when its position is not after the query's;
// since I is ascending, that is key index <= query index, so tiles past the
// workgroup's last query are skipped.

#include "ld_device.h"

namespace ld {

namespace {

constexpr int kTsaWaves = 4;
constexpr int kTsaQ = 16 * kTsaWaves;   // queries per workgroup
constexpr int kTsaKeys = 32;            // keys per tile
constexpr float kTsaLog2e = 1.4426950408889634f;

typedef __bf16 tsa_bf16x8_t __attribute__((ext_vector_type(8)));
typedef float tsa_f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ tsa_f32x4_t mfma16(const uint4& a, const uint4& b, tsa_f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(tsa_bf16x8_t, a),
                                                 __builtin_bit_cast(tsa_bf16x8_t, b), c, 0, 0, 0);
}

template <int D>
struct TsaSmem {
  static constexpr int KS = D + 8;          // K tile row stride (elements)
  static constexpr int VS = kTsaKeys + 8;   // transposed V tile row stride
  static constexpr int PS = kTsaKeys + 8;   // P row stride
  uint16_t kt[kTsaKeys * KS];
  uint16_t vt[D * VS];
  uint16_t pl[kTsaWaves][16 * PS];
  int qpos[kTsaQ];
};

// Max / sum over the 16 lanes that share lane >> 4.
__device__ __forceinline__ float max16(float v) {
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float sum16(float v) {
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) v += __shfl_xor(v, o);
  return v;
}

// Tile t of the selected keys: thread tid loads LPT 16-byte pieces of K and V rows
// (rows past kk repeat the last selected row; their keys are masked).
template <int D, int LPT>
__device__ __forceinline__ void tsa_load(const uint16_t* Kg, const uint16_t* Vg, const int32_t* I, int kk, int t,
                                         int tid, uint4 (&kreg)[LPT], uint4 (&vreg)[LPT]) {
#pragma unroll
  for (int i = 0; i < LPT; ++i) {
    const int u = tid + i * kTsaWaves * 64;
    const int r = u / (D / 8), c = u % (D / 8);
    const size_t pos = (size_t)I[min(t * kTsaKeys + r, kk - 1)];
    kreg[i] = *reinterpret_cast<const uint4*>(Kg + pos * D + c * 8);
    vreg[i] = *reinterpret_cast<const uint4*>(Vg + pos * D + c * 8);
  }
}

// The loaded pieces to LDS: K row-major, V transposed.
template <int D, int LPT>
__device__ __forceinline__ void tsa_store(TsaSmem<D>& sm, int tid, const uint4 (&kreg)[LPT],
                                          const uint4 (&vreg)[LPT]) {
  constexpr int KS = TsaSmem<D>::KS, VS = TsaSmem<D>::VS;
#pragma unroll
  for (int i = 0; i < LPT; ++i) {
    const int u = tid + i * kTsaWaves * 64;
    const int r = u / (D / 8), c = u % (D / 8);
    *reinterpret_cast<uint4*>(&sm.kt[r * KS + c * 8]) = make_uint4(kreg[i].x, kreg[i].y, kreg[i].z, kreg[i].w);
    const uint32_t w0 = vreg[i].x, w1 = vreg[i].y, w2 = vreg[i].z, w3 = vreg[i].w;
    uint16_t* vc = &sm.vt[(c * 8) * VS + r];
    vc[0 * VS] = (uint16_t)(w0 & 0xffffu); vc[1 * VS] = (uint16_t)(w0 >> 16);
    vc[2 * VS] = (uint16_t)(w1 & 0xffffu); vc[3 * VS] = (uint16_t)(w1 >> 16);
    vc[4 * VS] = (uint16_t)(w2 & 0xffffu); vc[5 * VS] = (uint16_t)(w2 >> 16);
    vc[6 * VS] = (uint16_t)(w3 & 0xffffu); vc[7 * VS] = (uint16_t)(w3 >> 16);
  }
}

template <int D>
__global__ __launch_bounds__(kTsaWaves * 64) void k_tsa(TsaParams p) {
  using Smem = TsaSmem<D>;
  constexpr int KS = Smem::KS, VS = Smem::VS, PS = Smem::PS;
  constexpr int KC = D / 32;                                  // k-steps over the head dimension
  constexpr int NO = D / 16;                                  // 16-dim output tiles
  constexpr int LPT = kTsaKeys * (D / 8) / (kTsaWaves * 64);  // 16-byte loads per thread per tile
  static_assert(LPT >= 1, "a tile fills the workgroup's loads");
  __shared__ Smem sm;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lq = lane >> 4;                   // operand row / k-group
  const int row = blockIdx.x / p.qtiles, qt = blockIdx.x % p.qtiles;
  const int b = row / p.Hq, h = row % p.Hq, g = h / (p.Hq / p.Hkv);
  const int kk = p.kk;
  const int32_t* I = p.idx + (size_t)row * kk;
  const size_t seq0 = (size_t)b * p.T;
  const size_t plane = (size_t)p.B * p.T * D;                 // one head's rows
  const uint16_t* Qh = p.q + (size_t)h * plane + seq0 * D;
  const uint16_t* Kg = p.k + (size_t)g * plane + seq0 * D;
  const uint16_t* Vg = p.v + (size_t)g * plane + seq0 * D;
  const int q0 = qt * kTsaQ;

  if (tid < kTsaQ) sm.qpos[tid] = (q0 + tid < kk) ? I[q0 + tid] : -1;
  __syncthreads();
  // q operand: query lr of the wave, dims kc * 32 + 8 * lq
  const int qp = sm.qpos[wave * 16 + lr];
  uint4 qa[KC];
#pragma unroll
  for (int kc = 0; kc < KC; ++kc)
    qa[kc] = (qp >= 0) ? *reinterpret_cast<const uint4*>(Qh + (size_t)qp * D + kc * 32 + 8 * lq)
                       : make_uint4(0, 0, 0, 0);

  int ntiles = (kk + kTsaKeys - 1) / kTsaKeys;
  if (p.causal) ntiles = min(ntiles, (min(q0 + kTsaQ, kk) + kTsaKeys - 1) / kTsaKeys);

  uint4 kreg[LPT], vreg[LPT];

  const float sl = p.scale * kTsaLog2e;
  float m[4], lsum[4];
  tsa_f32x4_t o[NO];
#pragma unroll
  for (int r = 0; r < 4; ++r) { m[r] = -LD_INF; lsum[r] = 0.f; }
#pragma unroll
  for (int n = 0; n < NO; ++n) o[n] = tsa_f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int qrow0 = q0 + wave * 16 + 4 * lq;   // query index of output row r: qrow0 + r

  if (ntiles > 0) tsa_load<D, LPT>(Kg, Vg, I, kk, 0, tid, kreg, vreg);
  for (int t = 0; t < ntiles; ++t) {
    __syncthreads();                 // the previous tile's LDS reads are done
    tsa_store<D, LPT>(sm, tid, kreg, vreg);
    __syncthreads();
    if (t + 1 < ntiles) tsa_load<D, LPT>(Kg, Vg, I, kk, t + 1, tid, kreg, vreg);
    // S = Q K^T over the tile's two 16-key halves: element r of s[st] is query
    // qrow0 + r against key t * 32 + st * 16 + lr
    tsa_f32x4_t s[2];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      s[st] = tsa_f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        const uint4 kb = *reinterpret_cast<const uint4*>(&sm.kt[(st * 16 + lr) * KS + kc * 32 + 8 * lq]);
        s[st] = mfma16(qa[kc], kb, s[st]);
      }
    }
    float x[2][4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float mt = -LD_INF;
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const int key = t * kTsaKeys + st * 16 + lr;
        const bool ok = key < kk && (!p.causal || key <= qrow0 + r);
        x[st][r] = ok ? s[st][r] * sl : -LD_INF;
        mt = fmaxf(mt, x[st][r]);
      }
      mt = max16(mt);
      const float mn = fmaxf(m[r], mt);
      const float mu = (mn == -LD_INF) ? 0.f : mn;
      const float alpha = exp2_fast(m[r] - mu);       // 0 while nothing was allowed
      const float p0 = exp2_fast(x[0][r] - mu), p1 = exp2_fast(x[1][r] - mu);
      lsum[r] = fmaf(lsum[r], alpha, p0 + p1);
      m[r] = mn;
#pragma unroll
      for (int n = 0; n < NO; ++n) o[n][r] *= alpha;
      sm.pl[wave][(4 * lq + r) * PS + lr] = f32_to_bf16(p0);
      sm.pl[wave][(4 * lq + r) * PS + 16 + lr] = f32_to_bf16(p1);
    }
    __syncthreads();                 // P of the wave is in LDS
    // O += P V: P row lr (query), keys 8 * lq .. + 7; V^T row n * 16 + lr (dim), same keys
    const uint4 pa = *reinterpret_cast<const uint4*>(&sm.pl[wave][lr * PS + 8 * lq]);
#pragma unroll
    for (int n = 0; n < NO; ++n) {
      const uint4 vb = *reinterpret_cast<const uint4*>(&sm.vt[(n * 16 + lr) * VS + 8 * lq]);
      o[n] = mfma16(pa, vb, o[n]);
    }
  }
  // O / l, scattered to the queries' own rows
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float L = sum16(lsum[r]);
    const int qi = qrow0 + r;
    if (qi < kk) {
      const float il = 1.f / L;
      uint16_t* dst = p.out + (size_t)h * plane + (seq0 + (size_t)sm.qpos[wave * 16 + 4 * lq + r]) * D;
#pragma unroll
      for (int n = 0; n < NO; ++n) dst[n * 16 + lr] = f32_to_bf16(o[n][r] * il);
    }
  }
}

}  // namespace

hipError_t launch_tsa(const TsaParams& p, hipStream_t st) {
  const dim3 grid((unsigned)((size_t)p.B * p.Hq * p.qtiles)), block(kTsaWaves * 64);
  if (p.D == 128)
    hipLaunchKernelGGL(k_tsa<128>, grid, block, 0, st, p);
  else
    hipLaunchKernelGGL(k_tsa<64>, grid, block, 0, st, p);
  return hipGetLastError();
}

int tsa_queries_per_block() { return kTsaQ; }

}  // namespace ld
