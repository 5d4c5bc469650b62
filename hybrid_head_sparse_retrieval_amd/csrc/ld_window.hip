// Sliding-window branch of a HySparse sparse layer (HySparse: A Hybrid Sparse
// Attention Architecture, section 3): every query head attends, in fp32, to the last W
// tokens of its sequence held in the layer's own small cache. The result goes to an
// fp32 buffer that the attention launch of the block-sparse branch reads when it
// writes O, mixing both through the sigmoid gate.
//
// One workgroup of four waves per (sequence, query head): wave w takes the window's
// 32-token rounds w, w + 4, ... For a round, lanes t and t + 32 compute the two halves
// of the logit of token t (each reads half its key row), and the lanes then split the
// head dimension for P·V over coalesced value rows, the weights broadcast from the lane
// that owns them; every load of a round is issued before the first use, so a round
// waits for memory once. The waves' online-softmax states are merged through LDS at the
// end.

#include "ld_device.h"

namespace ld {

namespace {

constexpr int kWinWaves = 4;

template <int D>
__global__ __launch_bounds__(kWinWaves * 64) void k_window(WindowParams p) {
  constexpr int DL = D / 64;   // adjacent head-dimension elements per lane in P·V
  __shared__ float qs[D];
  __shared__ float wm[kWinWaves], wl[kWinWaves];
  __shared__ float wacc[kWinWaves][D];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int row = blockIdx.x;   // b * Hq + h; the grid has B * Hq workgroups
  const int b = row / p.Hq, h = row % p.Hq;
  const int g = h / (p.Hq / p.Hkv);
  for (int i = threadIdx.x; i < D; i += kWinWaves * 64) qs[i] = bf_lo(p.q[(size_t)row * D + i]);
  __syncthreads();
  const size_t base = ((size_t)g * p.B + b) * (size_t)p.W * D;
  const uint16_t* K = p.kw + base;
  const uint16_t* V = p.vw + base;
  float m = -LD_INF, l = 0.f;
  float acc[DL];
#pragma unroll
  for (int j = 0; j < DL; ++j) acc[j] = 0.f;
  constexpr int RT = 32;        // tokens per round; lanes t and t + 32 split the token's dot product
  constexpr int HD = D / 2;     // dimensions per half
  const int tl = lane & 31, half = lane >> 5;
  for (int t0 = wave * RT; t0 < p.W; t0 += kWinWaves * RT) {
    const int t = t0 + tl;
    // half of the lane's key row and, for its DL dims, the round's 32 value rows (rows
    // past the window repeat the last row and get weight 0)
    uint4 kr[HD / 8];
    uint32_t vv[RT];
    const uint4* kp = reinterpret_cast<const uint4*>(K + (size_t)min(t, p.W - 1) * D + half * HD);
#pragma unroll
    for (int i = 0; i < HD / 8; ++i) kr[i] = kp[i];
#pragma unroll
    for (int u = 0; u < RT; ++u) {
      const uint16_t* vr = V + (size_t)min(t0 + u, p.W - 1) * D + lane * DL;
      vv[u] = (DL == 2) ? *reinterpret_cast<const uint32_t*>(vr) : (uint32_t)*vr;
    }
    float a = 0.f;
    const float* qh = &qs[half * HD];
#pragma unroll
    for (int i = 0; i < HD / 8; ++i) {
      const uint4 v = kr[i];
      const float4 q0 = *reinterpret_cast<const float4*>(&qh[i * 8]);
      const float4 q1 = *reinterpret_cast<const float4*>(&qh[i * 8 + 4]);
      a = fmaf(bf_lo(v.x & 0xffffu), q0.x, a); a = fmaf(bf_lo(v.x >> 16), q0.y, a);
      a = fmaf(bf_lo(v.y & 0xffffu), q0.z, a); a = fmaf(bf_lo(v.y >> 16), q0.w, a);
      a = fmaf(bf_lo(v.z & 0xffffu), q1.x, a); a = fmaf(bf_lo(v.z >> 16), q1.y, a);
      a = fmaf(bf_lo(v.w & 0xffffu), q1.z, a); a = fmaf(bf_lo(v.w >> 16), q1.w, a);
    }
    a = add_xor32(a);                            // both halves of the dot product, in both lanes
    const float s = (t < p.W) ? a * p.scale : -LD_INF;
    const float mn = fmaxf(m, wave_max_f(s));   // finite: the round holds token t0
    const float pt = (t < p.W) ? expf(s - mn) : 0.f;
    const float corr = (m == -LD_INF) ? 0.f : expf(m - mn);
    l = fmaf(l, corr, wave_sum_f(half == 0 ? pt : 0.f));   // each token once
#pragma unroll
    for (int j = 0; j < DL; ++j) acc[j] *= corr;
    const uint32_t pb = __float_as_uint(pt);
#pragma unroll
    for (int u = 0; u < RT; ++u) {
      const float pu = __uint_as_float(__builtin_amdgcn_readlane(pb, u));
      acc[0] = fmaf(pu, bf_lo(vv[u] & 0xffffu), acc[0]);
      if (DL == 2) acc[DL - 1] = fmaf(pu, bf_lo(vv[u] >> 16), acc[DL - 1]);
    }
    m = mn;
  }
  if (lane == 0) { wm[wave] = m; wl[wave] = l; }
#pragma unroll
  for (int j = 0; j < DL; ++j) wacc[wave][lane * DL + j] = acc[j];
  __syncthreads();
  if (wave == 0) {
    float M = -LD_INF;
#pragma unroll
    for (int w = 0; w < kWinWaves; ++w) M = fmaxf(M, wm[w]);
    float L = 0.f, o[DL];
#pragma unroll
    for (int j = 0; j < DL; ++j) o[j] = 0.f;
#pragma unroll
    for (int w = 0; w < kWinWaves; ++w) {
      const float c = (wm[w] == -LD_INF) ? 0.f : expf(wm[w] - M);   // waves without a round
      L = fmaf(wl[w], c, L);
#pragma unroll
      for (int j = 0; j < DL; ++j) o[j] = fmaf(wacc[w][lane * DL + j], c, o[j]);
    }
    const float il = 1.f / L;
#pragma unroll
    for (int j = 0; j < DL; ++j) p.o[(size_t)row * D + lane * DL + j] = o[j] * il;
  }
}

}  // namespace

hipError_t launch_window(const WindowParams& p, hipStream_t st) {
  const dim3 grid((unsigned)(p.B * p.Hq)), block(kWinWaves * 64);
  if (p.D == 128)
    hipLaunchKernelGGL(k_window<128>, grid, block, 0, st, p);
  else
    hipLaunchKernelGGL(k_window<64>, grid, block, 0, st, p);
  return hipGetLastError();
}

}  // namespace ld
