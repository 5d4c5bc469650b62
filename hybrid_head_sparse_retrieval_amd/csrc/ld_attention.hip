// Split-N decode attention for one layer on gfx950 (CDNA4, wave64).
//
// Computes, for each active query head h of KV group g and sequence b,
//   O = softmax(q K^T * scale) V
// over all N_b rows for retrieval heads and over the rows of S for sparse heads
// (LycheeDecode summary page, method steps 3 and 4). One workgroup handles a
// (b, g, split) tile of `ts` consecutive token rows and all query heads of the group:
//   * a group that contains a retrieval head streams every row of the tile once and
//     feeds it to all of the group's heads; sparse heads of that group drop the rows
//     outside their S (membership bitmaps),
//   * a group of sparse heads only reads the rows in the union of its heads' S and
//     each head accumulates its own rows.
// Each wave keeps an online softmax state per row slot (no block barriers while
// streaming); the states are merged at the end of the tile and written as split
// partials. The last workgroup of a (b, g) (integer ticket, agent-scope
// acquire/release) merges the partials into O, and, when selection is requested,
// turns the fused first-digit histogram of each retrieval head into the first
// selection digit for the argsTopK kernels.
//
// Lane layout: 8 lanes per K/V row (16 bf16 each at d=128, 8 at d=64), 8 rows per
// wave step, 4 waves -> 32 rows per workgroup step. q.K uses v_dot2c_f32_bf16 on
// packed bf16 (exact products, fp32 accumulate); P.V converts V to fp32 and uses FMA.

#include "ld_device.h"

namespace ld {

namespace {

constexpr float kLog2e = 1.4426950408889634f;

template <int D, int G, bool HIST>
struct AttnSmem {
  uint8_t hm[kMaxSplitRows];        // per-row membership mask of the group's heads
  uint16_t list[kMaxSplitRows];     // rows to visit (gather mode)
  int wcnt[4];
  int misc[4];
  union {
    uint32_t hist[HIST ? G : 1][kHist1Bins];
    struct {
      float acc[4][G][D];
      float m[4][G];
      float l[4][G];
    } red;
    struct {
      float w[G][kMaxSplits];   // split weights
      float inv_l[G];
    } cmb;
  } u;
  uint32_t res[2];
};

template <int D, int G, bool HIST>
__global__ __launch_bounds__(kThreads) void k_attention(const AttnParams p) {
  constexpr int LPR = 8;             // lanes per row
  constexpr int EPL = D / LPR;       // bf16 elements per lane
  constexpr int DWL = EPL / 2;       // dwords per lane
  constexpr int NV = DWL / 4;        // 16-byte loads per lane per row
  constexpr int U = 4;               // wave steps per chunk
  using Smem = AttnSmem<D, G, HIST>;
  __shared__ Smem sm;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int rg = lane >> 3, li = lane & 7;

  int bid = blockIdx.x;
  const int split = bid % p.nsplit;
  bid /= p.nsplit;
  const int gi = bid % p.ngroups;
  const int b = bid / p.ngroups;
  const int g = p.groups[gi];

  int64_t tok0;
  int nb;
  if (p.kv_indptr) {
    tok0 = p.kv_indptr[b];
    nb = (int)(p.kv_indptr[b + 1] - tok0);
  } else {
    tok0 = (int64_t)b * p.seq_len;
    nb = p.seq_len;
  }
  // never read past the cache or the per-row scratch, whatever kv_indptr holds
  nb = min(nb, p.seq_len);
  if (tok0 < 0 || tok0 >= p.total_tokens) nb = 0;
  else if ((int64_t)nb > p.total_tokens - tok0) nb = (int)(p.total_tokens - tok0);
  const int nsplit_b = (nb + p.ts - 1) / p.ts;
  if (nb <= 0 || split >= nsplit_b) return;
  const int r0 = split * p.ts;
  const int nrows = min(p.ts, nb - r0);

  // Head roles inside the group (bit j <-> query head g*G + j).
  uint32_t act = 0, ret = 0;
#pragma unroll
  for (int j = 0; j < G; ++j) {
    const int h = g * G + j;
    act |= (uint32_t)((p.active >> h) & 1ull) << j;
    ret |= (uint32_t)((p.retrieval >> h) & 1ull) << j;
  }
  ret &= act;
  const uint32_t spm = act & ~ret;
  const bool dense = ret != 0;

  // ---- membership of each row of the tile
  if (spm) {
    for (int r = tid; r < nrows; r += kThreads) {
      uint32_t m = ret;
      const int row = r0 + r;
#pragma unroll
      for (int j = 0; j < G; ++j) {
        if (spm >> j & 1) {
          const uint32_t w = p.bitmaps[(size_t)(b * p.Hq + g * G + j) * p.W + (row >> 5)];
          m |= ((w >> (row & 31)) & 1u) << j;
        }
      }
      sm.hm[r] = (uint8_t)m;
    }
  }
  if (HIST) {
    for (int i = tid; i < G * kHist1Bins; i += kThreads) (&sm.u.hist[0][0])[i] = 0;
  }
  __syncthreads();

  int nlist = nrows;
  if (!dense) {
    int total = 0;
    for (int base = 0; base < nrows; base += kThreads) {
      const int r = base + tid;
      const bool f = r < nrows && sm.hm[r] != 0;
      const uint64_t bal = __ballot(f);
      const int pre = __popcll(bal & ((1ull << lane) - 1ull));
      if (lane == 0) sm.wcnt[wave] = __popcll(bal);
      __syncthreads();
      int woff = 0, tot = 0;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        woff += (w < wave) ? sm.wcnt[w] : 0;
        tot += sm.wcnt[w];
      }
      if (f) sm.list[total + woff + pre] = (uint16_t)r;
      total += tot;
      __syncthreads();
    }
    nlist = total;
  }

  // ---- query registers: packed bf16 pairs of this lane's slice, per head
  uint32_t qv[G][DWL];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    const uint4* qp = reinterpret_cast<const uint4*>(p.q + (size_t)(b * p.Hq + g * G + j) * D + li * EPL);
#pragma unroll
    for (int c = 0; c < NV; ++c) {
      const uint4 x = qp[c];
      qv[j][4 * c + 0] = x.x; qv[j][4 * c + 1] = x.y; qv[j][4 * c + 2] = x.z; qv[j][4 * c + 3] = x.w;
    }
  }

  float m_[G], l_[G], acc[G][EPL];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    m_[j] = -LD_INF;
    l_[j] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[j][e] = 0.f;
  }

  const uint16_t* kbase = p.kc + (size_t)g * p.kv_head_stride + (size_t)(tok0 + r0) * D + li * EPL;
  const uint16_t* vbase = p.vc + (size_t)g * p.kv_head_stride + (size_t)(tok0 + r0) * D + li * EPL;
  float* lg_base[G];
#pragma unroll
  for (int j = 0; j < G; ++j)
    lg_base[j] = p.logits ? p.logits + (size_t)(b * p.Hq + g * G + j) * p.seq_len + r0 : nullptr;

  const int nsteps = (nlist + 7) >> 3;
  for (int st0 = wave; st0 < nsteps; st0 += 4 * U) {
    uint4 kr[U][NV], vr[U][NV];
    int rowv[U];
    bool valid[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int pos = (st0 + 4 * u) * 8 + rg;
      valid[u] = pos < nlist;
      const int row = valid[u] ? (dense ? pos : (int)sm.list[pos]) : 0;
      rowv[u] = row;
      const uint4* kp = reinterpret_cast<const uint4*>(kbase + (size_t)row * D);
      const uint4* vp = reinterpret_cast<const uint4*>(vbase + (size_t)row * D);
#pragma unroll
      for (int c = 0; c < NV; ++c) {
        if (valid[u]) {
          kr[u][c] = kp[c];
          vr[u][c] = vp[c];
        } else {
          kr[u][c] = make_uint4(0, 0, 0, 0);
          vr[u][c] = make_uint4(0, 0, 0, 0);
        }
      }
    }
    // q . k for every head and row slot
    float t[U][G];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t hm = valid[u] ? (spm ? (uint32_t)sm.hm[rowv[u]] : ret) : 0u;
      const uint32_t* kw = reinterpret_cast<const uint32_t*>(&kr[u][0]);
#pragma unroll
      for (int j = 0; j < G; ++j) {
        float d = 0.f;
#pragma unroll
        for (int c = 0; c < DWL; ++c) d = dot2_bf16(qv[j][c], kw[c], d);
        d = sum8(d);
        const float s = d * p.scale;
        const bool mem = (hm >> j) & 1u;
        if ((ret >> j & 1u) && mem && li == 0) {
          if (lg_base[j]) lg_base[j][rowv[u]] = s;
          if (HIST) atomicAdd(&sm.u.hist[j][score_key(s) >> 21], 1u);
        }
        t[u][j] = mem ? s * kLog2e : -LD_INF;
      }
    }
    // online softmax update (rescale only when some running max grows)
    float pr[U][G];
#pragma unroll
    for (int j = 0; j < G; ++j) {
      float mc = t[0][j];
#pragma unroll
      for (int u = 1; u < U; ++u) mc = fmaxf(mc, t[u][j]);
      const float mn = fmaxf(m_[j], mc);
      if (__any(mn > m_[j])) {
        const float mu = (mn == -LD_INF) ? 0.f : mn;
        const float alpha = exp2_fast(m_[j] - mu);
        l_[j] *= alpha;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[j][e] *= alpha;
        m_[j] = mn;
      }
      const float mu = (m_[j] == -LD_INF) ? 0.f : m_[j];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        pr[u][j] = exp2_fast(t[u][j] - mu);
        l_[j] += pr[u][j];
      }
    }
    // P . V
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t* vw = reinterpret_cast<const uint32_t*>(&vr[u][0]);
      float vf[EPL];
#pragma unroll
      for (int c = 0; c < DWL; ++c) {
        vf[2 * c] = bf_lo(vw[c]);
        vf[2 * c + 1] = bf_hi(vw[c]);
      }
#pragma unroll
      for (int j = 0; j < G; ++j) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[j][e] = fmaf(pr[u][j], vf[e], acc[j][e]);
      }
    }
  }

  // ---- flush the fused selection histogram
  if (HIST) {
    __syncthreads();
    for (int i = tid; i < G * kHist1Bins; i += kThreads) {
      const int j = i / kHist1Bins, bin = i % kHist1Bins;
      const uint32_t c = sm.u.hist[j][bin];
      if (c) atomicAdd(p.hist1 + (size_t)(b * p.Hq + g * G + j) * kHist1Bins + bin, c);
    }
    __syncthreads();
  }

  // ---- merge the 8 row slots of each wave (lanes li, li+8, ..., li+56)
#pragma unroll
  for (int off = 8; off < 64; off <<= 1) {
#pragma unroll
    for (int j = 0; j < G; ++j) {
      const float mo = shfl_xor_f(m_[j], off);
      const float lo = shfl_xor_f(l_[j], off);
      const float mn = fmaxf(m_[j], mo);
      const float mu = (mn == -LD_INF) ? 0.f : mn;
      const float a = exp2_fast(m_[j] - mu), c = exp2_fast(mo - mu);
      l_[j] = l_[j] * a + lo * c;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[j][e] = acc[j][e] * a + shfl_xor_f(acc[j][e], off) * c;
      m_[j] = mn;
    }
  }
  if (rg == 0) {
#pragma unroll
    for (int j = 0; j < G; ++j) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) sm.u.red.acc[wave][j][li * EPL + e] = acc[j][e];
      if (li == 0) {
        sm.u.red.m[wave][j] = m_[j];
        sm.u.red.l[wave][j] = l_[j];
      }
    }
  }
  __syncthreads();
  // ---- merge the 4 waves and write this split's partials
  for (int i = tid; i < G * D; i += kThreads) {
    const int j = i / D, d = i % D;
    if (!(act >> j & 1u)) continue;
    float mw[4], M = -LD_INF;
#pragma unroll
    for (int w = 0; w < 4; ++w) { mw[w] = sm.u.red.m[w][j]; M = fmaxf(M, mw[w]); }
    const float mu = (M == -LD_INF) ? 0.f : M;
    float a = 0.f, L = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float sc = exp2_fast(mw[w] - mu);
      a += sm.u.red.acc[w][j][d] * sc;
      L += sm.u.red.l[w][j] * sc;
    }
    const size_t slot = (size_t)(b * p.Hq + g * G + j) * p.P + split;
    p.part_acc[slot * D + d] = a;
    if (d == 0) {
      p.part_ml[slot * 2 + 0] = M;
      p.part_ml[slot * 2 + 1] = L;
    }
  }

  // ---- ticket: the last split of (b, g) merges all partials
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    const uint32_t old = __hip_atomic_fetch_add(p.tickets + b * p.Hkv + g, 1u, __ATOMIC_ACQ_REL,
                                                __HIP_MEMORY_SCOPE_AGENT);
    sm.misc[0] = (old == (uint32_t)(nsplit_b - 1));
  }
  __syncthreads();
  if (!sm.misc[0]) return;
  __threadfence();
  if (tid == 0) p.tickets[b * p.Hkv + g] = 0u;

  // split weights w_p = exp2(m_p - M) / L per head, kept in LDS
  constexpr int kMaxW = sizeof(sm.u.cmb.w[0]) / sizeof(float);
  const int np = nsplit_b;
  for (int j = 0; j < G; ++j) {
    if (!(act >> j & 1u)) continue;
    const size_t base = (size_t)(b * p.Hq + g * G + j) * p.P;
    float M = -LD_INF;
    for (int s = tid; s < np; s += kThreads) M = fmaxf(M, p.part_ml[(base + s) * 2]);
    // block max
    for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o, 64));
    if (lane == 0) sm.wcnt[wave] = __float_as_int(M);
    __syncthreads();
    M = fmaxf(fmaxf(__int_as_float(sm.wcnt[0]), __int_as_float(sm.wcnt[1])),
              fmaxf(__int_as_float(sm.wcnt[2]), __int_as_float(sm.wcnt[3])));
    __syncthreads();
    const float mu = (M == -LD_INF) ? 0.f : M;
    float L = 0.f;
    for (int s = tid; s < np; s += kThreads) {
      const float w = exp2_fast(p.part_ml[(base + s) * 2] - mu);
      if (s < kMaxW) sm.u.cmb.w[j][s] = w;
      L += p.part_ml[(base + s) * 2 + 1] * w;
    }
    for (int o = 32; o > 0; o >>= 1) L += __shfl_xor(L, o, 64);
    if (lane == 0) sm.wcnt[wave] = __float_as_int(L);
    __syncthreads();
    if (tid == 0)
      sm.u.cmb.inv_l[j] = 1.f / (__int_as_float(sm.wcnt[0]) + __int_as_float(sm.wcnt[1]) +
                                 __int_as_float(sm.wcnt[2]) + __int_as_float(sm.wcnt[3]));
    __syncthreads();
  }
  // O[d] = sum_p acc_p[d] * w_p / L ; 4-float columns, threads split over (head, column)
  {
    constexpr int COLS = D / 4;
    for (int i = tid; i < G * COLS; i += kThreads) {
      const int j = i / COLS, c = i % COLS;
      if (!(act >> j & 1u)) continue;
      const size_t base = (size_t)(b * p.Hq + g * G + j) * p.P;
      const float4* ap = reinterpret_cast<const float4*>(p.part_acc + base * D) + c;
      float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
      int s = 0;
      for (; s + 8 <= np; s += 8) {
        float4 x[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) x[q] = ap[(size_t)(s + q) * COLS];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const float w = (s + q < kMaxW) ? sm.u.cmb.w[j][s + q] : 0.f;
          o.x = fmaf(x[q].x, w, o.x); o.y = fmaf(x[q].y, w, o.y);
          o.z = fmaf(x[q].z, w, o.z); o.w = fmaf(x[q].w, w, o.w);
        }
      }
      for (; s < np; ++s) {
        const float4 x = ap[(size_t)s * COLS];
        const float w = (s < kMaxW) ? sm.u.cmb.w[j][s] : 0.f;
        o.x = fmaf(x.x, w, o.x); o.y = fmaf(x.y, w, o.y);
        o.z = fmaf(x.z, w, o.z); o.w = fmaf(x.w, w, o.w);
      }
      const float il = sm.u.cmb.inv_l[j];
      ushort4 r;
      r.x = f32_to_bf16(o.x * il); r.y = f32_to_bf16(o.y * il);
      r.z = f32_to_bf16(o.z * il); r.w = f32_to_bf16(o.w * il);
      reinterpret_cast<ushort4*>(p.out + (size_t)(b * p.Hq + g * G + j) * D)[c] = r;
    }
  }

  // ---- first selection digit for each retrieval head (fused histogram complete)
  if (HIST && p.do_topk) {
    for (int j = 0; j < G; ++j) {
      if (!(ret >> j & 1u)) continue;
      const int slot = b * p.Hq + g * G + j;
      uint32_t* hist = p.hist1 + (size_t)slot * kHist1Bins;
      int kk = p.k_dense;
      if (p.s_indptr) kk = (int)(p.s_indptr[slot + 1] - p.s_indptr[slot]);
      kk = min(kk, nb);
      if (tid == 0) { sm.res[0] = 0; sm.res[1] = 0; }
      __syncthreads();
      if (kk >= 1) {
        find_bin_from_top<kHist1Bins / kThreads>([&](int i) { return hist[i]; }, (uint32_t)kk,
                                                 sm.wcnt, sm.res);
      }
      __syncthreads();
      if (tid == 0) {
        p.sel_info[slot * 4 + 0] = sm.res[0];
        p.sel_info[slot * 4 + 1] = (uint32_t)kk - sm.res[1];   // still needed from bin b1
      }
      for (int i = tid; i < kHist1Bins; i += kThreads) hist[i] = 0u;
      __syncthreads();
    }
  }
}

template <int D, int G>
hipError_t launch_dg(const AttnParams& p, dim3 grid, hipStream_t st) {
  if (p.do_topk)
    hipLaunchKernelGGL((k_attention<D, G, true>), grid, dim3(kThreads), 0, st, p);
  else
    hipLaunchKernelGGL((k_attention<D, G, false>), grid, dim3(kThreads), 0, st, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attention(const AttnParams& p, int D, int G, dim3 grid, hipStream_t st) {
  if (D == 128) {
    switch (G) {
      case 1: return launch_dg<128, 1>(p, grid, st);
      case 2: return launch_dg<128, 2>(p, grid, st);
      case 4: return launch_dg<128, 4>(p, grid, st);
      case 8: return launch_dg<128, 8>(p, grid, st);
    }
  } else if (D == 64) {
    switch (G) {
      case 1: return launch_dg<64, 1>(p, grid, st);
      case 2: return launch_dg<64, 2>(p, grid, st);
      case 4: return launch_dg<64, 4>(p, grid, st);
      case 8: return launch_dg<64, 8>(p, grid, st);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace ld
