// Token Sparse Attention, dense stage (Token Sparse Attention: Efficient Long-Context
// Inference, "Core Concept" and Steps 2-3): each query head keeps its top-k tokens (a
// selection launch writes their ascending positions I), attends densely among them
// only, and scatters the result back to the tokens' own rows of the output.
//
// This is a dense contraction, so both products run on the matrix cores
// (v_mfma_f32_16x16x32_bf16). A workgroup takes 64 selected queries of one head, 16 per
// wave; it walks the head's selected keys in tiles of 64 gathered rows staged in LDS
// (K row-major for the q.k product, V transposed so that the P.V product reads runs of
// consecutive keys of one dimension per lane), two tiles deep: while one tile is
// computed the next is stored and the one after is loaded, at positions staged in LDS
// 1024 at a time. Both products run transposed (S^T = K Q^T, O^T = V^T P^T): the score
// layout of S^T is the operand layout of P^T, so P stays in registers, and a lane's
// softmax state is that of one query. The softmax runs online in log2 units.
// With the causal mask a key is allowed when its position is not after the query's;
// since I is ascending, that is key index <= query index, so tiles past the
// workgroup's last query are skipped. When the (row, query block) workgroups are too
// few to fill the chip, the keys are cut into splits of split_keys keys run by
// workgroups of their own, and a merge launch combines their partials (max, sum,
// unnormalised O) per query.

#include <type_traits>

#include "ld_tile.h"

namespace ld {

namespace {

template <int D>
__global__ __launch_bounds__(kTileWaves * 64) void k_tsa(TsaParams p) {
  using Smem = TileSmem<D>;
  constexpr int NT = kTileWaves * 64;
  constexpr int KS = Smem::KS;
  constexpr int KC = D / 32;                                  // k-steps over the head dimension
  constexpr int NO = D / 16;                                  // 16-dim output tiles
  static_assert(TileRegs<D>::LPT >= 1, "a tile fills the workgroup's loads");
  __shared__ Smem sm;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lq = lane >> 4;                   // operand row / k-group
  // key split, row and query block of this workgroup. Query blocks go out in the order
  // 0, 1, .., then from the last one down, each over all rows: with causal masks the
  // workgroups that share a compute unit (launched half a grid apart) then pair a short
  // block with a long one.
  const int sp = blockIdx.x % p.nsplit;
  const int rows = p.B * p.Hq;
  const int wi = blockIdx.x / p.nsplit, jq = wi / rows, row = wi % rows;
  const int half = (p.qtiles + 1) / 2;
  const int qt = jq < half ? jq : p.qtiles - 1 - (jq - half);
  const int b = row / p.Hq, h = row % p.Hq, g = h / (p.Hq / p.Hkv);
  const int kk = p.kk;
  const int32_t* I = p.idx + (size_t)row * kk;
  const size_t seq0 = (size_t)b * p.T;
  const size_t plane = (size_t)p.B * p.T * D;                 // one head's rows
  const uint16_t* Qh = p.q + (size_t)h * plane + seq0 * D;
  const uint16_t* Kg = p.k + (size_t)g * plane + seq0 * D;
  const uint16_t* Vg = p.v + (size_t)g * plane + seq0 * D;
  const int q0 = qt * kTileQ;
  auto clampT = [&](int x) { return min(max(x, 0), p.T - 1); };   // caller-given sets stay inside

  if (tid < kTileQ) sm.qpos[tid] = (q0 + tid < kk) ? clampT(I[q0 + tid]) : -1;
  __syncthreads();
  // q operand: query lr of the wave, dims kc * 32 + 8 * lq
  const int qp = sm.qpos[wave * 16 + lr];
  uint4 qa[KC];
#pragma unroll
  for (int kc = 0; kc < KC; ++kc)
    qa[kc] = (qp >= 0) ? *reinterpret_cast<const uint4*>(Qh + (size_t)qp * D + kc * 32 + 8 * lq)
                       : make_uint4(0, 0, 0, 0);

  const int nkeys = p.causal ? min(q0 + kTileQ, kk) : kk;     // keys any query here may see
  const int k_lo = sp * p.split_keys;                         // this split's keys: [k_lo, k_hi)
  const int k_hi = min(nkeys, k_lo + p.split_keys);
  if (k_lo >= k_hi) return;                                   // the same in every thread
  const float sl = p.scale * kTileLog2e;
  // The products run transposed, so that a lane holds one query: S^T = K Q^T gives lane
  // (lr, lq) the scores of query lr against keys 4 lq + r of each 16-key half, which is
  // already the operand layout of P^T in O^T = V^T P^T; element r of o[n] is dimension
  // n * 16 + 4 lq + r of query lr. The lanes lr, lr + 16, lr + 32, lr + 48 share a query.
  float m = -LD_INF, lsum = 0.f;               // running max (log2 units) and partial sum
  tile_f32x4_t o[NO];
#pragma unroll
  for (int n = 0; n < NO; ++n) o[n] = tile_f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int qi = q0 + wave * 16 + lr;          // this lane's query
  TileRegs<D> R;

  for (int cb = k_lo; cb < k_hi; cb += kTileIdx) {
    const int nk = min(kTileIdx, k_hi - cb);
    const int nt = (nk + kTileKeys - 1) / kTileKeys;
    __syncthreads();                             // the previous chunk is done with LDS
#pragma unroll 8
    for (int i = tid; i < nk; i += NT) sm.kidx[i] = clampT(I[cb + i]);
    __syncthreads();
    tile_load<D>(Kg, Vg, sm.kidx, nk, 0, tid, R);
    tile_store<D>(sm, 0, tid, R);
    if (nt > 1) tile_load<D>(Kg, Vg, sm.kidx, nk, 1, tid, R);
    // tiles in pairs, so that each step's LDS buffer is a compile-time constant
    auto step = [&](int t, auto bufc) {
      constexpr int buf = decltype(bufc)::value;
      __syncthreads();                           // tile t is in buf; the other buffer is free
      if (t + 1 < nt) tile_store<D>(sm, buf ^ 1, tid, R);
      if (t + 2 < nt) tile_load<D>(Kg, Vg, sm.kidx, nk, t + 2, tid, R);
      // S^T = K Q^T over the tile's four 16-row quarters (LDS rows st * 16 ..): element
      // r of s[st] is key cb + t * 64 + 32 (st >> 1) + 8 lq + 4 (st & 1) + r against
      // query qi
      constexpr int NST = kTileKeys / 16;
      tile_f32x4_t s[NST];
#pragma unroll
      for (int st = 0; st < NST; ++st) {
        s[st] = tile_f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
          const uint4 ka =
              *reinterpret_cast<const uint4*>(&sm.kt[buf][(st * 16 + lr) * KS + kc * 32 + 8 * lq]);
          s[st] = mfma16(ka, qa[kc], s[st]);
        }
      }
      const int kt0 = cb + t * kTileKeys;   // the tile's first key; the wave's first query is q0 + 16 * wave
      float x[NST][4];
      // `masked` checks every key (tiles at the end of the range or on the causal
      // diagonal); the interior tiles skip the checks
      auto scores = [&](auto masked) {
#pragma unroll
        for (int st = 0; st < NST; ++st)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            if constexpr (decltype(masked)::value) {
              const int key = kt0 + 32 * (st >> 1) + 8 * lq + 4 * (st & 1) + r;
              const bool ok = key < k_hi && (!p.causal || key <= qi);
              x[st][r] = ok ? s[st][r] * sl : -LD_INF;
            } else {
              x[st][r] = s[st][r] * sl;
            }
          }
      };
      if (kt0 + kTileKeys <= k_hi && (!p.causal || kt0 + kTileKeys - 1 <= q0 + wave * 16))
        scores(std::false_type{});
      else
        scores(std::true_type{});
      float mt = -LD_INF;
#pragma unroll
      for (int st = 0; st < NST; ++st)
        mt = fmaxf(mt, fmaxf(fmaxf(x[st][0], x[st][1]), fmaxf(x[st][2], x[st][3])));
      mt = max_xor32(max_xor16(mt));             // over the query's four lanes
      const float mn = fmaxf(m, mt);
      const float mu = (mn == -LD_INF) ? 0.f : mn;
      const float alpha = (mn > m) ? exp2_fast(m - mu) : 1.f;   // 0 while nothing was allowed
      float pr[NST][4];
      float ps = 0.f;
#pragma unroll
      for (int st = 0; st < NST; ++st)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          pr[st][r] = exp2_fast(x[st][r] - mu);
          ps += pr[st][r];
        }
      lsum = fmaf(lsum, alpha, ps);
      m = mn;
      // rescale when some query of the wave has a larger max (rare once the maxima settle)
      if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
#pragma unroll
        for (int n = 0; n < NO; ++n)
#pragma unroll
          for (int r = 0; r < 4; ++r) o[n][r] *= alpha;
      }
      // O^T += V^T P^T per 32-key half hh: P^T k slots 8 lq .. 8 lq + 7 hold keys
      // 32 hh + 8 lq .. + 7 (quarter 2 hh, then 2 hh + 1); the V^T row n * 16 + lr
      // (dimension) is read at the same keys, 16 consecutive bytes
#pragma unroll
      for (int hh = 0; hh < NST / 2; ++hh) {
        uint4 pb;
        pb.x = (uint32_t)tile_bf16(pr[2 * hh][0]) | ((uint32_t)tile_bf16(pr[2 * hh][1]) << 16);
        pb.y = (uint32_t)tile_bf16(pr[2 * hh][2]) | ((uint32_t)tile_bf16(pr[2 * hh][3]) << 16);
        pb.z = (uint32_t)tile_bf16(pr[2 * hh + 1][0]) | ((uint32_t)tile_bf16(pr[2 * hh + 1][1]) << 16);
        pb.w = (uint32_t)tile_bf16(pr[2 * hh + 1][2]) | ((uint32_t)tile_bf16(pr[2 * hh + 1][3]) << 16);
#pragma unroll
        for (int n = 0; n < NO; ++n) {
          const uint4 va = *reinterpret_cast<const uint4*>(&sm.vt[buf][Smem::vrow(n * 16 + lr) + 32 * hh + 8 * lq]);
          o[n] = mfma16(va, pb, o[n]);
        }
      }
    };
    for (int t = 0; t < nt; t += 2) {
      step(t, std::integral_constant<int, 0>{});
      if (t + 1 < nt) step(t + 1, std::integral_constant<int, 1>{});
    }
  }
  const float L = add_xor32(add_xor16(lsum));   // the query's sum over its four lanes
  if (p.nsplit > 1) {
    // this split's partial: max (log2 units), sum and unnormalised O of each query
    const size_t unit = ((size_t)row * p.qtiles + qt) * p.nsplit + sp;
    const int ql = wave * 16 + lr;
    if (lq == 0) {
      p.part_ml[(unit * kTileQ + ql) * 2 + 0] = m;
      p.part_ml[(unit * kTileQ + ql) * 2 + 1] = L;
    }
    float* po = p.part_o + (unit * kTileQ + ql) * D + 4 * lq;
#pragma unroll
    for (int n = 0; n < NO; ++n)
      *reinterpret_cast<float4*>(po + n * 16) = make_float4(o[n][0], o[n][1], o[n][2], o[n][3]);
    return;
  }
  // O / L, scattered to the query's own row (4 dimensions per lane and output tile)
  if (qi < kk) {
    const float il = 1.f / L;
    uint16_t* dst = p.out + (size_t)h * plane + (seq0 + (size_t)sm.qpos[wave * 16 + lr]) * D + 4 * lq;
#pragma unroll
    for (int n = 0; n < NO; ++n) {
      uint2 w;
      w.x = (uint32_t)tile_bf16(o[n][0] * il) | ((uint32_t)tile_bf16(o[n][1] * il) << 16);
      w.y = (uint32_t)tile_bf16(o[n][2] * il) | ((uint32_t)tile_bf16(o[n][3] * il) << 16);
      *reinterpret_cast<uint2*>(dst + n * 16) = w;
    }
  }
}

// Merge of the key splits of one (row, query block): O = sum_s o_s 2^(m_s - M) / L with
// M = max_s m_s and L = sum_s l_s 2^(m_s - M), written as bf16 to the queries' rows.
// A wave takes 4 queries at a time, a lane DL adjacent dimensions of each; every load
// of the 4 queries is issued before the first use.
template <int D>
__global__ __launch_bounds__(kTileWaves * 64) void k_tsa_merge(TsaParams p) {
  constexpr int DL = D / 64;
  constexpr int QW = 4;                                        // queries per step of a wave
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int row = blockIdx.x / p.qtiles, qt = blockIdx.x % p.qtiles;
  const int b = row / p.Hq, h = row % p.Hq;
  const int kk = p.kk, q0 = qt * kTileQ;
  const int nkeys = p.causal ? min(q0 + kTileQ, kk) : kk;
  const int ns = (nkeys + p.split_keys - 1) / p.split_keys;   // splits that ran (1..8)
  const int32_t* I = p.idx + (size_t)row * kk;
  const size_t base = ((size_t)row * p.qtiles + qt) * p.nsplit;
  uint16_t* out = p.out + (size_t)h * p.B * p.T * D + (size_t)b * p.T * D;
  for (int qs = wave * QW; qs < kTileQ; qs += kTileWaves * QW) {
    float ml[QW][8][2], po[QW][8][DL];
#pragma unroll
    for (int j = 0; j < QW; ++j)
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const size_t u = (base + min(s, ns - 1)) * kTileQ + qs + j;
        ml[j][s][0] = p.part_ml[u * 2];
        ml[j][s][1] = p.part_ml[u * 2 + 1];
#pragma unroll
        for (int e = 0; e < DL; ++e) po[j][s][e] = p.part_o[u * D + lane * DL + e];
      }
#pragma unroll
    for (int j = 0; j < QW; ++j) {
      const int qi = q0 + qs + j;
      if (qi >= kk) break;
      float M = -LD_INF;
#pragma unroll
      for (int s = 0; s < 8; ++s) M = (s < ns) ? fmaxf(M, ml[j][s][0]) : M;
      const float mu = (M == -LD_INF) ? 0.f : M;
      float L = 0.f, acc[DL];
#pragma unroll
      for (int e = 0; e < DL; ++e) acc[e] = 0.f;
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        if (s < ns) {
          const float w = exp2_fast(ml[j][s][0] - mu);         // 0 for a split without keys
          L = fmaf(ml[j][s][1], w, L);
#pragma unroll
          for (int e = 0; e < DL; ++e) acc[e] = fmaf(po[j][s][e], w, acc[e]);
        }
      }
      const int pos = min(max(I[qi], 0), p.T - 1);
      const float il = 1.f / L;
#pragma unroll
      for (int e = 0; e < DL; ++e) out[(size_t)pos * D + lane * DL + e] = tile_bf16(acc[e] * il);
    }
  }
}

}  // namespace

hipError_t launch_tsa(const TsaParams& p, hipStream_t st) {
  const dim3 grid((unsigned)((size_t)p.B * p.Hq * p.qtiles * p.nsplit)), block(kTileWaves * 64);
  if (p.D == 128)
    hipLaunchKernelGGL(k_tsa<128>, grid, block, 0, st, p);
  else
    hipLaunchKernelGGL(k_tsa<64>, grid, block, 0, st, p);
  if (p.nsplit > 1) {
    const dim3 mgrid((unsigned)((size_t)p.B * p.Hq * p.qtiles));
    if (p.D == 128)
      hipLaunchKernelGGL(k_tsa_merge<128>, mgrid, block, 0, st, p);
    else
      hipLaunchKernelGGL(k_tsa_merge<64>, mgrid, block, 0, st, p);
  }
  return hipGetLastError();
}

int tsa_queries_per_block() { return kTileQ; }

// Key splits only when the (row, query block) workgroups alone would leave most of
// the chip idle (fewer than 512 of them): splits of kTsaSplitKeys keys or more, at
// most 8 per query block, while their partials take at most 256 MiB. Otherwise one
// workgroup walks all keys (measured faster than splitting plus the merge once the
// chip is full).
void tsa_splits(int64_t rows, int kk, int D, int* nsplit, int* split_keys, size_t* part_bytes) {
  constexpr int kTsaSplitKeys = 256;
  const int64_t qtiles = (kk + kTileQ - 1) / kTileQ;
  int ks = max(kTsaSplitKeys, ((kk + 7) / 8 + kTileKeys - 1) / kTileKeys * kTileKeys);
  int ns = (kk + ks - 1) / ks;
  size_t bytes = (size_t)rows * qtiles * ns * kTileQ * (D + 2) * 4;
  if (ns <= 1 || rows * qtiles >= 512 || bytes > ((size_t)256 << 20)) {
    ns = 1;
    ks = kk;
    bytes = 0;
  }
  *nsplit = ns;
  *split_keys = ks;
  *part_bytes = bytes;
}

}  // namespace ld
