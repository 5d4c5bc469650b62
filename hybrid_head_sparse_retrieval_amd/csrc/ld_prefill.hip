// The hybrid-head layer over a causal prefill of T prompt tokens per sequence: the
// extension to the prefill stage that the LycheeDecode summary page (arXiv 2602.04541)
// names in its future-work paragraph, with method steps (3) and (4) read for T query
// rows at once. Query row t sees prompt tokens 0..t of its own sequence.
//  - k_prefill_attn: a retrieval head's row t attends to every token up to t; a sparse
//    head's row t attends to the tokens of its set S (ascending) up to t, and a row that
//    sees none of them is zero. Retrieval rows also leave their log-sum-exp (log2
//    units), which the column sums need.
//  - k_prefill_colsum: for every retrieval head, the column sums of its attention
//    matrix A (the attention mass each token receives over the prompt). argsTopK of
//    these sums is the head's next S (the selection launches of the decode step).
//
// Both are dense contractions on the matrix cores, on the tile scheme of ld_tile.h. The
// attention kernel is the dense stage of the token-sparse kernel with the prompt rows
// as queries and, as keys, either every earlier token or the gathered tokens of S. The
// column-sum kernel swaps the roles: a workgroup holds 64 keys in registers and walks
// the query rows that see them in tiles staged through LDS; each score becomes a
// probability with the row's final log-sum-exp and is summed per key.

#include <type_traits>

#include "ld_tile.h"

namespace ld {

namespace {

// 8 waves of 16 rows: a workgroup's 128 prompt rows (or, for the column sums, 128 keys)
// share every K/V (or Q) tile it loads, which halves the re-reads against 64 rows; with
// about 200 VGPRs per lane a compute unit holds one such workgroup, the same waves as
// two of 4.
constexpr int kPfWaves = 8;
constexpr int kPfRows = 16 * kPfWaves;

template <int D>
__global__ __launch_bounds__(kPfWaves * 64) void k_prefill_attn(PrefillParams p) {
  using Smem = TileSmem<D>;
  constexpr int NT = kPfWaves * 64;
  constexpr int KS = Smem::KS;
  constexpr int KC = D / 32;                                  // k-steps over the head dimension
  constexpr int NO = D / 16;                                  // 16-dim output tiles
  __shared__ Smem sm;
  __shared__ int cnt;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lq = lane >> 4;
  // row (b, h) and query block; blocks go out in the order 0, 1, .., then from the last
  // one down, each over all rows, so that workgroups sharing a compute unit pair a
  // short block with a long one. The rows rotate by one per block, so that a row's
  // blocks do not all land on one XCD (consecutive workgroup ids take turns on them)
  const int rows = p.B * p.Hq;
  const int jq = blockIdx.x / rows, row = (blockIdx.x % rows + jq) % rows;
  const int half = (p.qtiles + 1) / 2;
  const int qt = jq < half ? jq : p.qtiles - 1 - (jq - half);
  const int b = row / p.Hq, h = row % p.Hq, g = h / (p.Hq / p.Hkv);
  const bool ret = (p.retrieval >> h) & 1ull;
  const int T = p.T;
  const size_t seq0 = (size_t)b * T;
  const size_t plane = (size_t)p.B * T * D;                   // one head's rows
  const uint16_t* Qh = p.q + (size_t)h * plane + seq0 * D;
  const uint16_t* Kg = p.k + (size_t)g * plane + seq0 * D;
  const uint16_t* Vg = p.v + (size_t)g * plane + seq0 * D;
  const int q0 = qt * kPfRows;
  const int qi = q0 + wave * 16 + lr;                         // this lane's query row
  const int lim = min(q0 + kPfRows, T) - 1;                   // the block's last row
  uint4 qa[KC];
#pragma unroll
  for (int kc = 0; kc < KC; ++kc)
    qa[kc] = (qi < T) ? *reinterpret_cast<const uint4*>(Qh + (size_t)qi * D + kc * 32 + 8 * lq)
                      : make_uint4(0, 0, 0, 0);
  const int32_t* Srow = p.s_in + (size_t)row * p.kk;          // read for sparse rows only
  const float sl = p.scale * kTileLog2e;
  // S^T = K Q^T gives lane (lr, lq) the scores of query lr against keys 4 lq + r of each
  // 16-key half (the operand layout of P^T in O^T = V^T P^T); lanes lr, lr + 16, lr + 32,
  // lr + 48 share a query
  float m = -LD_INF, lsum = 0.f;
  tile_f32x4_t o[NO];
#pragma unroll
  for (int n = 0; n < NO; ++n) o[n] = tile_f32x4_t{0.f, 0.f, 0.f, 0.f};
  TileRegs<D, kPfWaves> R;

  // keys in chunks of kTileIdx positions staged in LDS: a retrieval row's keys are the
  // tokens 0 .. lim; a sparse row's, the entries of S up to lim (a prefix, S ascending)
  for (int cb = 0;; cb += kTileIdx) {
    const int avail = ret ? min(kTileIdx, lim + 1 - cb) : min(kTileIdx, p.kk - cb);
    if (avail <= 0) break;                                    // the same in every thread
    __syncthreads();                                          // the previous chunk is done with LDS
    if (tid == 0) cnt = 0;
    __syncthreads();
    int mine = 0;
    for (int i = tid; i < avail; i += NT) {
      const int pos = ret ? cb + i : min(max(Srow[cb + i], 0), T - 1);
      sm.kidx[i] = pos;
      mine += pos <= lim;
    }
    if (!ret) atomicAdd(&cnt, mine);
    __syncthreads();
    const int nk = ret ? avail : cnt;                         // keys of the chunk the block may see
    if (nk == 0) break;
    const int nt = (nk + kTileKeys - 1) / kTileKeys;
    tile_load<D, kPfWaves>(Kg, Vg, sm.kidx, nk, 0, tid, R);
    tile_store<D, kPfWaves>(sm, 0, tid, R);
    if (nt > 1) tile_load<D, kPfWaves>(Kg, Vg, sm.kidx, nk, 1, tid, R);
    auto step = [&](int t, auto bufc) {
      constexpr int buf = decltype(bufc)::value;
      __syncthreads();                           // tile t is in buf; the other buffer is free
      if (t + 1 < nt) tile_store<D, kPfWaves>(sm, buf ^ 1, tid, R);
      if (t + 2 < nt) tile_load<D, kPfWaves>(Kg, Vg, sm.kidx, nk, t + 2, tid, R);
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
      const int lt0 = t * kTileKeys;             // the tile's first key within the chunk
      float x[NST][4];
      // the checked form compares every key's position with the query's (tiles at the end
      // of the chunk or reaching past the wave's first query); the others skip it
      auto scores = [&](auto masked) {
#pragma unroll
        for (int st = 0; st < NST; ++st)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            if constexpr (decltype(masked)::value) {
              const int lk = lt0 + 32 * (st >> 1) + 8 * lq + 4 * (st & 1) + r;
              const bool ok = lk < nk && sm.kidx[min(lk, nk - 1)] <= qi;
              x[st][r] = ok ? s[st][r] * sl : -LD_INF;
            } else {
              x[st][r] = s[st][r] * sl;
            }
          }
      };
      if (lt0 + kTileKeys <= nk && sm.kidx[lt0 + kTileKeys - 1] <= q0 + wave * 16)
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
      if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
#pragma unroll
        for (int n = 0; n < NO; ++n)
#pragma unroll
          for (int r = 0; r < 4; ++r) o[n][r] *= alpha;
      }
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
    if (nk < avail) break;                       // the rest of S lies past the block
  }
  const float L = add_xor32(add_xor16(lsum));   // the query's sum over its four lanes
  if (qi >= T) return;
  // O / L to the query's row; a row that saw no key (L = 0) is zero
  const float il = L > 0.f ? 1.f / L : 0.f;
  uint16_t* dst = p.out + (size_t)h * plane + (seq0 + (size_t)qi) * D + 4 * lq;
#pragma unroll
  for (int n = 0; n < NO; ++n) {
    uint2 w;
    w.x = (uint32_t)tile_bf16(o[n][0] * il) | ((uint32_t)tile_bf16(o[n][1] * il) << 16);
    w.y = (uint32_t)tile_bf16(o[n][2] * il) | ((uint32_t)tile_bf16(o[n][3] * il) << 16);
    *reinterpret_cast<uint2*>(dst + n * 16) = w;
  }
  if (ret && lq == 0 && p.lse) p.lse[(size_t)row * T + qi] = m + __log2f(L);
}

// ---------------------------------------------------------------- column sums

template <int D>
struct ColSmem {
  static constexpr int KS = D + 8;
  alignas(16) uint16_t qt[2][kTileKeys * KS];   // two tiles of 64 query rows (tile_krow order)
  float ls[2][kTileKeys];                       // their log-sum-exp (log2 units)
};

template <int D>
struct ColRegs {
  static constexpr int LPT = kTileKeys * (D / 8) / (kPfWaves * 64);
  uint4 r[LPT];
  float ls;
};

template <int D>
__device__ __forceinline__ void col_load(const uint16_t* Qh, const float* lse, int T, int t0, int tid,
                                         ColRegs<D>& R) {
#pragma unroll
  for (int i = 0; i < ColRegs<D>::LPT; ++i) {
    const int u = tid + i * kPfWaves * 64;
    const int r = u / (D / 8), c = u % (D / 8);
    R.r[i] = *reinterpret_cast<const uint4*>(Qh + (size_t)min(t0 + r, T - 1) * D + c * 8);
  }
  if (tid < kTileKeys) R.ls = (t0 + tid < T) ? lse[t0 + tid] : LD_INF;
}

template <int D>
__device__ __forceinline__ void col_store(ColSmem<D>& sm, int buf, int tid, const ColRegs<D>& R) {
#pragma unroll
  for (int i = 0; i < ColRegs<D>::LPT; ++i) {
    const int u = tid + i * kPfWaves * 64;
    const int r = u / (D / 8), c = u % (D / 8);
    *reinterpret_cast<uint4*>(&sm.qt[buf][tile_krow(r) * ColSmem<D>::KS + c * 8]) =
        make_uint4(R.r[i].x, R.r[i].y, R.r[i].z, R.r[i].w);
  }
  if (tid < kTileKeys) sm.ls[buf][tid] = R.ls;
}

template <int D>
__global__ __launch_bounds__(kPfWaves * 64) void k_prefill_colsum(PrefillParams p) {
  using Smem = ColSmem<D>;
  constexpr int KS = Smem::KS;
  constexpr int KC = D / 32;
  constexpr int NST = kTileKeys / 16;
  __shared__ Smem sm;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lq = lane >> 4;
  // retrieval row rr = b * nret + i and key block kb; the first key blocks (seen by the
  // most query rows) go out first
  const int rrows = p.B * p.nret;
  const int kb = blockIdx.x / rrows, rr = (blockIdx.x % rrows + kb) % rrows;   // rotated as above
  const int b = rr / p.nret, h = p.heads[rr % p.nret], g = h / (p.Hq / p.Hkv);
  const int row = b * p.Hq + h;
  const int T = p.T;
  const size_t seq0 = (size_t)b * T;
  const size_t plane = (size_t)p.B * T * D;
  const uint16_t* Qh = p.q + (size_t)h * plane + seq0 * D;
  const uint16_t* Kg = p.k + (size_t)g * plane + seq0 * D;
  const float* lse = p.lse + (size_t)row * T;
  const int j = kb * kPfRows + wave * 16 + lr;                // this lane's key
  uint4 ka[KC];
#pragma unroll
  for (int kc = 0; kc < KC; ++kc)
    ka[kc] = (j < T) ? *reinterpret_cast<const uint4*>(Kg + (size_t)j * D + kc * 32 + 8 * lq)
                     : make_uint4(0, 0, 0, 0);
  const float sl = p.scale * kTileLog2e;
  float acc = 0.f;
  const int t_first = kb * (kPfRows / kTileKeys);             // 64-row query tiles that see the block
  const int nt = (T + kTileKeys - 1) / kTileKeys - t_first;
  ColRegs<D> R;
  col_load<D>(Qh, lse, T, t_first * kTileKeys, tid, R);
  col_store<D>(sm, 0, tid, R);
  if (nt > 1) col_load<D>(Qh, lse, T, (t_first + 1) * kTileKeys, tid, R);
  auto step = [&](int t, auto bufc) {
    constexpr int buf = decltype(bufc)::value;
    __syncthreads();
    if (t + 1 < nt) col_store<D>(sm, buf ^ 1, tid, R);
    if (t + 2 < nt) col_load<D>(Qh, lse, T, (t_first + t + 2) * kTileKeys, tid, R);
    // element r of s[st]: query row t0 + 32 (st >> 1) + 8 lq + 4 (st & 1) + r against key j
    tile_f32x4_t s[NST];
#pragma unroll
    for (int st = 0; st < NST; ++st) {
      s[st] = tile_f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        const uint4 qv = *reinterpret_cast<const uint4*>(&sm.qt[buf][(st * 16 + lr) * KS + kc * 32 + 8 * lq]);
        s[st] = mfma16(qv, ka[kc], s[st]);
      }
    }
    const int t0 = (t_first + t) * kTileKeys;
    // rows past T carry an infinite log-sum-exp (weight 0); rows before the key are
    // masked on the tiles that overlap the key block only
    const bool diag = t < kPfRows / kTileKeys;
#pragma unroll
    for (int st = 0; st < NST; ++st)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int lt = 32 * (st >> 1) + 8 * lq + 4 * (st & 1) + r;
        const float w = exp2_fast(s[st][r] * sl - sm.ls[buf][lt]);
        acc += (diag && t0 + lt < j) ? 0.f : w;
      }
  };
  for (int t = 0; t < nt; t += 2) {
    step(t, std::integral_constant<int, 0>{});
    if (t + 1 < nt) step(t + 1, std::integral_constant<int, 1>{});
  }
  acc = add_xor32(add_xor16(acc));                            // the key's four lanes
  if (lq == 0 && j < T) p.imp[(size_t)row * T + j] = acc;
}

}  // namespace

int prefill_rows_per_block() { return kPfRows; }

hipError_t launch_prefill_attention(const PrefillParams& p, hipStream_t st) {
  const dim3 grid((unsigned)((size_t)p.B * p.Hq * p.qtiles)), block(kPfWaves * 64);
  if (p.D == 128)
    hipLaunchKernelGGL(k_prefill_attn<128>, grid, block, 0, st, p);
  else
    hipLaunchKernelGGL(k_prefill_attn<64>, grid, block, 0, st, p);
  return hipGetLastError();
}

hipError_t launch_prefill_colsum(const PrefillParams& p, hipStream_t st) {
  const dim3 grid((unsigned)((size_t)p.B * p.nret * p.qtiles)), block(kPfWaves * 64);
  if (p.D == 128)
    hipLaunchKernelGGL(k_prefill_colsum<128>, grid, block, 0, st, p);
  else
    hipLaunchKernelGGL(k_prefill_colsum<64>, grid, block, 0, st, p);
  return hipGetLastError();
}

}  // namespace ld
