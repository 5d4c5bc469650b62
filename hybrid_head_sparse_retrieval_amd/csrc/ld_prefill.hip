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
// column-sum kernel swaps the roles: a workgroup holds 128 keys in registers and walks
// the query rows that see them in tiles staged through LDS; each score becomes a
// probability with the row's final log-sum-exp and is summed per key.

#include <type_traits>

#include "ld_tile.h"

namespace ld {

namespace {

// The attention workgroup: 4 waves of 32 prompt rows, two 16-row blocks per wave that
// share every operand read from LDS (each K and V tile read feeds two matrix products),
// 128 rows per workgroup sharing every K/V tile loaded. The column-sum workgroup alike:
// 4 waves of 32 keys (two 16-key blocks), 128 keys per workgroup.
constexpr int kPfWaves = 4;
constexpr int kPfBlocks = 2;                                  // 16-row blocks per wave
constexpr int kPfRows = 16 * kPfBlocks * kPfWaves;
constexpr int kColWaves = 4;

template <int D>
__global__ __launch_bounds__(kPfWaves * 64) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_prefill_attn(PrefillParams p) {
  using Smem = TileSmem<D>;
  constexpr int NT = kPfWaves * 64;
  constexpr int NB = kPfBlocks;
  constexpr int KS = Smem::KS;
  constexpr int KC = D / 32;                                  // k-steps over the head dimension
  constexpr int NO = D / 16;                                  // 16-dim output tiles
  constexpr int NST = kTileKeys / 16;
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
  const int w0 = q0 + wave * 16 * NB;                         // the wave's first row
  const int lim = min(q0 + kPfRows, T) - 1;                   // the block's last row
  int qi[NB];                                                 // this lane's query row, per block
  uint4 qa[NB][KC];
#pragma unroll
  for (int bb = 0; bb < NB; ++bb) {
    qi[bb] = w0 + 16 * bb + lr;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc)
      qa[bb][kc] = (qi[bb] < T) ? *reinterpret_cast<const uint4*>(Qh + (size_t)qi[bb] * D + kc * 32 + 8 * lq)
                                : make_uint4(0, 0, 0, 0);
  }
  const int32_t* Srow = p.s_in + (size_t)row * p.kk;          // read for sparse rows only
  const float sl = p.scale * kTileLog2e;
  // S^T = K Q^T gives lane (lr, lq) the scores of query lr of each block against keys
  // 4 lq + r of each 16-key half (the operand layout of P^T in O^T = V^T P^T); lanes lr,
  // lr + 16, lr + 32, lr + 48 share a query
  float m[NB], lsum[NB];
  tile_f32x4_t o[NB][NO];
#pragma unroll
  for (int bb = 0; bb < NB; ++bb) {
    m[bb] = -LD_INF;
    lsum[bb] = 0.f;
#pragma unroll
    for (int n = 0; n < NO; ++n) o[bb][n] = tile_f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
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
      tile_f32x4_t s[NB][NST];
#pragma unroll
      for (int st = 0; st < NST; ++st) {
#pragma unroll
        for (int bb = 0; bb < NB; ++bb) s[bb][st] = tile_f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
          const uint4 ka =
              *reinterpret_cast<const uint4*>(&sm.kt[buf][(st * 16 + lr) * KS + kc * 32 + 8 * lq]);
#pragma unroll
          for (int bb = 0; bb < NB; ++bb) s[bb][st] = mfma16(ka, qa[bb][kc], s[bb][st]);
        }
      }
      const int lt0 = t * kTileKeys;             // the tile's first key within the chunk
      // the checked form compares every key's position with the query's (tiles at the end
      // of the chunk or reaching past the wave's first row); the others skip it
      const bool plain = lt0 + kTileKeys <= nk && sm.kidx[lt0 + kTileKeys - 1] <= w0;
      int kpos[NST][4];
      if (!plain) {
#pragma unroll
        for (int st = 0; st < NST; ++st)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int lk = lt0 + 32 * (st >> 1) + 8 * lq + 4 * (st & 1) + r;
            kpos[st][r] = lk < nk ? sm.kidx[min(lk, nk - 1)] : 0x7fffffff;
          }
      }
      uint4 pb[NB][NST / 2];
#pragma unroll
      for (int bb = 0; bb < NB; ++bb) {
        float x[NST][4];
#pragma unroll
        for (int st = 0; st < NST; ++st)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            x[st][r] = (plain || kpos[st][r] <= qi[bb]) ? s[bb][st][r] * sl : -LD_INF;
        float mt = -LD_INF;
#pragma unroll
        for (int st = 0; st < NST; ++st)
          mt = fmaxf(mt, fmaxf(fmaxf(x[st][0], x[st][1]), fmaxf(x[st][2], x[st][3])));
        mt = max_xor32(max_xor16(mt));           // over the query's four lanes
        const float mn = fmaxf(m[bb], mt);
        const float mu = (mn == -LD_INF) ? 0.f : mn;
        const float alpha = (mn > m[bb]) ? exp2_fast(m[bb] - mu) : 1.f;   // 0 while nothing was allowed
        float pr[NST][4];
        float ps = 0.f;
#pragma unroll
        for (int st = 0; st < NST; ++st)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            pr[st][r] = exp2_fast(x[st][r] - mu);
            ps += pr[st][r];
          }
        lsum[bb] = fmaf(lsum[bb], alpha, ps);
        m[bb] = mn;
        if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
#pragma unroll
          for (int n = 0; n < NO; ++n)
#pragma unroll
            for (int r = 0; r < 4; ++r) o[bb][n][r] *= alpha;
        }
#pragma unroll
        for (int hh = 0; hh < NST / 2; ++hh) {
          pb[bb][hh].x = (uint32_t)tile_bf16(pr[2 * hh][0]) | ((uint32_t)tile_bf16(pr[2 * hh][1]) << 16);
          pb[bb][hh].y = (uint32_t)tile_bf16(pr[2 * hh][2]) | ((uint32_t)tile_bf16(pr[2 * hh][3]) << 16);
          pb[bb][hh].z = (uint32_t)tile_bf16(pr[2 * hh + 1][0]) | ((uint32_t)tile_bf16(pr[2 * hh + 1][1]) << 16);
          pb[bb][hh].w = (uint32_t)tile_bf16(pr[2 * hh + 1][2]) | ((uint32_t)tile_bf16(pr[2 * hh + 1][3]) << 16);
        }
      }
      // O^T += V^T P^T: each V operand read from LDS feeds both blocks
#pragma unroll
      for (int hh = 0; hh < NST / 2; ++hh)
#pragma unroll
        for (int n = 0; n < NO; ++n) {
          const uint4 va = *reinterpret_cast<const uint4*>(&sm.vt[buf][Smem::vrow(n * 16 + lr) + 32 * hh + 8 * lq]);
#pragma unroll
          for (int bb = 0; bb < NB; ++bb) o[bb][n] = mfma16(va, pb[bb][hh], o[bb][n]);
        }
    };
    for (int t = 0; t < nt; t += 2) {
      step(t, std::integral_constant<int, 0>{});
      if (t + 1 < nt) step(t + 1, std::integral_constant<int, 1>{});
    }
    if (nk < avail) break;                       // the rest of S lies past the block
  }
#pragma unroll
  for (int bb = 0; bb < NB; ++bb) {
    const float L = add_xor32(add_xor16(lsum[bb]));   // the query's sum over its four lanes
    if (qi[bb] >= T) continue;
    // O / L to the query's row; a row that saw no key (L = 0) is zero
    const float il = L > 0.f ? 1.f / L : 0.f;
    uint16_t* dst = p.out + (size_t)h * plane + (seq0 + (size_t)qi[bb]) * D + 4 * lq;
#pragma unroll
    for (int n = 0; n < NO; ++n) {
      uint2 w;
      w.x = (uint32_t)tile_bf16(o[bb][n][0] * il) | ((uint32_t)tile_bf16(o[bb][n][1] * il) << 16);
      w.y = (uint32_t)tile_bf16(o[bb][n][2] * il) | ((uint32_t)tile_bf16(o[bb][n][3] * il) << 16);
      *reinterpret_cast<uint2*>(dst + n * 16) = w;
    }
    if (ret && lq == 0 && p.lse) p.lse[(size_t)row * T + qi[bb]] = m[bb] + __log2f(L);
  }
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
  static constexpr int LPT = kTileKeys * (D / 8) / (kColWaves * 64);
  uint4 r[LPT];
  float ls;
};

template <int D>
__device__ __forceinline__ void col_load(const uint16_t* Qh, const float* lse, int T, int t0, int tid,
                                         ColRegs<D>& R) {
#pragma unroll
  for (int i = 0; i < ColRegs<D>::LPT; ++i) {
    const int u = tid + i * kColWaves * 64;
    const int r = u / (D / 8), c = u % (D / 8);
    R.r[i] = *reinterpret_cast<const uint4*>(Qh + (size_t)min(t0 + r, T - 1) * D + c * 8);
  }
  if (tid < kTileKeys) R.ls = (t0 + tid < T) ? lse[t0 + tid] : LD_INF;
}

template <int D>
__device__ __forceinline__ void col_store(ColSmem<D>& sm, int buf, int tid, const ColRegs<D>& R) {
#pragma unroll
  for (int i = 0; i < ColRegs<D>::LPT; ++i) {
    const int u = tid + i * kColWaves * 64;
    const int r = u / (D / 8), c = u % (D / 8);
    *reinterpret_cast<uint4*>(&sm.qt[buf][tile_krow(r) * ColSmem<D>::KS + c * 8]) =
        make_uint4(R.r[i].x, R.r[i].y, R.r[i].z, R.r[i].w);
  }
  if (tid < kTileKeys) sm.ls[buf][tid] = R.ls;
}

template <int D>
__global__ __launch_bounds__(kColWaves * 64) void k_prefill_colsum(PrefillParams p) {
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
  constexpr int NB = kPfBlocks;
  int j[NB];                                                  // this lane's key, per block
  uint4 ka[NB][KC];
#pragma unroll
  for (int bb = 0; bb < NB; ++bb) {
    j[bb] = kb * kPfRows + wave * 16 * NB + 16 * bb + lr;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc)
      ka[bb][kc] = (j[bb] < T) ? *reinterpret_cast<const uint4*>(Kg + (size_t)j[bb] * D + kc * 32 + 8 * lq)
                               : make_uint4(0, 0, 0, 0);
  }
  const float sl = p.scale * kTileLog2e;
  float acc[NB];
#pragma unroll
  for (int bb = 0; bb < NB; ++bb) acc[bb] = 0.f;
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
    // element r of s[bb][st]: query row t0 + 32 (st >> 1) + 8 lq + 4 (st & 1) + r against
    // key j[bb]; each operand read from LDS feeds both key blocks
    tile_f32x4_t s[NB][NST];
#pragma unroll
    for (int st = 0; st < NST; ++st) {
#pragma unroll
      for (int bb = 0; bb < NB; ++bb) s[bb][st] = tile_f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        const uint4 qv = *reinterpret_cast<const uint4*>(&sm.qt[buf][(st * 16 + lr) * KS + kc * 32 + 8 * lq]);
#pragma unroll
        for (int bb = 0; bb < NB; ++bb) s[bb][st] = mfma16(qv, ka[bb][kc], s[bb][st]);
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
        const float ls = sm.ls[buf][lt];
#pragma unroll
        for (int bb = 0; bb < NB; ++bb) {
          const float w = exp2_fast(s[bb][st][r] * sl - ls);
          acc[bb] += (diag && t0 + lt < j[bb]) ? 0.f : w;
        }
      }
  };
  for (int t = 0; t < nt; t += 2) {
    step(t, std::integral_constant<int, 0>{});
    if (t + 1 < nt) step(t + 1, std::integral_constant<int, 1>{});
  }
#pragma unroll
  for (int bb = 0; bb < NB; ++bb) {
    const float a = add_xor32(add_xor16(acc[bb]));           // the key's four lanes
    if (lq == 0 && j[bb] < T) p.imp[(size_t)row * T + j[bb]] = a;
  }
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
  const dim3 grid((unsigned)((size_t)p.B * p.nret * p.qtiles)), block(kColWaves * 64);
  if (p.D == 128)
    hipLaunchKernelGGL(k_prefill_colsum<128>, grid, block, 0, st, p);
  else
    hipLaunchKernelGGL(k_prefill_colsum<64>, grid, block, 0, st, p);
  return hipGetLastError();
}

}  // namespace ld
