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
//
// Per wave, rows are consumed in 16-row tiles:
//   q.K   on the matrix cores: v_mfma_f32_16x16x32_bf16 with the K tile as the A
//         operand (16 rows x 32 dims, loaded straight from HBM in operand layout) and
//         the group's queries as the B operand (heads padded to 16 columns). bf16
//         products are exact, accumulation is fp32.
//   softmax in the MFMA output layout (lane = head column, 4 rows); the running max
//         of each head is wave-uniform; the probabilities go through LDS.
//   P.V   on the vector ALU in fp32 (8 lanes per V row, 16 dims per lane).
// The next chunk's K and V are loaded while the current one is computed. Each
// workgroup writes one partial (max in log2 units, sum, unnormalised output) per
// head; the last workgroup of a (b, g) (integer ticket, device-coherent stores and
// loads, no cache-wide fences) merges them into O and, when selection is requested,
// turns the fused first-digit histogram of each retrieval head into the first
// selection digit for the argsTopK kernels.

#include <atomic>

#include "ld_device.h"

namespace ld {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kTile = 16;        // rows per MFMA tile
constexpr int kMaxTPC = 2;       // tiles per chunk per wave, at most
constexpr int kChunkRows = kTile * kMaxTPC;
constexpr int kCandLds = 8192;     // selection candidates staged in LDS

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4_t mfma_bf16(const uint4& a, const uint4& b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ float4 ld_dev4_b(__amdgpu_buffer_rsrc_t r, int byte_off) {
  const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, kSc1);
  return make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z), __uint_as_float(v.w));
}
__device__ __forceinline__ void st_dev4_b(__amdgpu_buffer_rsrc_t r, int byte_off, float4 x) {
  u32x4_t v = {__float_as_uint(x.x), __float_as_uint(x.y), __float_as_uint(x.z), __float_as_uint(x.w)};
  __builtin_amdgcn_raw_buffer_store_b128(v, r, byte_off, 0, kSc1);
}

// Workgroup of NW waves. After the in-wave reduction each wave keeps RP row parts.
template <int NW>
struct WaveCfg {
  static constexpr int NT = 64 * NW;
  static constexpr int RP = 16 / NW;        // row parts per wave written to LDS (4 or 2)
};

template <int D, int G, int NW>
struct AttnSmem {
  static constexpr int RP = WaveCfg<NW>::RP;
  static constexpr int COLS = G * (D / 4);  // float4 output columns
  static constexpr int TPCOL = (64 * NW) / COLS >= 4 ? 4 : ((64 * NW) / COLS >= 2 ? 2 : 1);
  uint8_t hmp[kMaxSplitRows];        // membership mask (bit j = head g*G+j) per visit position
  uint16_t list[kMaxSplitRows];      // token row (within the tile) of each visit position
  int wcnt[NW];
  int tmp4[NW][4];
  int poff[kMaxParts + 1];           // selection: candidate sub-list offsets, part order
  int pcnt[kMaxParts];               // selection: each part's keys above bin b1
  int misc[4];
  uint64_t relw;                     // release word seen by thread 0
  uint32_t res[2];
  int scan[NW][kMaxSplitRows / (64 * NW) / 2 > 2 ? kMaxSplitRows / (64 * NW) / 2 : 2];   // wave totals of scans
  int cnt4[NW][2];
  int ncnt[kRep];                    // candidate counts of the sub-lists
  int pages[kMaxSplitRows / 16 + 1]; // paged KV: page ids of the split's rows
  uint16_t blk[kMaxSplitRows / 64];  // block sets: the split's share of its group's union of 64-row blocks
  float pl[NW][kChunkRows][G];       // per wave: probabilities of the chunk's rows (up to)
  union {
    uint32_t hist[G][kHist1Bins];
    struct {
      uint32_t hist[kHist2Bins + kHist3Bins];
      uint32_t cand[kCandLds];       // the row's candidates, when they fit
    } sel;
    struct {
      float acc[NW][RP][G * D];      // [wave][row part][head*D + dim]
      float m[NW][G];
      float l[NW][G];
    } red;
    struct {
      float w[G][kMaxSplits];        // split maxima, then split weights
      float lp[G][kMaxSplits];       // split sums
      float inv_l[G];
      float mtot[G];
      float ltot[G];
      float4 part[TPCOL > 1 ? TPCOL - 1 : 1][COLS];   // partial column sums of the merge
    } cmb;
  } u;
};

// Four output columns of row `row` (b * Hq + h): o * il as bf16, or, with the HySparse
// gate set, w * o * il + (1 - w) * o_win with w = sigmoid(gate[row]).
template <int D>
__device__ __forceinline__ void store_o(const AttnParams& p, int row, int d0, float4 o, float il) {
  float x = o.x * il, y = o.y * il, z = o.z * il, t = o.w * il;
  if (p.gate) {
    const float w = 1.f / (1.f + expf(-p.gate[row]));
    const float4 c = *reinterpret_cast<const float4*>(p.o_win + (size_t)row * D + d0);
    x = fmaf(w, x - c.x, c.x); y = fmaf(w, y - c.y, c.y);
    z = fmaf(w, z - c.z, c.z); t = fmaf(w, t - c.w, c.w);
  }
  ushort4 r;
  r.x = f32_to_bf16(x); r.y = f32_to_bf16(y); r.z = f32_to_bf16(z); r.w = f32_to_bf16(t);
  *reinterpret_cast<ushort4*>(p.out + (size_t)row * D + d0) = r;
}

// Merge `cnt` split partials (max in log2 units, sum, unnormalised output) of every
// active head of the group, taken from src_ml/src_acc at positions s0.. of each head's
// row of `stride` partials. FINAL: write O = sum acc_p w_p / sum l_p w_p as bf16.
// Otherwise: write one merged partial at position `upos` of the level-1 arrays
// (device-coherent, for the merge that follows in another workgroup).
template <int D, int G, int NW, bool FINAL>
__device__ __forceinline__ void merge_splits(AttnSmem<D, G, NW>& sm, const AttnParams& p, uint32_t act,
                                             int hq0, const float* src_ml, const float* src_acc,
                                             int stride, int s0, int cnt, float* dst_ml, float* dst_acc,
                                             int upos) {
  using Smem = AttnSmem<D, G, NW>;
  constexpr int NT = 64 * NW;
  constexpr int COLS = Smem::COLS;
  constexpr int TPCOL = Smem::TPCOL;    // threads per column, each over a share of the splits
  constexpr int PF = 32;                // partial columns fetched per round
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = tid % COLS, part = tid / COLS;
  const int j = col / (D / 4), d0 = (col % (D / 4)) * 4;
  const bool live = part < TPCOL && (act >> j & 1u);
  const int s_lo = (cnt * part) / TPCOL;
  const int s_hi = (cnt * (part + 1)) / TPCOL;
  // one workgroup-uniform resource (a per-lane base would need a waterfall loop)
  const __amdgpu_buffer_rsrc_t rr = rsrc(src_acc + ((size_t)hq0 * stride + s0) * D);
  const int jrow = j * stride * D;      // this column's head row, in floats
  float4 x[PF];
  if (live) {
#pragma unroll
    for (int q = 0; q < PF; ++q)
      if (s_lo + q < s_hi) x[q] = ld_dev4_b(rr, (jrow + (s_lo + q) * D + d0) * 4);
  }
  // maxima and sums of every (head, split), as (max, sum) pairs of 8 bytes: issued in
  // one round with the partials above
  {
    // bounded to the group's rows: positions past them read 0
    const __amdgpu_buffer_rsrc_t rm = rsrc_n(src_ml + (size_t)hq0 * stride * 2, G * stride * 2 * 4);
    for (int i0 = 0; i0 < G * cnt; i0 += 4 * NT) {
      u32x2_t ml[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = i0 + u * NT + tid;
        const int jj = i / cnt, ss = i % cnt;
        ml[u] = __builtin_amdgcn_raw_buffer_load_b64(rm, ((jj * stride + s0 + ss) * 2) * 4, 0, kSc1);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = i0 + u * NT + tid;
        const int jj = i / cnt, ss = i % cnt;
        if (i < G * cnt && (act >> jj & 1u)) {
          sm.u.cmb.w[jj][ss] = __uint_as_float(ml[u].x);
          sm.u.cmb.lp[jj][ss] = __uint_as_float(ml[u].y);
        }
      }
    }
  }
  __syncthreads();
  for (int jj = wave; jj < G; jj += NW) {
    if (!(act >> jj & 1u)) continue;
    float M = -LD_INF;
    for (int ss = lane; ss < cnt; ss += 64) M = fmaxf(M, sm.u.cmb.w[jj][ss]);
    M = wave_max_f(M);
    const float mu = (M == -LD_INF) ? 0.f : M;
    float L = 0.f;
    for (int ss = lane; ss < cnt; ss += 64) {
      const float w = exp2_fast(sm.u.cmb.w[jj][ss] - mu);
      sm.u.cmb.w[jj][ss] = w;
      L += sm.u.cmb.lp[jj][ss] * w;
    }
    L = wave_sum_f(L);
    if (lane == 0) {
      sm.u.cmb.inv_l[jj] = p.v_scale / L;
      sm.u.cmb.mtot[jj] = M;
      sm.u.cmb.ltot[jj] = L;
    }
  }
  __syncthreads();
  float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
  if (live) {
    for (int sb = s_lo; sb < s_hi; sb += PF) {
#pragma unroll
      for (int q = 0; q < PF; ++q) {
        if (sb + q < s_hi) {
          const float w = sm.u.cmb.w[j][sb + q];
          o.x = fmaf(x[q].x, w, o.x); o.y = fmaf(x[q].y, w, o.y);
          o.z = fmaf(x[q].z, w, o.z); o.w = fmaf(x[q].w, w, o.w);
        }
      }
      if (sb + PF < s_hi) {
#pragma unroll
        for (int q = 0; q < PF; ++q)
          if (sb + PF + q < s_hi) x[q] = ld_dev4_b(rr, (jrow + (sb + PF + q) * D + d0) * 4);
      }
    }
  }
  if (TPCOL > 1 && live && part > 0) sm.u.cmb.part[part - 1][col] = o;
  __syncthreads();
  if (live && part == 0) {
#pragma unroll
    for (int q = 1; q < TPCOL; ++q) {
      const float4 y = sm.u.cmb.part[q - 1][col];
      o.x += y.x; o.y += y.y; o.z += y.z; o.w += y.w;
    }
    if (FINAL) {
      store_o<D>(p, hq0 + j, d0, o, sm.u.cmb.inv_l[j]);
    } else {
      const size_t us = (size_t)(hq0 + j) * p.P1 + upos;
      st_dev4_b(rsrc(dst_acc + (size_t)hq0 * p.P1 * D), ((j * p.P1 + upos) * D + d0) * 4, o);
      if (d0 == 0) {
        st_dev(dst_ml + us * 2 + 0, sm.u.cmb.mtot[j]);
        st_dev(dst_ml + us * 2 + 1, sm.u.cmb.ltot[j]);
      }
    }
  }
  __syncthreads();
}

// k of the row: the row's selection length, at most the sequence length nb.
__device__ __forceinline__ int select_k(const AttnParams& p, int slot, int nb) {
  int64_t so;
  int kk;
  s_row(p.s_indptr, p.k_dense, p.s_cap, slot, &so, &kk);
  return min(kk, nb);
}

// The value of v in this lane's partner of a combining step over aligned groups of 2 OFF
// lanes: DPP moves inside rows of 16 lanes, and the row-pair / half-wave swaps across
// rows. After the steps below OFF, every lane of an aligned group of OFF lanes holds a
// fold of all of that group's states, so any lane of the neighbouring group serves as
// the partner: the half-row mirror gives the step of 4.
template <int OFF>
__device__ __forceinline__ float partner(float v) {
  if constexpr (OFF == 1) return dpp_f<0xB1>(v);          // quad_perm [1,0,3,2]
  else if constexpr (OFF == 2) return dpp_f<0x4E>(v);     // quad_perm [2,3,0,1]
  else if constexpr (OFF == 4) return dpp_f<0x141>(v);    // row_half_mirror
  else if constexpr (OFF == 8) return xor8_f(v);
  else {
    const int lane = (int)(threadIdx.x & 63u);
    const auto w = OFF == 16 ? __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false)
                             : __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float((lane & OFF) ? w[0] : w[1]);
  }
}
// Folds the online-softmax state (max in log2 units, sum, unnormalised output) of the
// partner lane into this lane's.
template <int OFF>
__device__ __forceinline__ void fold_partner(float& m, float& l, float4& o) {
  const float m2 = partner<OFF>(m), l2 = partner<OFF>(l);
  const float ox = partner<OFF>(o.x), oy = partner<OFF>(o.y);
  const float oz = partner<OFF>(o.z), ow = partner<OFF>(o.w);
  const float mn = fmaxf(m, m2);
  const float mu = (mn == -LD_INF) ? 0.f : mn;
  const float w1 = exp2_fast(m - mu), w2 = exp2_fast(m2 - mu);
  l = l * w1 + l2 * w2;
  o.x = o.x * w1 + ox * w2; o.y = o.y * w1 + oy * w2;
  o.z = o.z * w1 + oz * w2; o.w = o.w * w1 + ow * w2;
  m = mn;
}

// Output columns [c_lo, c_hi) (float4 columns, head-major) of the group's active heads
// from its ns split partials (max in log2 units, sum, unnormalised output), by one
// workgroup without a barrier: TP adjacent lanes share each column, each folds every
// TP-th split into an online-softmax state (its loads issued a round at a time), and the
// lanes combine their states by shuffles; the first lane of the column writes O.
template <int D, int G, int NW>
__device__ __forceinline__ void merge_final(const AttnParams& p, uint32_t act, int hq0, int ns, int c_lo,
                                            int c_hi) {
  constexpr int NT = 64 * NW;
  constexpr int CH = 8;                         // splits per lane and round
  const int ncol = max(1, c_hi - c_lo);
  int TP = 1;                                   // lanes per column: a power of two, <= 64
  while (TP < 64 && TP * 2 * ncol <= NT) TP <<= 1;
  const int tid = threadIdx.x;
  const int c = c_lo + tid / TP, r = tid & (TP - 1);
  const int j = c / (D / 4), d0 = (c % (D / 4)) * 4;
  const bool live = c < c_hi && (act >> j & 1u);
  float m = -LD_INF, l = 0.f;
  float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
  if (live) {
    const __amdgpu_buffer_rsrc_t ra = rsrc_n(p.part_acc + (size_t)(hq0 + j) * p.P * D, ns * D * 4);
    const __amdgpu_buffer_rsrc_t rm = rsrc_n(p.part_ml + (size_t)(hq0 + j) * p.P * 2, ns * 2 * 4);
    for (int s0 = r; s0 < ns; s0 += TP * CH) {
      float4 a[CH];
      u32x2_t ml[CH];
#pragma unroll
      for (int u = 0; u < CH; ++u) {
        const int sp = s0 + u * TP;             // past ns: the bound reads 0 (masked below)
        a[u] = ld_dev4_b(ra, (sp * D + d0) * 4);
        ml[u] = __builtin_amdgcn_raw_buffer_load_b64(rm, sp * 8, 0, kSc1);
      }
#pragma unroll
      for (int u = 0; u < CH; ++u) {
        if (s0 + u * TP >= ns) break;
        const float ms = __uint_as_float(ml[u].x), ls = __uint_as_float(ml[u].y);
        const float mn = fmaxf(m, ms);
        const float mu = (mn == -LD_INF) ? 0.f : mn;
        const float wo = exp2_fast(m - mu), wn = exp2_fast(ms - mu);   // 0 for -inf maxima
        l = l * wo + ls * wn;
        o.x = o.x * wo + a[u].x * wn; o.y = o.y * wo + a[u].y * wn;
        o.z = o.z * wo + a[u].z * wn; o.w = o.w * wo + a[u].w * wn;
        m = mn;
      }
    }
  }
  // combine the TP lanes of the column (all lanes take part)
  if (TP > 1) fold_partner<1>(m, l, o);
  if (TP > 2) fold_partner<2>(m, l, o);
  if (TP > 4) fold_partner<4>(m, l, o);
  if (TP > 8) fold_partner<8>(m, l, o);
  if (TP > 16) fold_partner<16>(m, l, o);
  if (TP > 32) fold_partner<32>(m, l, o);
  if (live && r == 0) store_o<D>(p, hq0 + j, d0, o, p.v_scale / l);
}

// ---- selection of one retrieval row by one workgroup

// Exclusive prefix, in row order, of the per-(item, wave) counts buf[i * NW + w]
// (IT items of NT rows, item-major, at most NT entries): the prefixes replace the counts
// and the total is returned in every thread. The caller synchronises after writing
// the counts.
template <int NW, int IT>
__device__ __forceinline__ int scan_item_counts(int* buf, int* tmp) {
  constexpr int NE = IT * NW;
  static_assert(NE <= 64 * NW, "one entry per thread");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int v = tid < NE ? buf[tid] : 0;
  int wt;
  const int ex = wave_excl_scan(v, wt);
  if (lane == 0) tmp[wave] = wt;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int x = tmp[w];
    before += (w < wave) ? x : 0;
    all += x;
  }
  if (tid < NE) buf[tid] = before + ex;
  __syncthreads();
  return all;
}

// Sums over the workgroup of four counts, in every thread (tmp: LDS int[NW][4]).
template <int NW>
__device__ __forceinline__ int4 wg_sum4(int4 v, int (*tmp)[4]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int a = wave_total(v.x), b = wave_total(v.y), c = wave_total(v.z), d = wave_total(v.w);
  if (lane == 0) { tmp[wave][0] = a; tmp[wave][1] = b; tmp[wave][2] = c; tmp[wave][3] = d; }
  __syncthreads();
  int4 s = make_int4(0, 0, 0, 0);
#pragma unroll
  for (int i = 0; i < NW; ++i) { s.x += tmp[i][0]; s.y += tmp[i][1]; s.z += tmp[i][2]; s.w += tmp[i][3]; }
  __syncthreads();
  return s;
}

// argsTopK of row `slot` (method step 3), part `part` of `parts`: the parts are
// workgroups that each hold a contiguous share of the row's keys (order-preserving images
// of the fp32 logits, which every split of the KV group has stored device-coherently, with
// its digit-1 counts, before the parts start). Each part takes digit 1 (bits 31..21 of
// the threshold key T) from the summed histogram replicas, counts its keys above that
// bin and stores its keys in the bin (the candidates, key bits 20..0, in row order) in a
// sub-list of its own; after the parts meet (every part is already running, so the wait
// ends), each gathers every part's candidates, derives digits 2 and 3 of T from them, its
// output offset from the earlier parts' counts and candidates, and writes its kept rows
// (keys above T, and of the keys equal to T the first ones in row order) in ascending
// order with their membership words. The row's arrival counter starts at zero (the KV
// group's last split clears it before the parts are released). LDS: hist
// [kHist2Bins + kHist3Bins], cand [kCandLds], wcnt [NW], res [2], tmp4 [NW][4],
// poff [kMaxParts + 1], pcnt [kMaxParts].
template <int NW>
__device__ __forceinline__ void part_select(uint32_t* hist, uint32_t* cand_lds, int* wcnt, uint32_t* res,
                                            int (*tmp4)[4], int* poff, int* pcnt, const AttnParams& p, int slot,
                                            int nb, int part, int parts) {
  constexpr int NT = 64 * NW;
  constexpr int IT = 16;                        // keys per thread per pass
  constexpr int PASS = IT * NT;                 // rows per pass
  constexpr int PB1 = kHist1Bins / NT;
  constexpr int SPEC = 8;                       // candidates fetched per thread with the counts
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));   // lanes under this one
  const int kk = select_k(p, slot, nb);
  // this part's rows: [r0, r0 + ns), a whole number of NT-row items; its candidate
  // sub-list starts at r0 of the row's list (it holds at most ns entries)
  const int R = ((nb + parts - 1) / parts + NT - 1) / NT * NT;
  const int r0 = min(nb, part * R);
  const int ns = max(0, min(nb, r0 + R) - r0);
  const int npass = (ns + PASS - 1) / PASS;
  const float* lg = p.logits + (size_t)slot * p.seq_len + r0;
  uint32_t* gcnt = p.sel_cnt + (size_t)slot * 2;          // [0]: parts arrived
  uint32_t* gcand = p.sel_cand + (size_t)slot * p.seq_len;
  uint64_t* gpub = p.sel_pub + (size_t)slot * kMaxParts;  // per part: above | candidates << 32

  uint32_t key[IT];
  // device-coherent (sc1) buffer loads, all issued before the first use; rows past the
  // part read 0 from the buffer's bound and are masked by index
  auto load = [&](int ps) {
    const int lim = min(ns - ps * PASS, PASS);
    const __amdgpu_buffer_rsrc_t r = rsrc_n(lg + (size_t)ps * PASS, max(lim, 0) * 4);
    uint32_t raw[IT];
#pragma unroll
    for (int i = 0; i < IT; ++i) raw[i] = __builtin_amdgcn_raw_buffer_load_b32(r, (i * NT + tid) * 4, 0, kSc1);
#pragma unroll
    for (int i = 0; i < IT; ++i) key[i] = score_key(__uint_as_float(raw[i]));
  };
  if (kk >= 1 && npass) load(0);               // in flight with the histogram sum
  // ---- digit 1 from the row's counts (the sum of the replicas)
  hist1_sum<NT>(hist, p.hist1, slot);
  if (tid == 0) { res[0] = 0; res[1] = 0; }
  __syncthreads();
  if (parts == 1) hist1_clear(p.hist1, slot);   // the only reader
  if (kk < 1) {                                 // nothing to keep; no part uses the counts
    if (parts > 1 && part == 0) hist1_clear(p.hist1, slot);
    return;
  }
  uint32_t b1, k1;
  {
    uint32_t h1[PB1];
#pragma unroll
    for (int q = 0; q < PB1; ++q) h1[q] = hist[tid * PB1 + q];
    find_bin_regs<kHist1Bins, NT>(h1, (uint32_t)kk, wcnt, res);
    b1 = res[0];
    k1 = (uint32_t)kk - res[1];
    __syncthreads();
  }
  // ---- this part's keys above bin b1 (a count) and in it (its sub-list, in row order)
  int above = 0, ncand = 0;
  for (int ps = 0; ps < npass; ++ps) {
    if (ps) load(ps);
    const int lim = min(ns - ps * PASS, PASS);
    uint32_t cm = 0;
#pragma unroll
    for (int i = 0; i < IT; ++i) {
      const bool v = i * NT + tid < lim;
      const uint32_t d1 = key[i] >> 21;
      above += (v & (d1 > b1)) ? 1 : 0;
      cm |= (uint32_t)(v & (d1 == b1)) << i;
    }
    // positions in row order: per-(item, wave) counts, scanned
    int* cnt = reinterpret_cast<int*>(hist);
#pragma unroll
    for (int i = 0; i < IT; ++i) {
      const uint64_t cb = __ballot((cm >> i) & 1u);
      if (lane == 0) cnt[i * NW + wave] = __popcll(cb);
    }
    __syncthreads();
    const int ctot = scan_item_counts<NW, IT>(cnt, wcnt);
#pragma unroll
    for (int i = 0; i < IT; ++i) {
      const bool c = (cm >> i) & 1u;
      const uint64_t cb = __ballot(c);
      if (c) st_dev(gcand + r0 + ncand + cnt[i * NW + wave] + __popcll(cb & below), key[i] & 0x1fffffu);
    }
    ncand += ctot;
    __syncthreads();
  }
  {
    const int4 t = wg_sum4<NW>(make_int4(above, 0, 0, 0), tmp4);
    above = t.x;
  }
  if (parts > 1 && tid == 0) st_dev(gpub + part, (uint64_t)(uint32_t)above | ((uint64_t)(uint32_t)ncand << 32));
  // the digit-2 and digit-3 histograms start from zero (the append counts are done with
  // the LDS); the gather below counts digit 2 as the candidates arrive
  for (int i = tid; i < kHist2Bins + kHist3Bins; i += NT) hist[i] = 0u;
  uint32_t* h2 = hist;
  uint32_t* h3 = hist + kHist2Bins;
  __builtin_amdgcn_s_waitcnt(0);                // this part's candidates and counts are stored
  __syncthreads();
  // ---- the parts meet
  if (parts > 1) {
    if (tid == 0) {
      __hip_atomic_fetch_add(gcnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      int spins = 0;
      while (__hip_atomic_fetch_add(gcnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < (uint32_t)parts) {
        __builtin_amdgcn_s_sleep(1);
        if (++spins > kMaxSpins) { st_dev(p.err, 1u); break; }
      }
    }
    __syncthreads();
    if (part == 0) hist1_clear(p.hist1, slot);  // every part has read the replicas
  }
  // ---- every part's candidates, gathered in part order (in LDS when they fit). Each
  // part's sub-list is read by its own TPP threads (entry i by thread i mod TPP); the
  // first SPEC entries per thread are fetched with the counts, before those are known
  // (reads past a sub-list's count are ignored; the row's list bounds them).
  const __amdgpu_buffer_rsrc_t rl = rsrc_n(gcand, p.seq_len * 4);
  const int tpp = NT / parts;                   // threads per part (parts <= NT / 8)
  const int gq = tid / tpp, gi = tid - gq * tpp;
  const bool gin = gq < parts;
  uint32_t sv[SPEC];
  uint64_t pubv = 0;
  if (parts > 1) {
    if (tid < parts) pubv = ld_dev(gpub + tid);
#pragma unroll
    for (int u = 0; u < SPEC; ++u) {
      const int at = gin ? gq * R + gi + u * tpp : p.seq_len;
      sv[u] = __builtin_amdgcn_raw_buffer_load_b32(rl, at * 4, 0, kSc1);
    }
  }
  if (parts > 1) {
    if (tid < parts) { pcnt[tid] = (int)(uint32_t)pubv; poff[tid + 1] = (int)(uint32_t)(pubv >> 32); }
  } else if (tid == 0) {
    pcnt[0] = 0;
    poff[1] = ncand;
  }
  __syncthreads();
  if (tid == 0) {                               // sub-list counts -> offsets in part order
    int o = 0;
    for (int q = 0; q < parts; ++q) { const int c = poff[q + 1]; poff[q] = o; o += c; }
    poff[parts] = o;
  }
  __syncthreads();
  const int total = poff[parts];
  const bool in_lds = total <= kCandLds;
  if (in_lds && gin) {
    const int n_q = poff[gq + 1] - poff[gq];
    uint32_t* dstq = cand_lds + poff[gq];
    const int first = parts > 1 ? SPEC * tpp : 0;   // entries fetched above
    if (parts > 1) {
#pragma unroll
      for (int u = 0; u < SPEC; ++u)
        if (gi + u * tpp < n_q) {
          dstq[gi + u * tpp] = sv[u];
          atomicAdd(&h2[(sv[u] >> 10) & 0x7ffu], 1u);
        }
    }
    for (int i0 = first; i0 < n_q; i0 += SPEC * tpp) {
#pragma unroll
      for (int u = 0; u < SPEC; ++u) {
        const int i = i0 + gi + u * tpp;
        sv[u] = __builtin_amdgcn_raw_buffer_load_b32(rl, (i < n_q ? gq * R + i : p.seq_len) * 4, 0, kSc1);
      }
#pragma unroll
      for (int u = 0; u < SPEC; ++u)
        if (i0 + gi + u * tpp < n_q) {
          dstq[i0 + gi + u * tpp] = sv[u];
          atomicAdd(&h2[(sv[u] >> 10) & 0x7ffu], 1u);
        }
    }
  }
  // earlier parts' keys above bin b1
  int above_before = 0;
  for (int q = 0; q < part; ++q) above_before += pcnt[q];
  __syncthreads();
  // candidate i of the gathered list (parts in order)
  auto cand_at = [&](int i) -> uint32_t {
    if (in_lds) return cand_lds[i];
    int q = 0;
    while (q + 1 < parts && poff[q + 1] <= i) ++q;
    return ld_dev(gcand + (size_t)q * R + (i - poff[q]));
  };
  // candidates [0, n) of the gathered list in batches: each thread reads CB of them
  // before it uses any (entries past n read as ~0, which no 21-bit candidate equals)
  constexpr int CB = 8;
  auto for_cands = [&](int n, auto&& f) {
    for (int i0 = tid; i0 < n; i0 += CB * NT) {
      uint32_t c[CB];
#pragma unroll
      for (int u = 0; u < CB; ++u) c[u] = i0 + u * NT < n ? cand_at(i0 + u * NT) : ~0u;
#pragma unroll
      for (int u = 0; u < CB; ++u)
        if (c[u] != ~0u) f(c[u]);
    }
  };
  if (!in_lds) {                                // (in LDS, the gather counted digit 2)
    for_cands(total, [&](uint32_t c) { atomicAdd(&h2[(c >> 10) & 0x7ffu], 1u); });
    __syncthreads();
  }
  find_bin_from_top<kHist2Bins, NT>([&](int i) { return h2[i]; }, k1, wcnt, res);
  const uint32_t b2 = res[0], k2 = k1 - res[1];
  __syncthreads();
  if (tid == 0) { res[0] = 0; res[1] = 0; }
  for_cands(total, [&](uint32_t c) {
    if (((c >> 10) & 0x7ffu) == b2) atomicAdd(&h3[c & 0x3ffu], 1u);
  });
  __syncthreads();
  find_bin_from_top<kHist3Bins, NT>([&](int i) { return h3[i]; }, k2, wcnt, res);
  const uint32_t t21 = (b2 << 10) | res[0];     // T's bits 20..0
  const uint32_t T = (b1 << 21) | t21;
  const int et = (int)(k2 - res[1]);            // keys equal to T that are kept
  // ---- earlier parts' candidates above / equal to T; this part's keys equal to T
  int gt = 0, eqb = 0;
  for_cands(poff[part], [&](uint32_t c) {
    gt += c > t21 ? 1 : 0;
    eqb += c == t21 ? 1 : 0;
  });
  int eqm = 0;
  {
    int ps = 0;
    do {
      if (npass > 1) load(ps);
      const int lim = min(ns - ps * PASS, PASS);
#pragma unroll
      for (int i = 0; i < IT; ++i) eqm += ((i * NT + tid < lim) & (key[i] == T)) ? 1 : 0;
    } while (++ps < npass);
  }
  {
    // above_before is already whole in every thread (from LDS)
    const int4 t = wg_sum4<NW>(make_int4(0, gt, eqb, eqm), tmp4);
    gt = t.y; eqb = t.z; eqm = t.w;
  }
  const int keep_eq = max(0, min(et - eqb, eqm));   // this part's kept keys equal to T
  const int off = above_before + gt + min(et, eqb);
  // ---- kept rows, ascending, with their membership words
  int64_t so;
  int klen;
  s_row(p.s_indptr, p.k_dense, p.s_cap, slot, &so, &klen);
  klen = min(klen, nb);
  int32_t* out = p.s_out + so;
  uint32_t* bm = p.bitmaps ? p.bitmaps + (size_t)slot * p.W : nullptr;
  int* cnt = reinterpret_cast<int*>(hist);      // [IT][NW] counts, then prefixes
  int* tcnt = cnt + IT * NW;                    // [IT][NW] tie counts, then prefixes
  const bool eq_all = keep_eq == 0 || keep_eq == eqm;   // all of this part's ties are kept, or none
  int kept_before = off, ties_before = 0;
  for (int ps = 0; ps < npass; ++ps) {
    if (npass > 1) load(ps);
    const int lim = min(ns - ps * PASS, PASS);
    uint32_t kpm = 0;                           // bit i: item i of this lane is kept
    if (eq_all) {
#pragma unroll
      for (int i = 0; i < IT; ++i) {
        const bool v = i * NT + tid < lim;
        kpm |= (uint32_t)(v & ((key[i] > T) | ((key[i] == T) & (keep_eq > 0)))) << i;
      }
    } else {
      // the first keep_eq ties of this part in row order: ranks from per-item counts
      uint32_t eqm_l = 0;
#pragma unroll
      for (int i = 0; i < IT; ++i) {
        const bool e = (i * NT + tid < lim) & (key[i] == T);
        eqm_l |= (uint32_t)e << i;
        const uint64_t eb = __ballot(e);
        if (lane == 0) tcnt[i * NW + wave] = __popcll(eb);
      }
      __syncthreads();
      const int ttot = scan_item_counts<NW, IT>(tcnt, wcnt);
#pragma unroll
      for (int i = 0; i < IT; ++i) {
        const bool e = (eqm_l >> i) & 1u;
        const uint64_t eb = __ballot(e);
        const int rank = ties_before + tcnt[i * NW + wave] + __popcll(eb & below);
        const bool g = (i * NT + tid < lim) & (key[i] > T);
        kpm |= (uint32_t)(g | (e & (rank < keep_eq))) << i;
      }
      ties_before += ttot;
    }
#pragma unroll
    for (int i = 0; i < IT; ++i) {
      const uint64_t kb = __ballot((kpm >> i) & 1u);
      if (lane == 0) cnt[i * NW + wave] = __popcll(kb);
    }
    __syncthreads();
    const int ktot = scan_item_counts<NW, IT>(cnt, wcnt);
#pragma unroll
    for (int i = 0; i < IT; ++i) {
      const bool kp = (kpm >> i) & 1u;
      const uint64_t kb = __ballot(kp);
      const int row = r0 + ps * PASS + i * NT + tid;
      const int pos = kept_before + cnt[i * NW + wave] + __popcll(kb & below);
      if (kp & (pos < klen)) out[pos] = row;
      const int w0 = r0 + ps * PASS + i * NT + wave * 64;   // a multiple of 64
      if (bm && (lane & 31) == 0 && w0 + lane < r0 + ns && ((w0 + lane) >> 5) < p.W)
        bm[(w0 + lane) >> 5] = (uint32_t)(kb >> lane);
    }
    kept_before += ktot;
    __syncthreads();                            // the count buffers are reused
  }
}

// F8: K and V hold E4M3 codes (one byte per element, dequantised exactly to bf16 /
// fp32 in registers; their per-tensor scales are folded into p.scale and p.v_scale).
// BLK: token-block selection (the sets are whole 64-row blocks): stream mode also keeps
// the retrieval rows' block maxima, gather mode spreads the blocks over the waves; a
// separate instance, so that the token path carries none of it.
template <int D, int G, int NW, bool F8, bool BLK = false, bool PG = false>
__global__ __launch_bounds__(64 * NW, 8 / NW) void k_attention(const AttnParams p) {
  constexpr int NT = 64 * NW;
  constexpr int KCH = D / 32;        // MFMA k-steps per row
  constexpr int EPL = D / 8;         // dims per lane in the P.V layout
  constexpr int NV = D / 64;         // 16-byte V loads per lane per row
  // tiles per chunk per wave: two with E4M3 codes, so that a wave keeps as many bytes
  // in flight as with bf16
  constexpr int TPC = F8 ? 2 : 1;
  constexpr int CROWS = kTile * TPC;
  constexpr int RSC = 2 * TPC;      // P.V row steps (8 rows) per chunk
  using Smem = AttnSmem<D, G, NW>;
  constexpr int RP = Smem::RP;
  __shared__ Smem sm;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int mr = lane & 15, mk = lane >> 4;   // MFMA roles: row/column, k-group
  const int rg = lane >> 3, li = lane & 7;    // P.V roles: row in step, dim slice
  const bool do_hist = p.do_topk != 0;
  const bool do_blk = BLK && p.blk_out != nullptr;   // block maxima of the retrieval rows' logits

  {
    // touch every 64-byte line of the kernel arguments in one round, so that the argument
    // reads of the prologue hit the scalar cache instead of missing one line after another
    typedef const volatile uint32_t __attribute__((address_space(4))) karg_u32;
    karg_u32* ka = (karg_u32*)__builtin_amdgcn_kernarg_segment_ptr();
    uint32_t t = 0;
#pragma unroll
    for (int i = 0; i < (int)sizeof(AttnParams); i += 64) t ^= ka[i / 4];
    asm volatile("" ::"s"(t));
  }
  int bid = blockIdx.x;
  const int dense_blocks = p.B * p.ng_dense * p.nsplit_d;
  int split, gi, b, ts;
  if (bid < dense_blocks) {
    split = bid % p.nsplit_d;
    bid /= p.nsplit_d;
    gi = bid % p.ng_dense;
    b = bid / p.ng_dense;
    ts = p.ts_d;
  } else {
    const int ngs = p.ngroups - p.ng_dense;
    bid -= dense_blocks;
    split = bid % p.nsplit_s;
    bid /= p.nsplit_s;
    gi = p.ng_dense + bid % ngs;
    b = bid / ngs;
    ts = p.ts_s;
  }
  // the gi-th launched group: the streaming ones first, then the gathering ones, each in
  // ascending order (bit arithmetic on kernel arguments, no memory access)
  int g;
  {
    uint64_t m = gi < p.ng_dense ? p.dense_groups : p.sparse_groups;
    for (int i = gi < p.ng_dense ? gi : gi - p.ng_dense; i > 0; --i) m &= m - 1ull;
    g = (int)__builtin_ctzll(m);
  }

  // paged KV: an instance of its own for token sets, so that the unpaged one carries no
  // page arithmetic (the block instance decides at run time)
  const bool paged = BLK ? p.page_shift != 0 : PG;
  int64_t tok0;
  int nb;
  if (p.kv_indptr) {
    tok0 = p.kv_indptr[b];
    nb = (int)(p.kv_indptr[b + 1] - tok0);
  } else {
    tok0 = (int64_t)b * p.seq_len;
    nb = p.seq_len;
  }
  // never read past the cache or the per-row scratch, whatever kv_indptr holds (paged
  // rows are clamped to the pool through their page ids)
  nb = min(nb, p.seq_len);
  if (paged) {
    tok0 = 0;
  } else if (tok0 < 0 || tok0 >= p.total_tokens) {
    nb = 0;
  } else if ((int64_t)nb > p.total_tokens - tok0) {
    nb = (int)(p.total_tokens - tok0);
  }
  const int nsplit_b = (nb + ts - 1) / ts;
  if (nb <= 0 || split >= nsplit_b) return;
  int r0 = split * ts;
  int nrows = min(ts, nb - r0);

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
  const int hq0 = b * p.Hq + g * G;           // first query-head slot of the group

  // ---- query operand (B): column mr = head, k-group mk; zero for padding columns
  uint4 qb[KCH];
#pragma unroll
  for (int kk = 0; kk < KCH; ++kk) {
    if (mr < G)
      qb[kk] = *reinterpret_cast<const uint4*>(p.q + (size_t)(hq0 + mr) * D + kk * 32 + mk * 8);
    else
      qb[kk] = make_uint4(0, 0, 0, 0);
  }

  // ---- block sets (the caller's hint; unpaged KV, at most 512 blocks per wave): a
  // gathering split takes an equal share of its group's union of selected 64-row blocks
  // instead of a range of rows, so that the group's splits visit about the same number
  // of rows however the blocks fall (a few blocks per split leave contiguous ranges very
  // unequal). Thread t reads the membership words of blocks 8t .. 8t + 7 of the group's
  // sparse heads, the workgroup ranks the union's blocks, and the split keeps ranks
  // [U * split / nsplit_b, U * (split + 1) / nsplit_b) in sm.blk; local row r of the
  // split is then row 64 * blk[r / 64] + r % 64 of the sequence. Every row of a kept block
  // is visited, each head masked by its own membership.
  bool bsh = false;
  if constexpr (BLK) {
    bsh = !dense && !paged && p.gather_blocks != 0 && nb <= 8 * 64 * NT;
    if (bsh) {
      const int nblk = (nb + 63) >> 6;
      uint32_t wd[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) wd[i] = 0u;
#pragma unroll
      for (int j = 0; j < G; ++j) {
        if (!(spm >> j & 1)) continue;
        const __amdgpu_buffer_rsrc_t rb = rsrc_n(p.bitmaps + (size_t)(hq0 + j) * p.W, p.W * 4);
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const u32x4_t x = __builtin_amdgcn_raw_buffer_load_b128(rb, (16 * tid + 4 * q4) * 4, 0, 0);
          wd[4 * q4 + 0] |= x.x; wd[4 * q4 + 1] |= x.y; wd[4 * q4 + 2] |= x.z; wd[4 * q4 + 3] |= x.w;
        }
      }
      uint32_t u = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) u |= (uint32_t)(8 * tid + i < nblk && (wd[2 * i] | wd[2 * i + 1]) != 0u) << i;
      int wt;
      const int pre = wave_excl_scan(__popc(u), wt);
      if (lane == 0) sm.wcnt[wave] = wt;
      __syncthreads();
      int below = 0, U = 0;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const int c = sm.wcnt[w];
        below += w < wave ? c : 0;
        U += c;
      }
      const int lo = (int)((int64_t)U * split / nsplit_b), hi = (int)((int64_t)U * (split + 1) / nsplit_b);
      int rank = below + pre;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (u >> i & 1u) {
          if (rank >= lo && rank < hi) sm.blk[rank - lo] = (uint16_t)(8 * tid + i);
          ++rank;
        }
      }
      r0 = 0;
      nrows = (hi - lo) * 64;                 // at most ts: a share holds at most ts / 64 blocks
      __syncthreads();
    }
  }
  // row of the sequence, from r0, of local row r of the split
  auto lrow = [&](int r) -> int {
    if constexpr (BLK) {
      if (bsh) return ((int)sm.blk[(r >> 6) & (kMaxSplitRows / 64 - 1)] << 6) + (r & 63);
    }
    return r;
  };

  // ---- per-wave streaming state (tiles wave, wave+4, ...; TPC tiles per chunk)
  constexpr int EB = F8 ? 1 : 2;              // bytes per K/V element
  const char* kbase = static_cast<const char*>(p.kc) + ((size_t)g * p.kv_head_stride + (size_t)(tok0 + r0) * D) * EB;
  const char* vbase = static_cast<const char*>(p.vc) + ((size_t)g * p.kv_head_stride + (size_t)(tok0 + r0) * D) * EB;
  // Paged KV: the page ids of the split's rows go to LDS once; row r of the split (a
  // row of the sequence: r0 + r) is then pool row page << shift | offset.
  const int pshift = p.page_shift, pmask = (1 << pshift) - 1;
  const int pg0 = r0 >> pshift;
  if (paged) {
    const int npg = ((r0 + nrows - 1) >> pshift) - pg0 + 1;
    const int32_t* bt = p.block_table + (size_t)b * p.pages_per_seq + pg0;
    for (int i = tid; i < npg; i += NT) {
      const int64_t id = bt[i];
      sm.pages[i] = (int)(id < 0 ? 0 : (id >= p.npages ? p.npages - 1 : id));
    }
    __syncthreads();
  }
  // element offset of row r of the split from kbase / vbase (paged: from the head's pool)
  auto row_off = [&](int r) -> ptrdiff_t {
    if (!paged) return (ptrdiff_t)lrow(r) * D;
    const int i = r0 + r;
    return (((ptrdiff_t)sm.pages[(i >> pshift) - pg0] << pshift) + (i & pmask) - r0) * D;
  };
  // Stream mode: the waves take interleaved 16-row tiles of the split. Gather mode:
  // each wave owns a contiguous block of the split's rows [lbase, rend) and visits
  // positions lbase .. lbase + nl_w: first the block's first `head` rows as they are
  // (one chunk, loaded before the membership words arrive, non-members masked), then
  // the members of the rest of its block (its own visit list), so the list needs no
  // workgroup-wide step and memory is busy from the start.
  // With p.gather_blocks (sets made of whole 64-row blocks, clustered rather than spread),
  // a wave owns the interleaved 64-row steps wave, wave + NW, .. of the split instead, so
  // that the selected blocks spread over the waves; visit positions stay per wave.
  int nlist = nrows;
  int nl_w = 0;
  const int gR = ((ts + 64 * NW - 1) / (64 * NW)) * 64;   // gather: rows per wave
  const bool ilv = BLK && !dense;
  const int lbase = dense ? 0 : wave * gR;                // the wave's visit positions start here
  auto step_row = [&](int c) { return ilv ? (c * NW + wave) * 64 : lbase + c * 64; };   // first row of step c
  const int rend = dense ? nrows : min(nrows, lbase + gR);
  const int head = dense ? 0 : (ilv ? min(CROWS, max(0, nrows - wave * 64)) : min(CROWS, max(0, rend - lbase)));
  auto chunks_of = [&](int n) {
    const int ntiles = (n + kTile - 1) / kTile;
    const int my_tiles = ntiles > wave ? (ntiles - wave + NW - 1) / NW : 0;
    return (my_tiles + TPC - 1) / TPC;
  };
  auto tbase = [&](int c, int t) -> int {
    return dense ? (wave + NW * (c * TPC + t)) * kTile : lbase + (c * TPC + t) * kTile;
  };
  int lim = dense ? nrows : lbase + head;      // visit positions below lim are valid

  const bool head_lane = mr < G;
  const bool ret_lane = head_lane && ((ret >> mr) & 1u);
  // logits of the retrieval rows (stream mode: a visit position is the row), four rows per
  // lane and tile in one 16-byte store through a resource over the group's rows:
  // device-coherent (sc1) when selectors of this launch read them back, write-back when
  // the selection runs in launches of its own (the launch boundary publishes them)
  const bool lg_on = p.logits != nullptr && ret_lane;
  const __amdgpu_buffer_rsrc_t lrs = rsrc(p.logits ? p.logits + (size_t)hq0 * p.seq_len : nullptr);
  const bool lg_vec = (p.seq_len & 3) == 0 && ((uintptr_t)p.logits & 15u) == 0;
  const uint32_t lg_off = (uint32_t)(((size_t)mr * p.seq_len + r0) * 4);
  const bool lg_coh = p.fin != 0;
  const float scale = p.scale;

  float m_lane = -LD_INF, l_lane = 0.f;     // running max / sum of head mr (lanes mr < G)
  float acc[G][EPL];
#pragma unroll
  for (int j = 0; j < G; ++j)
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[j][e] = 0.f;

  uint4 kr[3][TPC][KCH], vr[3][RSC][NV];

  auto row_of = [&](int pos) -> int {
    if constexpr (BLK) {
      if (dense) return pos;
      if (pos < lbase + head) return ilv ? wave * 64 + (pos - lbase) : pos;   // the head rows
      return (int)sm.list[pos];
    } else {
      return (dense || pos < lbase + head) ? pos : (int)sm.list[pos];
    }
  };
  auto load_chunk = [&](int c, uint4 (&kd)[TPC][KCH], uint4 (&vd)[RSC][NV]) {
#pragma unroll
    for (int t = 0; t < TPC; ++t) {
      const int tb = tbase(c, t);
      const int pa = tb + mr;                 // A-operand row of this lane
      const bool va = pa < lim;
      const char* kp = kbase + (row_off(va ? row_of(pa) : 0) + mk * 8) * EB;
#pragma unroll
      for (int kk = 0; kk < KCH; ++kk) {
        if constexpr (F8) {
          const uint2 c = va ? *reinterpret_cast<const uint2*>(kp + kk * 32) : make_uint2(0, 0);
          kd[t][kk] = make_uint4(c.x, c.y, 0, 0);
        } else {
          kd[t][kk] = va ? ld_stream16(kp + kk * 64) : make_uint4(0, 0, 0, 0);
        }
      }
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const int pv = tb + h2 * 8 + rg;      // P.V row of this lane
        const bool vv = pv < lim;
        const char* vp = vbase + (row_off(vv ? row_of(pv) : 0) + li * 8) * EB;
#pragma unroll
        for (int c2 = 0; c2 < NV; ++c2) {
          if constexpr (F8) {
            const uint2 c = vv ? *reinterpret_cast<const uint2*>(vp + c2 * 64) : make_uint2(0, 0);
            vd[t * 2 + h2][c2] = make_uint4(c.x, c.y, 0, 0);
          } else {
            vd[t * 2 + h2][c2] = vv ? ld_stream16(vp + c2 * 128) : make_uint4(0, 0, 0, 0);
          }
        }
      }
    }
  };

  // The first chunks (unpaged KV) go through buffer resources over the split's rows: a
  // position past the valid ones reads zero from past the end of the resource, so the
  // loads need no per-lane branch. (Around a branch the compiler merged a loaded register
  // into the register holding the zero, and that copy waited for the load before the
  // prologue could go on.)
  const int sbytes = paged ? 0 : (bsh ? nb : nrows) * D * EB;
  const __amdgpu_buffer_rsrc_t krs = rsrc_n(kbase, sbytes), vrs = rsrc_n(vbase, sbytes);
  constexpr uint32_t kPast = 0x80000000u;     // past the end of every such resource
  auto load_chunk_b = [&](int c, uint4 (&kd)[TPC][KCH], uint4 (&vd)[RSC][NV]) {
#pragma unroll
    for (int t = 0; t < TPC; ++t) {
      const int tb = tbase(c, t);
      const int pa = tb + mr;
      const uint32_t ko = pa < lim ? (uint32_t)((lrow(row_of(pa)) * D + mk * 8) * EB) : kPast;
#pragma unroll
      for (int kk = 0; kk < KCH; ++kk) {
        if constexpr (F8) {
          const u32x2_t x = __builtin_amdgcn_raw_buffer_load_b64(krs, ko + kk * 32, 0, 0);
          kd[t][kk] = make_uint4(x.x, x.y, 0, 0);
        } else {
          const u32x4_t x = __builtin_amdgcn_raw_buffer_load_b128(krs, ko + kk * 64, 0, kNt);
          kd[t][kk] = make_uint4(x.x, x.y, x.z, x.w);
        }
      }
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const int pv = tb + h2 * 8 + rg;
        const uint32_t vo = pv < lim ? (uint32_t)((lrow(row_of(pv)) * D + li * 8) * EB) : kPast;
#pragma unroll
        for (int c2 = 0; c2 < NV; ++c2) {
          if constexpr (F8) {
            const u32x2_t x = __builtin_amdgcn_raw_buffer_load_b64(vrs, vo + c2 * 64, 0, 0);
            vd[t * 2 + h2][c2] = make_uint4(x.x, x.y, 0, 0);
          } else {
            const u32x4_t x = __builtin_amdgcn_raw_buffer_load_b128(vrs, vo + c2 * 128, 0, kNt);
            vd[t * 2 + h2][c2] = make_uint4(x.x, x.y, x.z, x.w);
          }
        }
      }
    }
  };

  // gather mode: the membership words of the wave's block, issued first so that their
  // wait does not include the head rows' loads
  constexpr int GCH = kMaxSplitRows / (64 * NW);   // 64-row steps of a wave's block
  static_assert(2 * GCH <= 64, "one word per lane");
  uint32_t gbw[G];
  if (!dense) {
    int word;
    bool ok;
    if constexpr (BLK) {
      const int srow = step_row(lane >> 1) + 32 * (lane & 1);   // lanes 2c, 2c+1: the words of step c
      const bool in = lane < 2 * GCH && srow < (ilv ? nrows : rend);
      word = in ? (r0 + lrow(srow)) >> 5 : 0;
      ok = in && word < p.W;
    } else {
      word = ((r0 + lbase) >> 5) + lane;
      ok = lane < 2 * GCH && lbase + 32 * lane < rend && word < p.W;
    }
#pragma unroll
    for (int j = 0; j < G; ++j)
      gbw[j] = ((spm >> j & 1) && ok) ? p.bitmaps[(size_t)(hq0 + j) * p.W + word] : 0u;
  }
  if (!paged) {
    // no branch: a chunk past the wave's rows reads zeros
    load_chunk_b(0, kr[0], vr[0]);            // gather mode: the head rows, no list needed
    if (dense) load_chunk_b(1, kr[1], vr[1]);
  } else if (dense) {
    const int nc0 = chunks_of(nrows);
    if (nc0 > 0) load_chunk(0, kr[0], vr[0]);
    if (nc0 > 1) load_chunk(1, kr[1], vr[1]);
  } else if (head > 0) {
    load_chunk(0, kr[0], vr[0]);
  }

  // ---- membership of each row of the tile, and the visit list
  if ((do_hist || do_blk) && ret) {           // histogram bins, or block-maximum keys
    for (int j = 0; j < G; ++j)
      if (ret >> j & 1u)
        for (int i = tid; i < kHist1Bins / 4; i += NT) reinterpret_cast<uint4*>(sm.u.hist[j])[i] = make_uint4(0, 0, 0, 0);
  }
  // Membership words: every lane loads one bitmap word per sparse head (the words
  // that cover the wave's rows), and each 64-row step takes its two words from lanes
  // 2c and 2c+1 (r0 and the wave's first row are multiples of 32, so row bit = lane).
  auto row_bits = [&](const uint32_t (&bw)[G], int c) -> uint32_t {
    uint32_t m = 0;
#pragma unroll
    for (int j = 0; j < G; ++j) {
      if (spm >> j & 1) {
        const uint32_t lo = __builtin_amdgcn_readlane(bw[j], 2 * c);
        const uint32_t hi = __builtin_amdgcn_readlane(bw[j], 2 * c + 1);
        m |= (((lane < 32 ? lo : hi) >> (lane & 31)) & 1u) << j;
      }
    }
    return m;
  };
  if (spm && dense) {
    // thread rows it * NT + tid: the wave's rows of step it are words
    // (r0 + it * NT + wave * 64) / 32 + {0, 1}
    constexpr int IT = kMaxSplitRows / NT;
    static_assert(2 * IT <= 64, "one word per lane");
    uint32_t bw[G];
    {
      const int it = lane >> 1;
      const int word = ((r0 + it * NT + wave * 64) >> 5) + (lane & 1);
      const bool ok = lane < 2 * IT && it * NT + wave * 64 < nrows && word < p.W;
#pragma unroll
      for (int j = 0; j < G; ++j)
        bw[j] = ((spm >> j & 1) && ok) ? p.bitmaps[(size_t)(hq0 + j) * p.W + word] : 0u;
    }
    uint32_t mrow[IT];
#pragma unroll
    for (int it = 0; it < IT; ++it) mrow[it] = ret | row_bits(bw, it);
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int r = it * NT + tid;
      if (r < nrows) sm.hmp[r] = (uint8_t)mrow[it];
    }
  }
  if (spm && !dense) {
    // rows owned by this wave: its 64-row steps (step_row), one per ballot; the head rows
    // keep their positions (their membership masks the softmax), the rest are listed
    constexpr int CH = GCH;
    const int rlim = ilv ? nrows : rend;
    uint32_t mrow[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int r = step_row(c) + lane;
      // (a block share's last block may reach past the sequence: its rows there are no members)
      mrow[c] = (r < rlim && (!bsh || lrow(r) < nb)) ? row_bits(gbw, c) : 0u;
    }
    if (lane < head) sm.hmp[lbase + lane] = (uint8_t)mrow[0];
    int cnt = head;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      if (step_row(c) >= rlim) break;
      const bool listed = mrow[c] != 0u && (c > 0 || lane >= head);
      const uint64_t bal = __ballot(listed);
      const int pre = __popcll(bal & ((1ull << lane) - 1ull));
      if (listed) {
        sm.list[lbase + cnt + pre] = (uint16_t)(step_row(c) + lane);
        sm.hmp[lbase + cnt + pre] = (uint8_t)mrow[c];
      }
      cnt += __popcll(bal);
    }
    nl_w = cnt;
    lim = lbase + nl_w;
  }
  __syncthreads();

  int nchunks = dense ? chunks_of(nlist) : (nl_w + CROWS - 1) / CROWS;
  if (!dense && nchunks > 1) {                // chunk 0 (the head) is on its way
    if (paged) load_chunk(1, kr[1], vr[1]);
    else load_chunk_b(1, kr[1], vr[1]);
  }

  auto compute_chunk = [&](int c, const uint4 (&kd)[TPC][KCH], const uint4 (&vd)[RSC][NV]) {
    // q . K on the matrix cores
    f32x4_t dacc[TPC];
#pragma unroll
    for (int t = 0; t < TPC; ++t) {
      dacc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KCH; ++kk) {
        if constexpr (F8) dacc[t] = mfma_bf16(fp8x8_to_bf16x8(kd[t][kk].x, kd[t][kk].y), qb[kk], dacc[t]);
        else dacc[t] = mfma_bf16(kd[t][kk], qb[kk], dacc[t]);
      }
    }
    // scores of head mr for rows tb + 4*mk + r
    float tl[TPC][4];
    float cm = -LD_INF;
#pragma unroll
    for (int t = 0; t < TPC; ++t) {
      const int tb = tbase(c, t);
      const int pos0 = tb + 4 * mk;
      uint32_t hm4 = 0;
      if (spm) hm4 = *reinterpret_cast<const uint32_t*>(&sm.hmp[pos0]);
      uint32_t bkey = 0u;                              // the lane's 4 rows share a 64-row block
      u32x4_t lv;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int pos = pos0 + r;
        const uint32_t hm = spm ? ((hm4 >> (8 * r)) & 0xffu) : ret;
        const bool mem = head_lane && pos < lim && ((hm >> mr) & 1u);
        const float s = dacc[t][r] * scale;
        lv[r] = __float_as_uint(s);
        if (ret_lane && pos < lim) {
          if (do_hist) atomicAdd(&sm.u.hist[mr][score_key(s) >> 21], 1u);
          if (do_blk) bkey = max(bkey, score_key(s));
        }
        tl[t][r] = mem ? s * kLog2e : -LD_INF;
        cm = fmaxf(cm, tl[t][r]);
      }
      if (lg_on && pos0 < lim) {
        const uint32_t o = lg_off + (uint32_t)pos0 * 4u;
        if (lg_vec && pos0 + 3 < lim) {
          if (lg_coh) __builtin_amdgcn_raw_buffer_store_b128(lv, lrs, o, 0, kSc1);
          else __builtin_amdgcn_raw_buffer_store_b128(lv, lrs, o, 0, 0);
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            if (pos0 + r < lim) {
              if (lg_coh) __builtin_amdgcn_raw_buffer_store_b32(lv[r], lrs, o + 4u * r, 0, kSc1);
              else __builtin_amdgcn_raw_buffer_store_b32(lv[r], lrs, o + 4u * r, 0, 0);
            }
          }
        }
      }
      if (do_blk && ret_lane && pos0 < lim) atomicMax(&sm.u.hist[mr][pos0 >> 6], bkey);
    }
    cm = max_xor32(max_xor16(cm));
    const float mn = fmaxf(m_lane, cm);
    const float mu = (mn == -LD_INF) ? 0.f : mn;
    const float alpha = exp2_fast(m_lane - mu);       // 0 when m_lane was -inf
    const bool grew = mn > m_lane;
    m_lane = mn;
    float ps = 0.f;
#pragma unroll
    for (int t = 0; t < TPC; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float pr = exp2_fast(tl[t][r] - mu);
        ps += pr;
        if (head_lane) sm.pl[wave][t * kTile + 4 * mk + r][mr] = pr;
      }
    l_lane = l_lane * (grew ? alpha : 1.f) + ps;
    // rescale the output accumulators of heads whose running max grew (wave-uniform)
#pragma unroll
    for (int j = 0; j < G; ++j) {
      const int gj = __builtin_amdgcn_readlane(__float_as_int(grew ? alpha : 1.f), j);
      const float aj = __int_as_float(gj);
      if (aj != 1.f) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[j][e] *= aj;
      }
    }
    // P . V
#pragma unroll
    for (int rs = 0; rs < RSC; ++rs) {
      const int tr = (rs >> 1) * kTile + (rs & 1) * 8 + rg;
      float pj[G];
#pragma unroll
      for (int j = 0; j < G; ++j) pj[j] = sm.pl[wave][tr][j];
      float vf[EPL];
#pragma unroll
      for (int c2 = 0; c2 < NV; ++c2) {
        if constexpr (F8) {
          fp8x4_to_f32(vd[rs][c2].x, &vf[c2 * 8]);
          fp8x4_to_f32(vd[rs][c2].y, &vf[c2 * 8 + 4]);
        } else {
          const uint32_t* vw = reinterpret_cast<const uint32_t*>(&vd[rs][c2]);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            vf[c2 * 8 + 2 * q] = bf_lo(vw[q]);
            vf[c2 * 8 + 2 * q + 1] = bf_hi(vw[q]);
          }
        }
      }
#pragma unroll
      for (int j = 0; j < G; ++j)
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[j][e] = fmaf(pj[j], vf[e], acc[j][e]);
    }
  };

  // ---- main loop: two chunks in flight while one is computed
  for (int c = 0; c < nchunks; c += 3) {
    if (c + 2 < nchunks) load_chunk(c + 2, kr[2], vr[2]);
    compute_chunk(c, kr[0], vr[0]);
    if (c + 1 < nchunks) {
      if (c + 3 < nchunks) load_chunk(c + 3, kr[0], vr[0]);
      compute_chunk(c + 1, kr[1], vr[1]);
      if (c + 2 < nchunks) {
        if (c + 4 < nchunks) load_chunk(c + 4, kr[1], vr[1]);
        compute_chunk(c + 2, kr[2], vr[2]);
      }
    }
  }

  // ---- flush the fused selection histogram
  if (do_hist && ret) {
    __syncthreads();
    for (int j = 0; j < G; ++j) {
      if (!(ret >> j & 1u)) continue;
      uint32_t* hg = hist1_mine(p.hist1, hq0 + j);
      for (int i = tid; i < kHist1Bins / 4; i += NT) {
        const uint4 c = reinterpret_cast<const uint4*>(sm.u.hist[j])[i];
        if (c.x) atomicAdd(hg + 4 * i + 0, c.x);
        if (c.y) atomicAdd(hg + 4 * i + 1, c.y);
        if (c.z) atomicAdd(hg + 4 * i + 2, c.z);
        if (c.w) atomicAdd(hg + 4 * i + 3, c.w);
      }
    }
  }
  // ---- block maxima of this split's rows (whole 64-row blocks: splits start at multiples
  // of 64 rows), as fp32 (NaN only for a block of NaN logits), one store per block
  if (do_blk && ret) {
    __syncthreads();
    const int nblk = p.seq_len / 64, b0 = r0 / 64, nbs = (nrows + 63) / 64;
    const int rb = b * __popcll(p.retrieval);
    for (int j = 0; j < G; ++j) {
      if (!(ret >> j & 1u)) continue;
      const int h = (hq0 + j) - b * p.Hq;
      float* dst = p.blk_out + (size_t)(rb + __popcll(p.retrieval & ((1ull << h) - 1ull))) * nblk + b0;
      for (int i = tid; i < nbs; i += NT) dst[i] = key_score(sm.u.hist[j][i]);
    }
  }
  __syncthreads();   // the LDS union is reused below

  // ---- wave totals: sum of head mr over the 4 k-groups; outputs over row pairs
  l_lane = add_xor32(add_xor16(l_lane));
#pragma unroll
  for (int j = 0; j < G; ++j)
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[j][e] += xor8_f(acc[j][e]);
  if (RP == 2) {
#pragma unroll
    for (int j = 0; j < G; ++j)
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[j][e] = add_xor16(acc[j][e]);
  }
  constexpr int RSTEP = 8 / RP;               // row slots folded into one part
  if ((rg % RSTEP) == 0) {
#pragma unroll
    for (int j = 0; j < G; ++j)
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const int d = (e < 8) ? (li * 8 + e) : (64 + li * 8 + (e - 8));
        sm.u.red.acc[wave][rg / RSTEP][j * D + d] = acc[j][e];
      }
  }
  if (lane < G) {
    sm.u.red.m[wave][lane] = m_lane;
    sm.u.red.l[wave][lane] = l_lane;
  }
  __syncthreads();

  // ---- merge the 4 waves and write this split's partials (4 dims per thread)
  for (int i = tid; i < G * (D / 4); i += NT) {
    const int j = i / (D / 4), d0 = (i % (D / 4)) * 4;
    if (!(act >> j & 1u)) continue;
    float M = -LD_INF;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, sm.u.red.m[w][j]);
    const float mu = (M == -LD_INF) ? 0.f : M;
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
    float L = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float sc = exp2_fast(sm.u.red.m[w][j] - mu);
      L += sm.u.red.l[w][j] * sc;
      float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int x2 = 0; x2 < RP; ++x2) {
        x.x += sm.u.red.acc[w][x2][j * D + d0 + 0];
        x.y += sm.u.red.acc[w][x2][j * D + d0 + 1];
        x.z += sm.u.red.acc[w][x2][j * D + d0 + 2];
        x.w += sm.u.red.acc[w][x2][j * D + d0 + 3];
      }
      a.x += x.x * sc; a.y += x.y * sc; a.z += x.z * sc; a.w += x.w * sc;
    }
    const size_t pslot = (size_t)(hq0 + j) * p.P + split;
    st_dev4_b(rsrc(p.part_acc + (size_t)hq0 * p.P * D), ((j * p.P + split) * D + d0) * 4, a);
    if (d0 == 0) {
      st_dev(p.part_ml + pslot * 2 + 0, M);
      st_dev(p.part_ml + pslot * 2 + 1, L);
    }
  }

  if (p.fin) {
    // ---- the last arrivals of the group finish it: the last one merges O; the nsel
    // before it each select retrieval rows of the group once it has arrived. They only
    // wait for splits of the launch that still have work, and the host keeps their
    // number far below the resident capacity, so every wait ends.
    const uint32_t selm = do_hist ? ret : 0u;
    const int nrow = __popc(selm);
    // The group's last arrivals finish it: the last one and the nmg - 1 before it merge
    // O, a slice of the output columns each; the nsel before those select the retrieval
    // rows: `parts` per row when the group has enough late splits and the budget allows
    // it, else one per row (whole rows, round robin); none: the last one selects them.
    // Helpers and selectors wait only for the last arrival, a split of the launch that
    // still has work; the host keeps their number below a quarter of the resident
    // capacity, so every wait ends.
    const int nmg = max(1, min(p.merge_w, nsplit_b));
    const int room = min(p.sel_cap, nsplit_b - nmg);
    int parts = nrow ? min(p.sel_parts, room / nrow) : 0;
    int nsel;
    if (parts >= 1) {
      nsel = nrow * parts;
    } else {
      parts = 1;
      nsel = max(0, min(nrow, room));
    }
    uint32_t* tk = p.tickets + b * p.Hkv + g;
    __builtin_amdgcn_s_waitcnt(0);            // partials, logits and counts are out
    __syncthreads();
    if (tid == 0)
      sm.misc[0] = (int)__hip_atomic_fetch_add(tk, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    const int t = sm.misc[0];
    // release flags: [0, nmg - 1) merge helpers, then the selectors; set by the last
    // arrival, cleared by their reader
    uint64_t* rel = p.gb_rel + (size_t)(b * p.Hkv + g) * p.P * kRelStride;
    const int late = nsplit_b - 1 - t;        // 0: the last arrival
    constexpr int COLS = G * (D / 4);
    int f = -1;                               // selector index
    if (late == 0) {
      // every split is in: release the others (the selectors once their rows' counters
      // are clear), and clear the ticket for the next call (ordered after this launch)
      if (nsel) {
        if (tid < G && (selm >> tid & 1u)) st_dev(p.sel_cnt + (size_t)(hq0 + tid) * 2, 0u);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
      }
      if (nmg - 1 + nsel) group_publish(rel, nmg - 1 + nsel, (uint64_t)1);
      if (tid == 0) st_dev(tk, 0u);
    } else if (late < nmg + nsel) {
      group_wait(rel, late - 1, (uint64_t)1, p.err);
      if (tid == 0) st_dev(rel + (size_t)(late - 1) * kRelStride, (uint64_t)0);   // ready for the next call
      if (late >= nmg) f = late - nmg;
    } else {
      return;
    }
    if (late < nmg) {
      merge_final<D, G, NW>(p, act, hq0, nsplit_b, late * COLS / nmg, (late + 1) * COLS / nmg);
      if (!(late == 0 && nsel == 0)) return;
    }
    // this workgroup's rows: with parts > 1, part f % parts of row f / parts; else rows
    // i with i % nsel == f (the last arrival takes them all when nsel is 0)
    int i = 0;
    for (int j = 0; j < G; ++j) {
      if (!(selm >> j & 1u)) continue;
      int part = 0;
      bool mine;
      if (parts > 1) {
        mine = f >= 0 && f < nsel && f / parts == i;
        part = f % parts;
      } else {
        mine = nsel ? (f >= 0 && f < nsel && i % nsel == f) : (late == 0);
      }
      ++i;
      if (mine)
        part_select<NW>(sm.u.sel.hist, sm.u.sel.cand, sm.wcnt, sm.res, sm.tmp4, sm.poff, sm.pcnt, p, hq0 + j, nb,
                        part, parts);
    }
    return;
  }

  // ---- two-level merge: the last split of each run of kMergeRun splits merges the run
  // into a level-1 partial while other splits still stream; the last run of (b, g)
  // merges the level-1 partials into O. One run only: straight into O.
  const int nu = (nsplit_b + kMergeRun - 1) / kMergeRun;
  const int u = split / kMergeRun;
  uint32_t* t2 = p.tickets + b * p.Hkv + g;
  if (nu == 1) {
    if (!arrive_last(t2, (uint32_t)nsplit_b, &sm.misc[0])) return;
    if (tid == 0) *t2 = 0u;
    merge_splits<D, G, NW, true>(sm, p, act, hq0, p.part_ml, p.part_acc, p.P, 0, nsplit_b, nullptr, nullptr, 0);
  } else {
    uint32_t* t1 = p.tickets_l1 + (size_t)(b * p.Hkv + g) * p.P1 + u;
    const int ucnt = min(kMergeRun, nsplit_b - u * kMergeRun);
    if (!arrive_last(t1, (uint32_t)ucnt, &sm.misc[0])) return;
    if (tid == 0) *t1 = 0u;
    merge_splits<D, G, NW, false>(sm, p, act, hq0, p.part_ml, p.part_acc, p.P, u * kMergeRun, ucnt,
                                  p.l1_ml, p.l1_acc, u);
    if (!arrive_last(t2, (uint32_t)nu, &sm.misc[0])) return;
    if (tid == 0) *t2 = 0u;
    merge_splits<D, G, NW, true>(sm, p, act, hq0, p.l1_ml, p.l1_acc, p.P1, 0, nu, nullptr, nullptr, 0);
  }

  // (the selection launches that follow read the fused digit-1 histogram: each of their
  // workgroups finds the first digit from it while its own scores load)
}

template <int D, int G, bool F8, bool PG>
int64_t capacity_dgf(int waves) {
  int per_cu = 0;
  hipError_t e;
  if (waves == 8)
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_attention<D, G, 8, F8, false, PG>, 512, 0);
  else
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_attention<D, G, 4, F8, false, PG>, 256, 0);
  return e == hipSuccess ? per_cu : 0;
}

template <int D, int G, bool F8, bool PG>
hipError_t launch_dgf(const AttnParams& p, dim3 grid, hipStream_t st) {
  if (p.waves == 8)
    hipLaunchKernelGGL((k_attention<D, G, 8, F8, false, PG>), grid, dim3(512), 0, st, p);
  else
    hipLaunchKernelGGL((k_attention<D, G, 4, F8, false, PG>), grid, dim3(256), 0, st, p);
  return hipGetLastError();
}

// token-block sets: the 4-wave block instance (the host sets 4 waves for them)
template <int D, int G, bool F8>
hipError_t launch_dgf_blk(const AttnParams& p, dim3 grid, hipStream_t st) {
  hipLaunchKernelGGL((k_attention<D, G, 4, F8, true>), grid, dim3(256), 0, st, p);
  return hipGetLastError();
}

}  // namespace

// This file is compiled once per KV group size (LD_ATTN_G = 1, 2, 4 or 8) and kind of
// instance (LD_ATTN_BLK 1: sets of whole token blocks; else LD_ATTN_PG 1: token sets
// over paged KV; neither: token sets over contiguous KV), so that the kernel instances
// compile in parallel, each kind in a code object of its own; the dispatch is in
// ld_api.hip.
#ifndef LD_ATTN_G
#error "compile ld_attention.hip with -DLD_ATTN_G=<1|2|4|8>"
#endif
#ifndef LD_ATTN_BLK
#define LD_ATTN_BLK 0
#endif
#ifndef LD_ATTN_PG
#define LD_ATTN_PG 0
#endif

#if LD_ATTN_BLK
template <int G>
hipError_t launch_attention_blk_g(const AttnParams& p, int D, dim3 grid, hipStream_t st) {
  if (D == 128) return p.kv_fp8 ? launch_dgf_blk<128, G, true>(p, grid, st) : launch_dgf_blk<128, G, false>(p, grid, st);
  if (D == 64) return p.kv_fp8 ? launch_dgf_blk<64, G, true>(p, grid, st) : launch_dgf_blk<64, G, false>(p, grid, st);
  return hipErrorInvalidValue;
}

template hipError_t launch_attention_blk_g<LD_ATTN_G>(const AttnParams&, int, dim3, hipStream_t);
#elif LD_ATTN_PG
template <int G>
int64_t attention_capacity_pg_g(int D, int waves, bool fp8) {
  if (D == 128) return fp8 ? capacity_dgf<128, G, true, true>(waves) : capacity_dgf<128, G, false, true>(waves);
  return fp8 ? capacity_dgf<64, G, true, true>(waves) : capacity_dgf<64, G, false, true>(waves);
}

template <int G>
hipError_t launch_attention_pg_g(const AttnParams& p, int D, dim3 grid, hipStream_t st) {
  if (D == 128)
    return p.kv_fp8 ? launch_dgf<128, G, true, true>(p, grid, st) : launch_dgf<128, G, false, true>(p, grid, st);
  if (D == 64)
    return p.kv_fp8 ? launch_dgf<64, G, true, true>(p, grid, st) : launch_dgf<64, G, false, true>(p, grid, st);
  return hipErrorInvalidValue;
}

template int64_t attention_capacity_pg_g<LD_ATTN_G>(int, int, bool);
template hipError_t launch_attention_pg_g<LD_ATTN_G>(const AttnParams&, int, dim3, hipStream_t);
#else
template <int G>
int64_t attention_capacity_g(int D, int waves, bool fp8) {
  if (D == 128) return fp8 ? capacity_dgf<128, G, true, false>(waves) : capacity_dgf<128, G, false, false>(waves);
  return fp8 ? capacity_dgf<64, G, true, false>(waves) : capacity_dgf<64, G, false, false>(waves);
}

template <int G>
hipError_t launch_attention_g(const AttnParams& p, int D, dim3 grid, hipStream_t st) {
  if (D == 128)
    return p.kv_fp8 ? launch_dgf<128, G, true, false>(p, grid, st) : launch_dgf<128, G, false, false>(p, grid, st);
  if (D == 64)
    return p.kv_fp8 ? launch_dgf<64, G, true, false>(p, grid, st) : launch_dgf<64, G, false, false>(p, grid, st);
  return hipErrorInvalidValue;
}

template int64_t attention_capacity_g<LD_ATTN_G>(int, int, bool);
template hipError_t launch_attention_g<LD_ATTN_G>(const AttnParams&, int, dim3, hipStream_t);
#endif

}  // namespace ld
