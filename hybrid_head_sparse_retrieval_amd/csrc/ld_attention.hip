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
  int misc[4];
  uint64_t relw;                     // release word seen by thread 0
  uint32_t res[2];
  int scan[NW][kMaxSplitRows / (64 * NW) / 2 > 2 ? kMaxSplitRows / (64 * NW) / 2 : 2];   // wave totals of scans
  int cnt4[NW][2];
  int ncnt[kRep];                    // candidate counts of the sub-lists
  int pages[kMaxSplitRows / 16 + 1]; // paged KV: page ids of the split's rows
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
  // maxima and sums of every (head, split) in one round
  for (int i = tid; i < G * cnt; i += NT) {
    const int jj = i / cnt, ss = i % cnt;
    if (act >> jj & 1u) {
      const size_t ms = ((size_t)(hq0 + jj) * stride + s0 + ss) * 2;
      sm.u.cmb.w[jj][ss] = ld_dev(src_ml + ms);
      sm.u.cmb.lp[jj][ss] = ld_dev(src_ml + ms + 1);
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

// ---- group-barrier mode

// O of a group from its ns split partials, spread over the group's workgroups: wave w
// of split s merges the float4 columns (s * NW + w) + t * ns * NW; its lanes run over
// the splits.
template <int D, int G, int NW>
__device__ __forceinline__ void merge_columns(const AttnParams& p, uint32_t act, int hq0, int split, int ns) {
  constexpr int NC = G * (D / 4);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  for (int c = split * NW + wave; c < NC; c += ns * NW) {
    const int j = c / (D / 4), d0 = (c % (D / 4)) * 4;
    if (!(act >> j & 1u)) continue;
    const float* ml = p.part_ml + (size_t)(hq0 + j) * p.P * 2;
    const __amdgpu_buffer_rsrc_t rr = rsrc(p.part_acc + (size_t)(hq0 + j) * p.P * D);
    float L = 0.f;
    float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
    if (ns <= 64) {
      float m = -LD_INF, l = 0.f;
      float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
      if (lane < ns) {
        m = ld_dev(ml + lane * 2);
        l = ld_dev(ml + lane * 2 + 1);
        a = ld_dev4_b(rr, (lane * D + d0) * 4);
      }
      const float M = wave_max_f(m);
      const float w = exp2_fast(m - ((M == -LD_INF) ? 0.f : M));   // 0 for unused lanes
      L = l * w;
      o = make_float4(a.x * w, a.y * w, a.z * w, a.w * w);
    } else {
      float M = -LD_INF;
      for (int s2 = lane; s2 < ns; s2 += 64) M = fmaxf(M, ld_dev(ml + s2 * 2));
      M = wave_max_f(M);
      const float mu = (M == -LD_INF) ? 0.f : M;
      for (int s2 = lane; s2 < ns; s2 += 64) {
        const float w = exp2_fast(ld_dev(ml + s2 * 2) - mu);
        L = fmaf(ld_dev(ml + s2 * 2 + 1), w, L);
        const float4 a = ld_dev4_b(rr, (s2 * D + d0) * 4);
        o.x = fmaf(a.x, w, o.x); o.y = fmaf(a.y, w, o.y); o.z = fmaf(a.z, w, o.z); o.w = fmaf(a.w, w, o.w);
      }
    }
    L = wave_sum_f(L);
    o.x = wave_sum_f(o.x); o.y = wave_sum_f(o.y); o.z = wave_sum_f(o.z); o.w = wave_sum_f(o.w);
    if (lane == 0) store_o<D>(p, hq0 + j, d0, o, p.v_scale / L);
  }
}

// Exclusive prefix of 0/1 flags in row order (row = i * NT + thread) over the
// workgroup, for IT items per thread: ex[i] = flags of earlier rows, tot[i] = flags of
// item i over the workgroup. Two items share an int (16-bit fields).
template <int NW, int IT>
__device__ __forceinline__ void rows_scan(const uint32_t (&f)[IT], int (&ex)[IT], int (&tot)[IT],
                                          int (&lds)[NW][IT / 2]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int inc[IT / 2], val[IT / 2];
#pragma unroll
  for (int q = 0; q < IT / 2; ++q) {
    val[q] = (int)(f[2 * q] | (f[2 * q + 1] << 16));
    inc[q] = wave_incl_sum(val[q]);
    if (lane == 63) lds[wave][q] = inc[q];
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < IT / 2; ++q) {
    int below = 0, all = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const int t = lds[w][q];
      below += (w < wave) ? t : 0;
      all += t;
    }
    const int e = below + inc[q] - val[q];
    ex[2 * q] = e & 0xffff;
    ex[2 * q + 1] = e >> 16;
    tot[2 * q] = all & 0xffff;
    tot[2 * q + 1] = all >> 16;
  }
  __syncthreads();
}

// Digit 1 of row `slot` (bin b1 and k1, the keys still to take from it) from the sum
// of its histogram replicas, stored in sel_info for the selection launch.
template <int D, int G, int NW>
__device__ __forceinline__ void digit1_info(AttnSmem<D, G, NW>& sm, const AttnParams& p, int slot, int kk) {
  constexpr int NT = 64 * NW;
  const int tid = threadIdx.x;
  uint32_t* hs = sm.u.sel.hist;
  __syncthreads();    // the LDS union is free
  if (kk >= 1) hist1_sum(hs, p.hist1, slot);
  if (tid == 0) { sm.res[0] = 0; sm.res[1] = 0; }
  __syncthreads();
  if (kk >= 1) find_bin_from_top<kHist1Bins, NT>([&](int i) { return hs[i]; }, (uint32_t)kk, sm.wcnt, sm.res);
  __syncthreads();
  if (tid == 0) {
    p.sel_info[slot * 4 + 0] = sm.res[0];
    p.sel_info[slot * 4 + 1] = (uint32_t)kk - sm.res[1];
  }
}

// k of the row: the row's selection length, at most the sequence length nb.
__device__ __forceinline__ int select_k(const AttnParams& p, int slot, int nb) {
  int kk = p.k_dense;
  if (p.s_indptr) kk = (int)(p.s_indptr[slot + 1] - p.s_indptr[slot]);
  return min(kk, nb);
}

// Digit 1 of the row's threshold from its digit-1 histogram (the sum of the kRep
// replicas), taken once per group by the workgroup that completed the group's first
// barrier, and published to the group as stage 2 of the release words, with the
// payload b1 (the bin, bits 0..31) and k1 (the keys still to take from it, bits 32..63).
template <int D, int G, int NW>
__device__ __forceinline__ void publish_digit1(AttnSmem<D, G, NW>& sm, const AttnParams& p, int slot, int kk,
                                               uint64_t* rel, int ns, uint32_t epoch) {
  constexpr int NT = 64 * NW;
  constexpr int PB1 = kHist1Bins / NT;          // digit-1 bins per thread
  const int tid = threadIdx.x;
  uint32_t* hs = sm.u.sel.hist;                 // free until the selection below
  hist1_sum(hs, p.hist1, slot);
  if (tid == 0) { sm.res[0] = 0; sm.res[1] = 0; }
  __syncthreads();
  uint32_t h[PB1];
#pragma unroll
  for (int q = 0; q < PB1; ++q) h[q] = hs[tid * PB1 + q];
  find_bin_regs<kHist1Bins, NT>(h, (uint32_t)kk, sm.wcnt, sm.res);
  const uint32_t b1 = sm.res[0], k1 = (uint32_t)kk - sm.res[1];
  __syncthreads();
  group_publish(rel, ns, rel_word(epoch, 2u), (uint64_t)b1 | ((uint64_t)k1 << 32));
}

// argsTopK of the group's one retrieval head by the workgroups of the group, each over
// its own rows (r0 .. r0 + nrows), with one more group barrier: every split takes
// digit 1 (b1, k1) from its release word, appends its candidates (keys whose digit 1
// is b1) to the candidate sub-list of its replica and publishes its count of keys
// above bin b1; after the barrier every split derives the threshold key T from all
// candidates (digits 2 and 3), its output offset from the earlier splits' counts, and
// writes its kept rows (keys equal to T are kept in row order, so the lower indices
// win ties).
template <int D, int G, int NW>
__device__ __forceinline__ void group_select(AttnSmem<D, G, NW>& sm, const AttnParams& p, uint32_t ret,
                                             int hq0, int split, int ns, int bid0, int nb, int r0, int nrows,
                                             uint32_t* gc, uint64_t* rel, uint32_t epoch) {
  constexpr int NT = 64 * NW;
  constexpr int IT = kMaxSplitRows / NT;        // rows per thread
  constexpr int SPEC = 32;                      // candidates fetched per thread before the counts
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  // the group's one retrieval head (the launch takes this path only when there is one)
  const int slot = hq0 + __builtin_ctz(ret);
  const int kk = select_k(p, slot, nb);
  if (kk < 1) return;                           // the same in every split of the group

  // ---- keys of this split's rows; digit 1
  uint32_t key[IT];
  {
    const float* lg = p.logits + (size_t)slot * p.seq_len + r0;
#pragma unroll
    for (int i = 0; i < IT; ++i) {
      const int r = i * NT + tid;
      key[i] = (r < nrows) ? score_key(ld_dev(lg + r)) : 0u;
    }
  }
  const uint64_t w1 = group_wait_payload(rel, split, rel_word(epoch, 2u), p.err, &sm.relw);
  const uint32_t b1 = (uint32_t)w1 & 0x7ffu, k1 = (uint32_t)(w1 >> 32);
  uint32_t* rcnt = p.row_cnt + ((size_t)(epoch & 1u) * p.B * p.Hq + slot) * kRep;   // this call's counts
  {
    // ---- append the candidates to the row's list; publish the count above bin b1
    uint32_t cm = 0;
    int na = 0;
#pragma unroll
    for (int i = 0; i < IT; ++i) {
      const bool v = i * NT + tid < nrows;
      const uint32_t d1 = key[i] >> 21;
      na += (v && d1 > b1) ? 1 : 0;
      cm |= (uint32_t)(v && d1 == b1) << i;
    }
    int wt;
    const int before = wave_excl_scan(__popc(cm), wt);
    const int wa = wave_total(na);
    if (lane == 0) { sm.scan[wave][0] = wt; sm.scan[wave][1] = wa; }
    __syncthreads();
    int woff = 0, tot = 0, atot = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      woff += (w < wave) ? sm.scan[w][0] : 0;
      tot += sm.scan[w][0];
      atot += sm.scan[w][1];
    }
    const int rep = rep_of_block();
    if (tid == 0) {
      sm.misc[2] = tot ? (int)__hip_atomic_fetch_add(rcnt + rep, (uint32_t)tot,
                                                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0;
      st_dev(p.pub + ((size_t)slot * p.P + split) * 2, (uint32_t)atot);
    }
    __syncthreads();
    // a candidate shares digit 1 with the others: it is stored as its split and the
    // low 21 bits of its key
    uint32_t* cl = p.cand + ((size_t)slot * kRep + rep) * p.sub_cap + sm.misc[2] + woff + before;
    int q = 0;
#pragma unroll
    for (int i = 0; i < IT; ++i) {
      if (cm >> i & 1u) {
        st_dev(cl + q, ((uint32_t)split << 21) | (key[i] & 0x1fffffu));
        ++q;
      }
    }
  }
  group_barrier(gc + (kRep + 1), rel, split, ns, bid0, rel_word(epoch, 3u), p.err, &sm.misc[1]);

  // ---- threshold from the whole candidate list, offset, write
  // The candidates sit in kRep sub-lists; the first PER entries of each are fetched
  // before the counts are known (entries past a count are ignored): register u holds
  // entry (u / kRep) * NT + tid of sub-list u % kRep. All of them then go to LDS
  // (sub-list after sub-list) when they fit, and the passes below read them there.
  static_assert(SPEC % kRep == 0, "speculative loads cover the sub-lists evenly");
  constexpr int PER = SPEC / kRep * NT;
  const uint32_t* cl = p.cand + (size_t)slot * kRep * p.sub_cap;
  uint32_t cv[SPEC];
#pragma unroll
  for (int u = 0; u < SPEC; ++u) cv[u] = ld_dev(cl + (size_t)(u % kRep) * p.sub_cap + (u / kRep) * NT + tid);
  if (tid < kRep) sm.ncnt[tid] = (int)ld_dev(rcnt + tid);
  int above = 0;                                  // keys above bin b1 in earlier splits
  for (int s2 = tid; s2 < split; s2 += NT) above += (int)ld_dev(p.pub + ((size_t)slot * p.P + s2) * 2);
  uint32_t* h2 = sm.u.sel.hist;                   // [kHist2Bins]
  uint32_t* h3 = h2 + kHist2Bins;                 // [kHist3Bins]
  uint32_t* cs = sm.u.sel.cand;                   // [kCandLds]
  for (int i = tid; i < kHist2Bins + kHist3Bins; i += NT) h2[i] = 0u;
  if (tid == 0) { sm.res[0] = 0; sm.res[1] = 0; }
  __syncthreads();
  int total = 0;
#pragma unroll
  for (int r = 0; r < kRep; ++r) total += sm.ncnt[r];
  const bool in_lds = total <= kCandLds;
  if (in_lds) {
    int off = 0;
#pragma unroll
    for (int r = 0; r < kRep; ++r) {
      const int n = sm.ncnt[r];
#pragma unroll
      for (int v = 0; v < SPEC / kRep; ++v) {
        const int o = v * NT + tid;
        if (o < n) cs[off + o] = cv[v * kRep + r];
      }
      for (int o = PER + tid; o < n; o += NT) cs[off + o] = ld_dev(cl + (size_t)r * p.sub_cap + o);
      off += n;
    }
    __syncthreads();
  }
  // visit(f): every candidate once, as its split and its full key
  auto for_cands = [&](auto f) {
    auto g = [&](uint32_t e) { f((b1 << 21) | (e & 0x1fffffu), (int)(e >> 21)); };
    if (in_lds) {
#pragma unroll 4
      for (int i = tid; i < total; i += NT) g(cs[i]);
    } else {
      for (int r = 0; r < kRep; ++r) {
        const int n = sm.ncnt[r];
        for (int o = tid; o < n; o += NT) g(ld_dev(cl + (size_t)r * p.sub_cap + o));
      }
    }
  };
  for_cands([&](uint32_t kv, int) { atomicAdd(&h2[(kv >> 10) & 0x7ffu], 1u); });
  __syncthreads();
  find_bin_from_top<kHist2Bins, NT>([&](int i) { return h2[i]; }, k1, sm.wcnt, sm.res);
  const uint32_t b2 = sm.res[0];
  const uint32_t k2 = k1 - sm.res[1];
  const uint32_t pre = (b1 << 11) | b2;
  __syncthreads();    // every wave has read the result before it is cleared
  if (tid == 0) { sm.res[0] = 0; sm.res[1] = 0; }
  __syncthreads();
  for_cands([&](uint32_t kv, int) { if ((kv >> 10) == pre) atomicAdd(&h3[kv & 0x3ffu], 1u); });
  __syncthreads();
  find_bin_from_top<kHist3Bins, NT>([&](int i) { return h3[i]; }, k2, sm.wcnt, sm.res);
  const uint32_t T = (pre << 10) | sm.res[0];
  const int et = (int)(k2 - sm.res[1]);           // keys equal to T that are kept
  // candidates of earlier splits above and equal to T; keys equal to T here
  int ga = 0, ge = 0, me = 0;
  for_cands([&](uint32_t kv, int s2) {
    const int early = s2 < split ? 1 : 0, here = s2 == split ? 1 : 0;
    const int gt1 = kv > T ? 1 : 0, eq1 = kv == T ? 1 : 0;
    ga += early & gt1;
    ge += early & eq1;
    me += here & eq1;
  });
  {
    // the four sums in one exchange
    const int w0 = wave_total(above), w1 = wave_total(ga), w2 = wave_total(ge), w3 = wave_total(me);
    if (lane == 0) { sm.scan[wave][0] = w0; sm.scan[wave][1] = w1; }
    if (lane == 0) { sm.cnt4[wave][0] = w2; sm.cnt4[wave][1] = w3; }
    __syncthreads();
    above = 0; ga = 0; ge = 0; me = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      above += sm.scan[w][0]; ga += sm.scan[w][1]; ge += sm.cnt4[w][0]; me += sm.cnt4[w][1];
    }
    __syncthreads();
  }
  const int off = above + ga + min(et, ge);       // kept rows of earlier splits
  const int keep_e = max(0, min(et - ge, me));    // kept keys equal to T here
  uint32_t gt[IT], eq[IT], kp[IT];
#pragma unroll
  for (int i = 0; i < IT; ++i) {
    const bool v = i * NT + tid < nrows;
    gt[i] = (v && key[i] > T) ? 1u : 0u;
    eq[i] = (v && key[i] == T) ? 1u : 0u;
  }
  if (keep_e == me) {
#pragma unroll
    for (int i = 0; i < IT; ++i) kp[i] = gt[i] | eq[i];
  } else if (keep_e == 0) {
#pragma unroll
    for (int i = 0; i < IT; ++i) kp[i] = gt[i];
  } else {
    int ex[IT], tot[IT];
    rows_scan<NW, IT>(eq, ex, tot, sm.scan);
    int before = 0;
#pragma unroll
    for (int i = 0; i < IT; ++i) {
      kp[i] = gt[i] | ((eq[i] && before + ex[i] < keep_e) ? 1u : 0u);
      before += tot[i];
    }
  }
  int ex[IT], tot[IT];
  rows_scan<NW, IT>(kp, ex, tot, sm.scan);
  int64_t so;
  int klen;
  if (p.s_indptr) { so = p.s_indptr[slot]; klen = (int)(p.s_indptr[slot + 1] - so); }
  else { so = (int64_t)slot * p.k_dense; klen = p.k_dense; }
  klen = min(klen, nb);
  int32_t* out = p.s_out + so;
  uint32_t* bm = p.bitmaps ? p.bitmaps + (size_t)slot * p.W : nullptr;
  int base = off;
#pragma unroll
  for (int i = 0; i < IT; ++i) {
    const int r = i * NT + tid;
    const int pos = base + ex[i];
    if (kp[i] && pos < klen) out[pos] = r0 + r;
    base += tot[i];
    if (bm) {
      const uint64_t bal = __ballot(kp[i] != 0u);
      // first row of this lane's word; words past this split's rows are another
      // split's (splits are whole words: r0 and the split size are multiples of 32)
      const int rr = i * NT + wave * 64 + (lane & 32);
      const int row32 = r0 + rr;
      if ((lane & 31) == 0 && rr < nrows && (row32 >> 5) < p.W)
        bm[row32 >> 5] = (uint32_t)(bal >> (lane & 32));
    }
  }
  __syncthreads();
}

// F8: K and V hold E4M3 codes (one byte per element, dequantised exactly to bf16 /
// fp32 in registers; their per-tensor scales are folded into p.scale and p.v_scale).
template <int D, int G, int NW, bool F8>
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

  int bid = blockIdx.x;
  const int dense_blocks = p.B * p.ng_dense * p.nsplit_d;
  int split, gi, b, ts, bid0;                 // bid0: id of the group's first split
  if (bid < dense_blocks) {
    split = bid % p.nsplit_d;
    bid0 = bid - split;
    bid /= p.nsplit_d;
    gi = bid % p.ng_dense;
    b = bid / p.ng_dense;
    ts = p.ts_d;
  } else {
    const int ngs = p.ngroups - p.ng_dense;
    bid -= dense_blocks;
    split = bid % p.nsplit_s;
    bid0 = dense_blocks + bid - split;
    bid /= p.nsplit_s;
    gi = p.ng_dense + bid % ngs;
    b = bid / ngs;
    ts = p.ts_s;
  }
  const int g = p.groups[gi];

  const bool paged = p.page_shift != 0;
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
  const int r0 = split * ts;
  const int nrows = min(ts, nb - r0);

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
    if (!paged) return (ptrdiff_t)r * D;
    const int i = r0 + r;
    return (((ptrdiff_t)sm.pages[(i >> pshift) - pg0] << pshift) + (i & pmask) - r0) * D;
  };
  // Stream mode: the waves take interleaved 16-row tiles of the split. Gather mode:
  // each wave owns a contiguous block of the split's rows and visits the members of
  // its own block (its own visit list at lbase, nl_w entries), so the list needs no
  // workgroup-wide step.
  int nlist = nrows;
  int lbase = 0, nl_w = 0;
  auto chunks_of = [&](int n) {
    const int ntiles = (n + kTile - 1) / kTile;
    const int my_tiles = ntiles > wave ? (ntiles - wave + NW - 1) / NW : 0;
    return (my_tiles + TPC - 1) / TPC;
  };
  auto tbase = [&](int c, int t) -> int {
    return dense ? (wave + NW * (c * TPC + t)) * kTile : lbase + (c * TPC + t) * kTile;
  };
  int lim = nrows;                            // visit positions below lim are valid

  const bool head_lane = mr < G;
  const bool ret_lane = head_lane && ((ret >> mr) & 1u);
  float* lg = (p.logits && ret_lane) ? p.logits + (size_t)(hq0 + mr) * p.seq_len + r0 : nullptr;
  const float scale = p.scale;

  float m_lane = -LD_INF, l_lane = 0.f;     // running max / sum of head mr (lanes mr < G)
  float acc[G][EPL];
#pragma unroll
  for (int j = 0; j < G; ++j)
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[j][e] = 0.f;

  uint4 kr[3][TPC][KCH], vr[3][RSC][NV];

  auto row_of = [&](int pos) -> int { return dense ? pos : (int)sm.list[pos]; };
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
          kd[t][kk] = va ? *reinterpret_cast<const uint4*>(kp + kk * 64) : make_uint4(0, 0, 0, 0);
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
            vd[t * 2 + h2][c2] = vv ? *reinterpret_cast<const uint4*>(vp + c2 * 128) : make_uint4(0, 0, 0, 0);
          }
        }
      }
    }
  };

  if (dense) {
    const int nc0 = chunks_of(nrows);
    if (nc0 > 0) load_chunk(0, kr[0], vr[0]);
    if (nc0 > 1) load_chunk(1, kr[1], vr[1]);
  }

  // ---- membership of each row of the tile, and the visit list
  if (do_hist && ret) {
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
    // rows owned by this wave: [lbase, lbase + R) of the split, 64 per ballot
    constexpr int CH = kMaxSplitRows / (64 * NW);
    static_assert(2 * CH <= 64, "one word per lane");
    const int R = ((ts + 64 * NW - 1) / (64 * NW)) * 64;
    lbase = wave * R;
    const int rend = min(nrows, lbase + R);
    uint32_t bw[G];
    {
      const int word = ((r0 + lbase) >> 5) + lane;
      const bool ok = lane < 2 * CH && lbase + 32 * lane < rend && word < p.W;
#pragma unroll
      for (int j = 0; j < G; ++j)
        bw[j] = ((spm >> j & 1) && ok) ? p.bitmaps[(size_t)(hq0 + j) * p.W + word] : 0u;
    }
    uint32_t mrow[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int r = lbase + c * 64 + lane;
      mrow[c] = r < rend ? row_bits(bw, c) : 0u;
    }
    int cnt = 0;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      if (lbase + c * 64 >= rend) break;
      const uint64_t bal = __ballot(mrow[c] != 0u);
      const int pre = __popcll(bal & ((1ull << lane) - 1ull));
      if (mrow[c]) {
        sm.list[lbase + cnt + pre] = (uint16_t)(lbase + c * 64 + lane);
        sm.hmp[lbase + cnt + pre] = (uint8_t)mrow[c];
      }
      cnt += __popcll(bal);
    }
    nl_w = cnt;
    lim = lbase + nl_w;
  }
  __syncthreads();

  // the group's epoch for the in-launch barriers, fetched here (after the membership
  // words, before the first gathered rows) so that it has long arrived when the
  // workgroup reaches its first barrier
  const uint32_t epoch0 = p.gb ? ld_dev(p.gb_cnt + (size_t)(b * p.Hkv + g) * kGbCounters + kEpochWord) : 0u;
  int nchunks = dense ? chunks_of(nlist) : (nl_w + CROWS - 1) / CROWS;
  if (!dense) {
    if (nchunks > 0) load_chunk(0, kr[0], vr[0]);
    if (nchunks > 1) load_chunk(1, kr[1], vr[1]);
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
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int pos = pos0 + r;
        const uint32_t hm = spm ? ((hm4 >> (8 * r)) & 0xffu) : ret;
        const bool mem = head_lane && pos < lim && ((hm >> mr) & 1u);
        const float s = dacc[t][r] * scale;
        if (ret_lane && pos < lim) {
          if (lg) lg[pos] = s;                           // stream mode: pos is the row
          if (do_hist) atomicAdd(&sm.u.hist[mr][score_key(s) >> 21], 1u);
        }
        tl[t][r] = mem ? s * kLog2e : -LD_INF;
        cm = fmaxf(cm, tl[t][r]);
      }
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

  if (p.gb) {
    uint32_t* gc = p.gb_cnt + (size_t)(b * p.Hkv + g) * kGbCounters;
    uint64_t* rel = p.gb_rel + (size_t)(b * p.Hkv + g) * p.P * kRelStride;
    // This call's epoch of the group (read in the prologue, before arriving; the
    // workgroup that completes the first barrier advances it for the next call).
    const uint32_t epoch = epoch0 + 1u;
    const bool rl = group_barrier(gc, rel, split, nsplit_b, bid0, rel_word(epoch, 1u), p.err, &sm.misc[1]);
    if (rl) {
      if (tid == 0) st_dev(gc + kEpochWord, epoch);
      // the next call's candidate counts of the group's rows start at zero
      if (tid < G * kRep)
        p.row_cnt[((size_t)((epoch + 1u) & 1u) * p.B * p.Hq + hq0) * kRep + tid] = 0u;
    }
    if (do_hist && ret && p.gb_select) {
      if (rl) {
        // the only reader of the row's histogram: clears it once digit 1 is out
        const int slot = hq0 + __builtin_ctz(ret), kk = select_k(p, slot, nb);
        if (kk >= 1) publish_digit1<D, G, NW>(sm, p, slot, kk, rel, nsplit_b, epoch);
        hist1_clear(p.hist1, slot);
      }
      merge_columns<D, G, NW>(p, act, hq0, split, nsplit_b);
      group_select<D, G, NW>(sm, p, ret, hq0, split, nsplit_b, bid0, nb, r0, nrows, gc, rel, epoch);
    } else {
      // digit 1 of the i-th retrieval row of the group by split i (mod the splits)
      if (do_hist && ret) {
        int i = 0;
        for (int j = 0; j < G; ++j) {
          if (!(ret >> j & 1u)) continue;
          if (i % nsplit_b == split) {
            digit1_info<D, G, NW>(sm, p, hq0 + j, select_k(p, hq0 + j, nb));
            hist1_clear(p.hist1, hq0 + j);
          }
          ++i;
        }
      }
      merge_columns<D, G, NW>(p, act, hq0, split, nsplit_b);
    }
    // nothing to clear on the way out: barrier counters return to zero by themselves,
    // release words carry the epoch, histograms are cleared by their readers and the
    // next call's counts were cleared above
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

  // ---- first selection digit for each retrieval head (fused histogram complete)
  if (do_hist) {
    for (int j = 0; j < G; ++j) {
      if (!(ret >> j & 1u)) continue;
      const int slot = hq0 + j;
      digit1_info<D, G, NW>(sm, p, slot, select_k(p, slot, nb));
      hist1_clear(p.hist1, slot);
      __syncthreads();
    }
  }
}

template <int D, int G, bool F8>
int64_t capacity_dgf(int waves) {
  int per_cu = 0;
  hipError_t e;
  if (waves == 8)
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_attention<D, G, 8, F8>, 512, 0);
  else
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_attention<D, G, 4, F8>, 256, 0);
  return e == hipSuccess ? per_cu : 0;
}
template <int D, int G>
int64_t capacity_dg(int waves, bool fp8) {
  return fp8 ? capacity_dgf<D, G, true>(waves) : capacity_dgf<D, G, false>(waves);
}

template <int D, int G, bool F8>
hipError_t launch_dgf(const AttnParams& p, dim3 grid, hipStream_t st) {
  if (p.waves == 8)
    hipLaunchKernelGGL((k_attention<D, G, 8, F8>), grid, dim3(512), 0, st, p);
  else
    hipLaunchKernelGGL((k_attention<D, G, 4, F8>), grid, dim3(256), 0, st, p);
  return hipGetLastError();
}
template <int D, int G>
hipError_t launch_dg(const AttnParams& p, dim3 grid, hipStream_t st) {
  return p.kv_fp8 ? launch_dgf<D, G, true>(p, grid, st) : launch_dgf<D, G, false>(p, grid, st);
}

}  // namespace

int64_t attention_capacity(int D, int G, int waves, bool fp8) {
  // cached per device and (D, G, waves, KV format)
  static std::atomic<int64_t> cache[64][2][4][2][2];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  const int di = D == 128 ? 1 : 0;
  const int gi = G == 1 ? 0 : G == 2 ? 1 : G == 4 ? 2 : 3;
  const int wi = waves == 8 ? 1 : 0;
  const int fi = fp8 ? 1 : 0;
  int64_t c = cache[dev][di][gi][wi][fi].load(std::memory_order_relaxed);
  if (c > 0) return c;
  int64_t per_cu = 0;
  if (D == 128) {
    switch (G) {
      case 1: per_cu = capacity_dg<128, 1>(waves, fp8); break;
      case 2: per_cu = capacity_dg<128, 2>(waves, fp8); break;
      case 4: per_cu = capacity_dg<128, 4>(waves, fp8); break;
      case 8: per_cu = capacity_dg<128, 8>(waves, fp8); break;
    }
  } else {
    switch (G) {
      case 1: per_cu = capacity_dg<64, 1>(waves, fp8); break;
      case 2: per_cu = capacity_dg<64, 2>(waves, fp8); break;
      case 4: per_cu = capacity_dg<64, 4>(waves, fp8); break;
      case 8: per_cu = capacity_dg<64, 8>(waves, fp8); break;
    }
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  c = per_cu * cus;
  cache[dev][di][gi][wi][fi].store(c, std::memory_order_relaxed);
  return c;
}

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
