// Tiles of 64 gathered K/V rows for matrix-core attention kernels: 4 waves, 16 query
// rows per wave, v_mfma_f32_16x16x32_bf16 for both products. K rows are staged
// row-major in LDS (in the order tile_krow gives) for the q.k product, V transposed for
// the P.V product, so that a lane's scores of the q.k product are already its operand
// of the P.V product. Rows are gathered by positions staged in LDS (kidx).
#pragma once

#include "ld_device.h"

namespace ld {
namespace {

constexpr int kTileWaves = 4;
constexpr int kTileQ = 16 * kTileWaves;   // queries per workgroup
constexpr int kTileKeys = 64;            // keys per tile
constexpr int kTileIdx = 1024;           // selected positions staged in LDS at a time
constexpr float kTileLog2e = 1.4426950408889634f;

typedef __bf16 tile_bf16x8_t __attribute__((ext_vector_type(8)));
typedef float tile_f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ tile_f32x4_t mfma16(const uint4& a, const uint4& b, tile_f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(tile_bf16x8_t, a),
                                                 __builtin_bit_cast(tile_bf16x8_t, b), c, 0, 0, 0);
}

template <int D>
struct TileSmem {
  static constexpr int KS = D + 8;          // K tile row stride (elements)
  static constexpr int VS = kTileKeys + 8;   // transposed V tile row stride
  // (16-byte aligned so that operand reads are single 16-byte LDS reads)
  alignas(16) uint16_t kt[2][kTileKeys * KS];   // two tiles: one computed, one being filled
  alignas(16) uint16_t vt[2][D * VS + (D / 8) * 32];   // rows at vrow(dim)
  // Row of dimension `dim` in vt: each group of 8 dimensions starts 32 elements (16
  // banks) after the previous group's end, so that consecutive groups fall in opposite
  // bank halves and the transposed stores and the operand reads are conflict-free.
  static __device__ __forceinline__ int vrow(int dim) { return dim * VS + (dim >> 3) * 32; }
  int qpos[kTileQ];
  int kidx[kTileIdx];                        // selected positions of the current key chunk
};

// bf16 bits of x, rounded to nearest even by the hardware conversion (the softmax
// weights are finite and in [0, 1]).
__device__ __forceinline__ uint16_t tile_bf16(float x) { return __builtin_bit_cast(uint16_t, (__bf16)x); }

// Tile t of the key chunk: K as LPT 16-byte pieces of rows per thread (row-major,
// coalesced); V as pairs of rows (2p, 2p + 1) at one 16-byte column piece, so that
// the transposed store writes whole words (two keys of one dimension). Rows past the
// chunk's nk keys repeat its last key; they are masked.
template <int D, int NW = kTileWaves>
struct TileRegs {   // per thread of a workgroup of NW waves
  static constexpr int LPT = kTileKeys * (D / 8) / (NW * 64);        // K pieces per thread
  static constexpr int VITEMS = (kTileKeys / 2) * (D / 8);                   // V row pairs x pieces
  static constexpr int LPV = (VITEMS + NW * 64 - 1) / (NW * 64);
  uint4 k[LPT];
  uint4 v[LPV][2];
};

template <int D, int NW = kTileWaves>
__device__ __forceinline__ void tile_load(const uint16_t* Kg, const uint16_t* Vg, const int* kidx, int nk, int t,
                                         int tid, TileRegs<D, NW>& R) {
  using RG = TileRegs<D, NW>;
  const int base = t * kTileKeys;
#pragma unroll
  for (int i = 0; i < RG::LPT; ++i) {
    const int u = tid + i * NW * 64;
    const int r = u / (D / 8), c = u % (D / 8);
    const size_t pos = (size_t)kidx[min(base + r, nk - 1)];
    R.k[i] = *reinterpret_cast<const uint4*>(Kg + pos * D + c * 8);
  }
#pragma unroll
  for (int i = 0; i < RG::LPV; ++i) {
    const int u = tid + i * NW * 64;
    if (u < RG::VITEMS) {
      const int rp = u % (kTileKeys / 2), c = u / (kTileKeys / 2);
      const size_t p0 = (size_t)kidx[min(base + 2 * rp, nk - 1)];
      const size_t p1 = (size_t)kidx[min(base + 2 * rp + 1, nk - 1)];
      R.v[i][0] = *reinterpret_cast<const uint4*>(Vg + p0 * D + c * 8);
      R.v[i][1] = *reinterpret_cast<const uint4*>(Vg + p1 * D + c * 8);
    }
  }
}

// LDS row of key r of a tile: within each 32-key half, key 8a + 4q + b goes to row
// 16q + 4a + b, so that the q.k product's quarter q (LDS rows 16q .. 16q + 15, read as
// 16 consecutive rows) leaves lane group a holding keys 8a + 4q .. + 3, and the two
// quarters of a half together give each lane group 8 consecutive keys for P.V.
__device__ __forceinline__ int tile_krow(int r) {
  return (r & ~31) | (((r >> 2) & 1) << 4) | (((r >> 3) & 3) << 2) | (r & 3);
}

// The loaded pieces to LDS buffer `buf`: K rows permuted by tile_krow, V transposed (word j of a pair
// holds dimension c * 8 + j of keys 2p and 2p + 1).
template <int D, int NW = kTileWaves>
__device__ __forceinline__ void tile_store(TileSmem<D>& sm, int buf, int tid, const TileRegs<D, NW>& R) {
  using RG = TileRegs<D, NW>;
  constexpr int KS = TileSmem<D>::KS, VS = TileSmem<D>::VS;
#pragma unroll
  for (int i = 0; i < RG::LPT; ++i) {
    const int u = tid + i * NW * 64;
    const int r = u / (D / 8), c = u % (D / 8);
    *reinterpret_cast<uint4*>(&sm.kt[buf][tile_krow(r) * KS + c * 8]) =
        make_uint4(R.k[i].x, R.k[i].y, R.k[i].z, R.k[i].w);
  }
#pragma unroll
  for (int i = 0; i < RG::LPV; ++i) {
    const int u = tid + i * NW * 64;
    if (u < RG::VITEMS) {
      const int rp = u % (kTileKeys / 2), c = u / (kTileKeys / 2);
      const uint32_t a[4] = {R.v[i][0].x, R.v[i][0].y, R.v[i][0].z, R.v[i][0].w};
      const uint32_t b[4] = {R.v[i][1].x, R.v[i][1].y, R.v[i][1].z, R.v[i][1].w};
      uint32_t* col = reinterpret_cast<uint32_t*>(&sm.vt[buf][TileSmem<D>::vrow(c * 8) + 2 * rp]);
#pragma unroll
      for (int w = 0; w < 4; ++w) {   // dims c*8 .. c*8+7 share one bank half
        col[(2 * w) * (VS / 2)] = (a[w] & 0xffffu) | (b[w] << 16);
        col[(2 * w + 1) * (VS / 2)] = (a[w] >> 16) | (b[w] & 0xffff0000u);
      }
    }
  }
}

}  // namespace
}  // namespace ld
