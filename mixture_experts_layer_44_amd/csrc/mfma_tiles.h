// Device helpers shared by the grouped-GEMM translation units (forward and backward): LDS
// address type, the vmcnt wait immediate, the XCD-aware tile walk over a Schedule, SiLU and
// the LDS swizzle of [rows][BK] stages. Internal; not part of the C ABI.
#pragma once

#include "moe_internal.h"

namespace moe {
namespace {

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// s_waitcnt immediate that waits until at most n vector-memory ops are outstanding
// (expcnt and lgkmcnt left unconstrained)
constexpr int wait_vm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0F70; }

struct TileCoord {
  int g, m_local, n0, mt_global, rows, off;
  int mtg;   // m-tiles of group g
};

// Tile for this workgroup, or false if it has none. Uniform across the workgroup.
// Workgroups are dealt round-robin to the 8 XCDs (xcd = b % 8). By default each XCD walks one
// contiguous range of the tile list. With sc.xcd_chunk, the list is dealt to the XCDs in chunks
// of kXcdChunk consecutive tiles instead, so that the tiles of the few segments at a capacity
// limit (L2-bound: their m-tiles share each weight tile) spread over every XCD's L2 rather than
// landing on the first few XCDs; a chunk keeps an n-tile's m-tiles together. The grid then has
// whole multiples of 8 * kXcdChunk workgroups (grid_for). The chunks are taken alternately
// from the front and the back of the tile list, so tiles of the heavily loaded segments and of
// the lightly loaded ones (weight-streaming, HBM-bound) run side by side rather than one after
// the other (skewed layer with a capacity limit: 0.87 -> 0.86 ms).
template <bool IDENT = false>
__device__ __forceinline__ bool tile_coord(const Schedule& sc, int NT, int bn, TileCoord& tc,
                                           int S = 1, int* half = nullptr) {
  const int bid = blockIdx.x;
  int L, g, ms, mtg, rows, off;
  auto from_info = [&](int m) {
    const int4 i0 = ((const int4*)sc.mt_info)[2 * m];
    const int4 i1 = ((const int4*)sc.mt_info)[2 * m + 1];
    g = i0.x;
    ms = i0.y;
    mtg = i0.z;
    rows = i0.w;
    off = i1.x;
  };
  if (IDENT && sc.mt_info) {
    // identity walk (S == 1): workgroup b runs tile b. Its m-tile slot and the m-tile count
    // are loaded together, so the tile is known after one round trip.
    L = bid;
    const int m = L / NT;
    if (m >= sc.max_mtiles) return false;
    const int mt_total = sc.mt_start[sc.G];
    from_info(m);
    if (m >= mt_total) return false;
  } else {
    const int total = sc.mt_start[sc.G] * NT;
    const int xcd = bid & 7, slot = bid >> 3;
    if (sc.xcd_chunk) {
      const int per = (total * S + 8 * kXcdChunk - 1) / (8 * kXcdChunk) * kXcdChunk;
      if (slot >= per) return false;
      int q = (slot / kXcdChunk) * 8 + xcd;
      const int Q = (total * S + kXcdChunk - 1) / kXcdChunk;
      if (q < Q) q = (q & 1) ? Q - 1 - (q >> 1) : (q >> 1);
      L = q * kXcdChunk + slot % kXcdChunk;
    } else {
      const int per = (total * S + 7) >> 3;
      if (slot >= per) return false;
      L = xcd * per + slot;
    }
    if (L >= total * S) return false;
    if (half) *half = L / total;   // work unit L = half * total + tile
    L %= total;
    if (sc.mt_info) {
      from_info(L / NT);
    } else {
      g = sc.mt_group[L / NT];
      ms = sc.mt_start[g];
      mtg = sc.mt_start[g + 1] - ms;
      rows = sc.grp_rows[g];
      off = sc.grp_off[g];
    }
  }
  const int lp = L - ms * NT;
  // Inside a group the tiles run n-tile by n-tile, its m-tiles together, so those share each
  // weight tile in L2. A group of many m-tiles (the shared expert: every token) walks them in
  // blocks of kMBlock m-tiles instead, n-tile by n-tile inside a block: a window of concurrent
  // tiles then also shares its gathered rows (A) over several n-tiles rather than streaming all
  // of the group's rows once per n-tile.
  constexpr int kMBlock = 4;
  int n_tile, m_local;
  if (mtg >= 2 * kMBlock) {
    const int b = lp / (kMBlock * NT);
    const int rem = lp - b * kMBlock * NT;
    const int sz = min(kMBlock, mtg - b * kMBlock);
    n_tile = rem / sz;
    m_local = b * kMBlock + rem - n_tile * sz;
  } else {
    n_tile = lp / mtg;
    m_local = lp - n_tile * mtg;
  }
  tc.g = g;
  tc.mtg = mtg;
  tc.m_local = m_local;
  tc.n0 = n_tile * bn;
  tc.mt_global = ms + tc.m_local;
  tc.rows = rows;
  tc.off = off;
  return true;
}

// SiLU(u) = u * sigmoid(u) with the hardware exp and reciprocal (a few ulp; the result is
// rounded to bf16 right after). exp(-u) overflows to inf for u < -88: u * rcp(inf) = -0.
__device__ __forceinline__ float silu_f(float u) {
  return u * __builtin_amdgcn_rcpf(1.0f + __expf(-u));
}

// Element offset of (row, 16-byte chunk) in a swizzled [rows][BK] bf16 stage. A 256-byte
// LDS cycle spans W = 128/BK rows; chunk c of row r goes to slot c ^ ((r / W) % (BK/8)), so
// 16 consecutive rows read at one logical chunk hit 16 distinct 16-byte bank groups.
template <int BK>
__device__ __forceinline__ int swz(int r, int c) {
  constexpr int CH = BK / 8, W = 128 / BK;
  return r * BK + ((c ^ ((r / W) & (CH - 1))) << 3);
}

}  // namespace
}  // namespace moe
