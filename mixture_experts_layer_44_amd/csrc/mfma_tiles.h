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
};

// Tile for this workgroup, or false if it has none. Uniform across the workgroup.
__device__ __forceinline__ bool tile_coord(const Schedule& sc, int NT, int bn, TileCoord& tc,
                                           int S = 1, int* half = nullptr) {
  const int total = sc.mt_start[sc.G] * NT;
  const int bid = blockIdx.x;
  const int xcd = bid & 7, slot = bid >> 3;
  const int per = (total * S + 7) >> 3;
  if (slot >= per) return false;
  int L = xcd * per + slot;
  if (L >= total * S) return false;
  if (half) *half = L / total;   // work unit L = half * total + tile
  L %= total;
  const int g = sc.mt_group[L / NT];
  const int ms = sc.mt_start[g];
  const int mtg = sc.mt_start[g + 1] - ms;
  const int lp = L - ms * NT;
  const int n_tile = lp / mtg;
  tc.g = g;
  tc.m_local = lp - n_tile * mtg;
  tc.n0 = n_tile * bn;
  tc.mt_global = ms + tc.m_local;
  tc.rows = sc.grp_rows[g];
  tc.off = sc.grp_off[g];
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
