// Pieces shared by the 256 x 256 tile kernels (bf16 and E4M3 inputs): the LDS operand layout
// of a 128-byte K step per row, and the tile-to-workgroup mapping.
#pragma once

#include "common.h"

namespace fusedops {
namespace t256 {

// 16-byte chunk `chunk` of LDS row `row` sits at chunk position chunk ^ f(row) with
// f(row) = (row & 7) ^ ((row >> 3) & 1): any 8 consecutive rows at one logical chunk use 8
// distinct positions (128-byte bank window) and any 16 consecutive rows use 16 distinct
// (position, row parity) pairs (256-byte bank window), for reads and fills alike.
__device__ __forceinline__ int swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }
__device__ __forceinline__ uint32_t lds_off(int row, int chunk) {
  return (uint32_t)(row * 128 + ((chunk ^ swz(row)) << 4));
}

// Map a linear tile id to (token tile, feature tile). Consecutive workgroups are
// dealt round-robin to the 8 XCDs; regroup so that each XCD walks a contiguous
// range of tile ids, and within that range cover GROUP_T token tiles x all
// feature tiles so concurrently running tiles share operand rows in the XCD's L2.
__device__ __forceinline__ void tile_coords(int pid, int tiles_t, int tiles_f, int& tt, int& ft) {
  const int G = tiles_t * tiles_f;
  const int xcd = pid & 7, local = pid >> 3;
  const int base = G >> 3, rem = G & 7;
  const int p2 = xcd * base + min(xcd, rem) + local;
  constexpr int GROUP_T = 4;
  const int group_size = GROUP_T * tiles_f;
  const int g = p2 / group_size;
  const int first_t = g * GROUP_T;
  const int gt = min(tiles_t - first_t, GROUP_T);
  const int in = p2 - g * group_size;
  tt = first_t + in % gt;
  ft = in / gt;
}

}  // namespace t256
}  // namespace fusedops
