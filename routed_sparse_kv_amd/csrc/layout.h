// HBM layouts of the cache, chosen so that each MFMA operand a wave needs is
// one contiguous 16-byte (or 8-byte) load per lane.
//
// MFMA lane conventions on gfx950 (16x16 output tile, wave64, lane l):
//   A operand: row i = l % 16, K elements from lane group g = l / 16;
//   B operand: column j = l % 16, the same K elements from lane group g;
//   D (4 fp32 per lane): column j = l % 16, rows 4 g + 0..3.
// A and B pair element e of lane group g with each other, so any fixed map
// (g, e) -> k works as long as both operands use it.
//
// Offsets below are in elements, relative to the start of one (sequence,
// KV head) unit, and are shared by the kernels and the host-side export /
// import, which convert to and from the row-major canonical layout.
#pragma once

#include <stddef.h>

#ifndef RSKV_HD
#define RSKV_HD __host__ __device__ __forceinline__
#endif

namespace rskv {

// Full-resolution keys, "K16" tiles: 16 rows x 32 columns per (tile, kk)
// block of 512 elements; lane l holds row 16 t + l % 16, columns
// 32 kk + 8 (l / 16) + 0..7 (A operand of the 16x16x32 QK product).
RSKV_HD size_t k16_off(int r, int c, int d) {
  const int lane = (((c & 31) >> 3) << 4) | (r & 15);
  return (static_cast<size_t>(r >> 4) * (d >> 5) + (c >> 5)) * 512 + lane * 8 + (c & 7);
}

// Row of a 32-row "V32" tile held by element e of lane group g: the first
// four elements come from the rows the 16x16 QK product of rows 0..15 leaves
// in lane group g, the last four from rows 16..31.
RSKV_HD int v32_row(int g, int e) { return e < 4 ? 4 * g + e : 16 + 4 * g + (e - 4); }

// Values (full-resolution rows, or span means), "V32" tiles: per 32-row
// tile and 16-column block, lane l = 16 g + (c % 16) holds column c of the
// rows v32_row(g, 0..7) (A operand of the transposed 16x16x32 PV product).
RSKV_HD size_t v32_off(int r, int c, int d) {
  const int rr = r & 31;
  const int g = rr < 16 ? (rr >> 2) : ((rr - 16) >> 2);
  const int e = rr < 16 ? (rr & 3) : 4 + ((rr - 16) & 3);
  const int lane = (g << 4) | (c & 15);
  return (static_cast<size_t>(r >> 5) * (d >> 4) + (c >> 4)) * 512 + lane * 8 + e;
}

// Summary logits, fp32: per 16-span tile, per query head, 16 spans.
RSKV_HD size_t slogit_off(int j, int g, int G) {
  return (static_cast<size_t>(j >> 4) * G + g) * 16 + (j & 15);
}

// A_K: row-major [rows][r], span j starting at its padded offset (spans are
// padded to a multiple of 16 rows).  A_V is stored transposed per 16-row
// tile: [tile][k][16], so lane (k = l % 16, group g) reads rows 4 g..4 g+3.
RSKV_HD size_t avt_off(int t, int k, int r) {
  return (static_cast<size_t>(t >> 4) * r + k) * 16 + (t & 15);
}

// W_K is row-major [span][r][d] (row k = k-th right singular vector).
//
// W_V feeds the transposed PV product out^T += W_V^T w, whose A operand for
// the 16-column block cb is lane (c = l % 16, group g) -> W_V[4 g..4 g+3][c].
// Blocks are stored in pairs so that one 16-byte load per lane serves two
// of them: per span, per 32-column pair, lane (c, g) finds the four ranks
// of column c of the first block followed by those of the second.  Ranks
// are padded to a multiple of 4 (rank4), with zeros.
RSKV_HD int rank4(int r) { return (r + 3) & ~3; }
RSKV_HD size_t wvt_off(int j, int k, int c, int d, int r) {
  const int r4 = rank4(r);
  return static_cast<size_t>(j) * d * r4 + static_cast<size_t>(c >> 5) * 32 * r4 +
         static_cast<size_t>((c & 15) * (r4 >> 2) + (k >> 2)) * 8 + ((c >> 4) & 1) * 4 + (k & 3);
}

RSKV_HD int round_up(int x, int m) { return (x + m - 1) / m * m; }

}  // namespace rskv
