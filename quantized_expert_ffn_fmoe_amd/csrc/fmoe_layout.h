// fmoe_layout.h -- where the packed code bytes of a quantized matrix sit.
//
// A rows x row_bytes code matrix (row_bytes = cols * bits / 8) is stored in blocks of 32
// consecutive rows. Within a block every row is cut into pieces of 4 groups of 64 columns
// (128 bytes at 4 bits, 64 at 2 bits), and piece p of all the block's rows is stored
// together, in row order: block base + p * rows_in_block * piece bytes + (row in block) *
// piece size. A block is therefore a sequence of 4-KB (2-KB) runs, each holding the same
// 4 groups of its 32 rows. Inside its piece a row's 16-byte chunks are rotated: chunk k
// sits at position (k + rot(r)) mod (chunks in the piece), rot(r) = r mod 8 at 4 bits and
// (r mod 16) / 4 at 2 bits. A row whose length is not a whole number of pieces ends in one
// shorter piece (stored the same way with its own size), and a final block of fewer rows
// uses its own row count, so the matrix occupies exactly rows * row_bytes bytes.
//
// Why: the multi-token kernels give each wave 32 rows of a matrix and stream them 4 groups
// per step through LDS-DMA, one 16-byte-per-lane instruction per 8 (16) rows. In this
// layout such an instruction reads one contiguous KB in lane order (the address unit
// handles a quad of lanes on one cache line at a time, so lane-ordered runs are the cheap
// case), the steps walk the block front to back, and the rotation makes the matrix-core
// fragment reads of the staged rows conflict-free in LDS. The single-token kernels keep
// each lane on fixed 16-byte chunks of a row: a row's piece is still one 128-byte line
// (64 bytes at 2 bits), so a row load touches as many lines as with row-major codes.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace fmoe {

template <int BITS>
struct CodeLayout {
  static_assert(BITS == 4 || BITS == 2, "4-bit or 2-bit codes (a 3-bit matrix's low plane is laid out as 2-bit)");
  static constexpr int kBlockRows = 32;  // measured against 16, 64 and 256 rows: best for the batched kernels
  static constexpr int kPieceBytes = BITS * 32;  // 4 groups of 64 columns
  static constexpr int kSubRows = 1024 / kPieceBytes;  // rows of one contiguous KB
  __host__ __device__ static constexpr int rot(int r) { return BITS == 4 ? r % 8 : (r % 16) / 4; }
};

// Byte offset of byte b of row r (b a multiple of 16 keeps a 16-byte chunk whole: pieces
// are multiples of 16 bytes for every accepted shape).
template <int BITS>
__host__ __device__ __forceinline__ size_t code_offset(int rows, size_t row_bytes, int r, size_t b) {
  using CL = CodeLayout<BITS>;
  constexpr int RB = CL::kBlockRows, P = CL::kPieceBytes;
  const int r0 = r / RB * RB;
  const int nr = rows - r0 < RB ? rows - r0 : RB;  // rows of this block
  const size_t p = b / P;
  const size_t left = row_bytes - p * P;
  const int piece = left < (size_t)P ? (int)left : P;
  const int pos = ((int)(b % P) / 16 + CL::rot(r)) % (piece / 16);
  return (size_t)r0 * row_bytes + p * (size_t)nr * P + (size_t)(r - r0) * piece + pos * 16 + b % 16;
}

// Scale/bias words (one uint32 per (row, group)) are blocked the same way: blocks of 32
// rows, each row's words cut into pieces of 4 groups (16 bytes), piece p of the block's
// rows stored together in row order (a short last piece and a short last block keep their
// own sizes). A 4-group stage's words for 32 rows are then one contiguous 512 bytes, and
// the words of one (row, piece) stay one 16-byte load. Word offset of group g of row r:
__host__ __device__ __forceinline__ size_t sb_offset(int rows, int groups, int r, int g) {
  constexpr int RB = 32, PG = 4;
  const int r0 = r / RB * RB;
  const int nr = rows - r0 < RB ? rows - r0 : RB;
  const int p = g / PG;
  const int pg = groups - p * PG < PG ? groups - p * PG : PG;  // groups of this piece
  return (size_t)r0 * groups + (size_t)p * nr * PG + (size_t)(r - r0) * pg + g % PG;
}

// 3-bit codes are stored as two planes. The low plane holds the low 2 bits of every code
// laid out exactly as a 2-bit matrix of the same shape (code_offset<2> with row bytes
// cols / 4), so every 2-bit reader takes it as it is. The high plane follows it and holds
// the third bit of every code, one uint32 per 32 columns (two per group), blocked like the
// scale/bias words with two words per group: blocks of 32 rows, each row's words cut into
// pieces of 4 groups (32 bytes), piece p of the block's rows stored together in row order.
// A 4-group stage of 32 rows is one contiguous KB, and the two words of one (row, group)
// are one 8-byte load. Word offset of word h (0, 1) of group g of row r:
__host__ __device__ __forceinline__ size_t hi_offset(int rows, int groups, int r, int g, int h) {
  constexpr int RB = 32, PG = 4;
  const int r0 = r / RB * RB;
  const int nr = rows - r0 < RB ? rows - r0 : RB;
  const int p = g / PG;
  const int pg = groups - p * PG < PG ? groups - p * PG : PG;
  return (size_t)r0 * groups * 2 + (size_t)p * nr * PG * 2 + (size_t)(r - r0) * pg * 2 + (size_t)(g % PG) * 2 + h;
}
// Bit of column c (0..31 of a high-plane word's 32 columns) in that word. The columns of a
// 16-column code dword t = c / 16 are split into even and odd ones as the integer dot
// product takes them (operand s = 2 t + c % 2, nibble n = (c % 16) / 2), and the bit sits
// at 4 n + s: then (word >> s) & 0x11111111 puts the high bits of operand s in its nibbles,
// and for the matrix-core unpack, whose byte m after a shift by 2 r holds column
// 16 t + 4 m + r, (word >> (2 t)) has that column's bit at 8 m + 4 (r / 2) + r % 2.
__host__ __device__ constexpr int hi_bit(int c) { return 4 * ((c % 16) / 2) + 2 * (c / 16) + (c % 2); }

// Bytes of the low plane of a 3-bit matrix (the high plane starts there).
__host__ __device__ __forceinline__ size_t lo_plane_bytes(int rows, int cols) { return (size_t)rows * cols / 4; }

}  // namespace fmoe
