// qgemv_layout.h -- the gfx950 blob written by qgemv_repack and read by the kernels.
//
// Blob = header | codes | meta | row_ptr | entries | boff | bent, every
// section 256-byte aligned.
//
// Tiles.  Rows are grouped in tiles of 16 (the M side of a 16x16x32 MFMA);
// K is padded to Kp, a multiple of 128, and cut into K-blocks of 128 codes
// (four MFMA K-steps of 32).  For tile t and K-block b, the 64 lanes of a
// wave each own one 32-code chunk:
//
//     lane l  ->  row 16*t + (l % 16),  codes 128*b + 32*(l / 16) .. +31
//
// which is exactly the A-operand footprint of four 16x16x32 MFMAs (lane l
// supplies row l % 16 and K-slice 8*(l / 16) .. +7 of each).  The 64 chunks of
// a (tile, K-block) are stored back to back, lane order, so one wave load of
// 4*bits bytes per lane reads 768 B (3 bit) or 1 KiB (4 bit) contiguously.
// Blocks are ordered tile-major: (t, b) at index t * nkb + b.  Padding rows
// (>= M) and padding columns (>= K) hold code 0 and decode against zero
// statistics / zero activations.
//
// Inside a chunk the 32 codes are re-placed so that a lane turns one dword
// into FP16 pairs with a few bitwise ops.  Pair m (m = 0..15) is canonical
// chunk codes (2m, 2m+1); MFMA step i of the K-block takes pairs 4i..4i+3.
//
//   U4 (uniform, 4 bit; 4 dwords): dword d, slot t = 0..3 holds pair 4d+t;
//      low code at bits 4t..4t+3, high code at bits 16+4t..16+4t+3.
//   U3 (uniform, 3 bit; 3 dwords): dword d, slot t = 0..4 holds pair 5d+t;
//      slots start at bits 0, 3, 6, 10, 13 (low code) and 16 more (high code).
//      Pair 15: low code = bit 9 of dwords 0,1,2 (code bits 0,1,2), high code =
//      bit 25 of dwords 0,1,2.
//   L4 (LUT, 4 bit; 4 dwords): byte k of dword d holds A = code 8d+k and
//      B = code 8d+4+k as: bits 0-2 = A&7, bits 3-5 = B&7, bit 6 = A>>3,
//      bit 7 = B>>3.
//   L3 (LUT, 3 bit; 3 dwords): byte k of dword d: bits 0-2 = code 8d+k,
//      bits 3-5 = code 8d+4+k.  Bits 6-7 of the bytes of dword 0 are the low
//      bits of code 24+k, of dword 1 the low bits of code 28+k; bit 6 (7) of
//      byte k of dword 2 is bit 2 of code 24+k (28+k).
//
//   BPDQ codes (3 bit) use the L3 placement.
//
//   HPTQ codes (prefix codewords, 32 per lane chunk): for each (tile,
//   K-block) the 64 chunks' codewords in lane order, as one bit sequence
//   stored in 32-bit words most significant bit first (bit p is bit 31 -
//   p % 32 of word p / 32), starting on a 16-byte boundary; hidx holds each
//   block's first word (and the end), hlane each lane's bit offset inside its
//   block.  Chunks of padding rows are empty.
//
// meta    LUT: per row (tiles*16 rows) the canonical FP16 table, 2^bits entries.
//         BPDQ: per (tile, K-block) the FP16 coefficients [16 rows][128/group
//         groups][bits + 1] (C0 first); a lane's chunk lies in one group, whose
//         coefficients are one 8-byte piece.
//         HPTQ: per (tile, K-block) the 16 rows' FP16 steps (group 128 = the
//         K-block).
// hidx    HPTQ: uint32 [tiles*nkb + 1]; hlane: uint16 [tiles*nkb*64];
//         the header's hmaxw is the largest block's word count.
// htab    HPTQ: int32 [256]: for the next 8 bits of a chunk, the FP16 bits
//         of the integer of the codeword they start with (bits 16-31) and its
//         length (bits 0-7) if the length is at most 8; if they start a
//         longer codeword, 256 times the index of their second-level table
//         (bits 16-31) and length 0; else 0.  Then int32 [4][17]: per length
//         l the first canonical codeword, the number of codewords, the index
//         of the first in hsym, and the end of the codewords of length l
//         left-justified to 16 bits (the first codeword of length l + 1 would
//         start there; equal to the previous length's for a length with no
//         codewords, 0 before the first).  Then int32 [hsub][256]: for each
//         8-bit prefix of a longer codeword (in prefix order), indexed by
//         the next 8 bits, FP16 bits of the integer << 16 | length (9-16),
//         or 16 where no codeword starts; at least one table (with no longer
//         codeword, one of length-16 entries).
// hsym    HPTQ: int16 [hsym]: the codewords' integers in canonical order.
//         UNIFORM: 512 bytes per (tile, K-block) for its 16 rows x 8 groups of
//         16 codes: a z plane, FP16 zero points [row][group] (256 B), then an
//         s plane, FP16 scales [group / 2][row][group % 2] (256 B).  Lane l's
//         two groups (2*(l/16), 2*(l/16)+1) of row l % 16 are one dword in each
//         plane; the scales of one group for four consecutive rows are one
//         16-byte piece of the s plane.
// row_ptr int32 [M+1] (as given).
// entries uint32 [nnz]: column (low 16 bits) | FP16 value bits (high 16 bits).
// boff    int32 [tiles * nkb + 1]: the outliers of (tile, K-block) index i =
//         t * nkb + b are bent[boff[i] .. boff[i+1]).
// bent    uint32 [nnz]: the same outliers grouped by (tile, K-block), rows
//         and then columns ascending inside a group: column inside the
//         K-block (bits 0-6) | row inside the tile (bits 7-10) | FP16 value
//         bits (16-31).
#pragma once

#include <stdint.h>

namespace qgemv_layout {

constexpr uint32_t kMagic = 0x564d4751u;  // "QGMV"
constexpr uint32_t kVersion = 9;
constexpr int kTileRows = 16;
constexpr int kBlockK = 128;
constexpr int kChunkCodes = 32;
constexpr int kMaxK = 16384;
constexpr uint64_t kAlign = 256;
constexpr uint64_t kHeaderBytes = 256;
constexpr int kHuffBits = 8;                // HPTQ first-level table index: the next 8 bits
constexpr int kHuffTable = 1 << kHuffBits;
constexpr int kHuffMaxLen = 16;
constexpr int kHuffSub = 1 << (kHuffMaxLen - kHuffBits);  // entries of a second-level table
constexpr int kHuffMaxSym = 4096;

struct BlobHeader {
  uint32_t magic;
  uint32_t version;
  int32_t M, K, bits, format, group_size, tiles;
  int64_t nnz;
  uint64_t off_codes, off_meta, off_rowptr, off_entries, total_bytes;
  uint32_t block_bytes;      // 64 * 4 * bits: codes of one (tile, K-block)
  uint32_t meta_unit_bytes;  // LUT: bytes per row; UNIFORM: bytes per (tile, K-block)
  int32_t Kp;                // K padded to a multiple of kBlockK
  int32_t nkb;               // Kp / kBlockK
  uint64_t off_boff, off_bent;  // outliers grouped by (tile, K-block)
  // HPTQ only (0 otherwise): block word offsets, lane bit offsets, decode
  // tables, codeword integers; number of codewords and of code words.
  uint64_t off_hidx, off_hlane, off_htab, off_hsym;
  int32_t hsym;
  uint32_t hwords, hmaxw, hsub;
};
static_assert(sizeof(BlobHeader) <= kHeaderBytes, "header too large");

inline uint64_t align_up(uint64_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// Section offsets of a blob for the given shape.
inline BlobHeader make_header(int32_t M, int32_t K, int32_t bits, int32_t format, int32_t group,
                              int64_t nnz, int32_t hsym = 0, uint32_t hwords = 0, uint32_t hmaxw = 0,
                              uint32_t hsub = 0) {
  const bool hptq = format == 3;
  if (hptq) bits = 0;
  BlobHeader h{};
  h.magic = kMagic;
  h.version = kVersion;
  h.M = M;
  h.K = K;
  h.bits = bits;
  h.format = format;
  h.group_size = format == 1 ? 0 : group;
  h.tiles = (M + kTileRows - 1) / kTileRows;
  h.nnz = nnz;
  h.Kp = (K + kBlockK - 1) / kBlockK * kBlockK;
  h.nkb = h.Kp / kBlockK;
  h.block_bytes = (uint32_t)(64 * 4 * bits);
  h.meta_unit_bytes = format == 0   ? 64u * 8u
                      : format == 1 ? (uint32_t)(2u << bits)
                      : hptq        ? (uint32_t)(kTileRows * 2)
                                    : (uint32_t)(kTileRows * (kBlockK / (group > 0 ? group : kBlockK)) * (bits + 1) * 2);
  const uint64_t nblocks = (uint64_t)h.tiles * h.nkb;
  const uint64_t meta_bytes =
      format == 1 ? (uint64_t)h.tiles * kTileRows * h.meta_unit_bytes : nblocks * h.meta_unit_bytes;
  h.off_codes = kHeaderBytes;
  h.hsym = hptq ? hsym : 0;
  h.hwords = hptq ? hwords : 0;
  h.hmaxw = hptq ? hmaxw : 0;
  h.hsub = hptq ? hsub : 0;
  h.off_meta = align_up(h.off_codes + (hptq ? 4ull * hwords : nblocks * h.block_bytes));
  h.off_rowptr = align_up(h.off_meta + meta_bytes);
  h.off_entries = align_up(h.off_rowptr + 4ull * ((uint64_t)M + 1));
  h.off_boff = align_up(h.off_entries + 4ull * (uint64_t)nnz);
  h.off_bent = align_up(h.off_boff + 4ull * (nblocks + 1));
  h.total_bytes = align_up(h.off_bent + 4ull * (uint64_t)nnz);
  if (hptq) {
    h.off_hidx = h.total_bytes;
    h.off_hlane = align_up(h.off_hidx + 4ull * (nblocks + 1));
    h.off_htab = align_up(h.off_hlane + 2ull * 64ull * nblocks);
    h.off_hsym = align_up(h.off_htab + 4ull * (kHuffTable + 4 * 17 + (uint64_t)kHuffSub * hsub));
    h.total_bytes = align_up(h.off_hsym + 2ull * (uint64_t)hsym);
  }
  return h;
}

}  // namespace qgemv_layout
