// qgemv_layout.h -- the gfx950 blob written by qgemv_repack and read by the kernels.
//
// Blob = header | codes | meta | row_ptr | entries, every section 256-byte aligned.
//
// codes   M rows of K*bits/8 bytes.  A row is the canonical sequence of 32-code
//         chunks (chunk c holds canonical codes 32c..32c+31 and occupies the same
//         4*bits bytes as in the canonical bitstream); only the bit placement
//         inside a chunk changes, so that each kernel lane turns one dword into
//         dot-product-ready FP16 pairs with a handful of bitwise ops.  Lane l of
//         wave step s owns chunk 64*s + l.
//
//         Inside a chunk, pair m (m = 0..15) is canonical codes (2m, 2m+1) and is
//         multiplied with x[32c + 2m], x[32c + 2m + 1].  Slot placement per format:
//
//         U4 (uniform, 4 bit; 4 dwords): dword d, slot t = 0..3 holds pair 4d+t;
//            low code at bits 4t..4t+3, high code at bits 16+4t..16+4t+3.
//         U3 (uniform, 3 bit; 3 dwords): dword d, slot t = 0..4 holds pair 5d+t;
//            slots start at bits 0, 3, 6, 10, 13 (low code) and 16 more (high
//            code).  Pair 15: low code = bit 9 of dwords 0,1,2 (code bits 0,1,2),
//            high code = bit 25 of dwords 0,1,2.
//         L4 (LUT, 4 bit; 4 dwords): byte k of dword d holds A = code 8d+k and
//            B = code 8d+4+k as: bits 0-2 = A&7, bits 3-5 = B&7, bit 6 = A>>3,
//            bit 7 = B>>3.
//         L3 (LUT, 3 bit; 3 dwords): byte k of dword d: bits 0-2 = code 8d+k,
//            bits 3-5 = code 8d+4+k.  Bits 6-7 of the bytes of dword 0 are the
//            low bits of code 24+k, of dword 1 the low bits of code 28+k; bit 6
//            (7) of byte k of dword 2 is bit 2 of code 24+k (28+k).
//
// meta    UNIFORM: per row K/16 dwords, dword g = FP16 scale (low half) | FP16
//         zero (high half) of group g.
//         LUT: per row the table split into byte planes for v_perm:
//           3 bit: 4 dwords = lo bytes e0-3, lo e4-7, hi e0-3, hi e4-7
//           4 bit: 8 dwords = lo e0-3, lo e4-7, lo e8-11, lo e12-15,
//                             hi e0-3, hi e4-7, hi e8-11, hi e12-15
// row_ptr int32 [M+1] (as given).
// entries uint32 [nnz]: column (low 16 bits) | FP16 value bits (high 16 bits).
#pragma once

#include <stdint.h>

namespace qgemv_layout {

constexpr uint32_t kMagic = 0x564d4751u;  // "QGMV"
constexpr uint32_t kVersion = 1;
constexpr int kLanes = 64;
constexpr int kChunkCodes = 32;
constexpr int kStepCodes = kLanes * kChunkCodes;  // 2048 codes per wave step
constexpr int kMaxSteps = 8;                      // K <= 16384
constexpr int kMaxK = kStepCodes * kMaxSteps;
constexpr uint64_t kAlign = 256;
constexpr uint64_t kHeaderBytes = 256;

struct BlobHeader {
  uint32_t magic;
  uint32_t version;
  int32_t M, K, bits, format, group_size, steps;
  int64_t nnz;
  uint64_t off_codes, off_meta, off_rowptr, off_entries, total_bytes;
  uint32_t row_bytes;       // K * bits / 8
  uint32_t meta_row_bytes;  // UNIFORM: 4 * K / 16; LUT: 2 << bits
};
static_assert(sizeof(BlobHeader) <= kHeaderBytes, "header too large");

inline uint64_t align_up(uint64_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// Section offsets of a blob for the given shape.
inline BlobHeader make_header(int32_t M, int32_t K, int32_t bits, int32_t format, int32_t group,
                              int64_t nnz) {
  BlobHeader h{};
  h.magic = kMagic;
  h.version = kVersion;
  h.M = M;
  h.K = K;
  h.bits = bits;
  h.format = format;
  h.group_size = format == 0 ? group : 0;
  h.steps = (K + kStepCodes - 1) / kStepCodes;
  h.nnz = nnz;
  h.row_bytes = (uint32_t)((int64_t)K * bits / 8);
  h.meta_row_bytes = format == 0 ? (uint32_t)(4 * (K / group)) : (uint32_t)(2u << bits);
  h.off_codes = kHeaderBytes;
  h.off_meta = align_up(h.off_codes + (uint64_t)M * h.row_bytes);
  h.off_rowptr = align_up(h.off_meta + (uint64_t)M * h.meta_row_bytes);
  h.off_entries = align_up(h.off_rowptr + 4ull * ((uint64_t)M + 1));
  h.total_bytes = align_up(h.off_entries + 4ull * (uint64_t)nnz);
  return h;
}

}  // namespace qgemv_layout
