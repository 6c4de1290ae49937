// qgemv_host.cpp -- host side of the C ABI: validation, the offline repacker,
// its host inverse, and status strings.  No GPU is touched here.

#include <algorithm>
#include <cmath>
#include <cstring>
#include <vector>

#include "../../include/qgemv.h"
#include "qgemv_internal.h"
#include "qgemv_layout.h"

using namespace qgemv_layout;

namespace {

thread_local int g_last_hip_error = 0;

// IEEE binary16 bits of an integer of magnitude at most 2048 (exact).
uint16_t int_to_half(int v) {
  const uint32_t sign = v < 0 ? 0x8000u : 0u;
  uint32_t m = (uint32_t)(v < 0 ? -v : v);
  if (m == 0) return (uint16_t)sign;
  int e = 0;
  while ((m >> (e + 1)) != 0) ++e;  // m = 1.f * 2^e
  const uint32_t man = e <= 10 ? (m << (10 - e)) & 1023u : (m >> (e - 10)) & 1023u;
  return (uint16_t)(sign | ((uint32_t)(e + 15) << 10) | man);
}

// IEEE binary16 bits -> float.
float half_to_float(uint16_t h) {
  const uint32_t sign = (uint32_t)(h >> 15) << 31;
  const int exp = (h >> 10) & 31;
  const uint32_t man = h & 1023u;
  float v;
  if (exp == 0) {
    v = std::ldexp((float)man, -24);
  } else if (exp == 31) {
    v = man ? NAN : INFINITY;
  } else {
    v = std::ldexp((float)(man | 1024u), exp - 25);
  }
  uint32_t bits;
  std::memcpy(&bits, &v, 4);
  bits |= sign;
  std::memcpy(&v, &bits, 4);
  return v;
}

bool half_finite(uint16_t h) { return ((h >> 10) & 31) != 31; }

// All K codes of one canonical row into out[0..K) (one byte each).
void canon_unpack_row(const uint8_t* row, int K, int bits, uint8_t* out) {
  if (bits == 4) {
    for (int j = 0; j < K; j += 2) {
      out[j] = row[j >> 1] & 15u;
      out[j + 1] = row[j >> 1] >> 4;
    }
    return;
  }
  // 3 bits: every 3 bytes hold 8 codes
  for (int j = 0; j < K; j += 8) {
    const uint8_t* p = row + 3 * (j / 8);
    const uint32_t v = (uint32_t)p[0] | ((uint32_t)p[1] << 8) | ((uint32_t)p[2] << 16);
    for (int q = 0; q < 8; ++q) out[j + q] = (uint8_t)((v >> (3 * q)) & 7u);
  }
}

// ---- chunk placement: 32 canonical codes <-> the kernel's dwords ----------

void place_u4(const uint32_t* c, uint32_t* w) {
  for (int d = 0; d < 4; ++d) {
    uint32_t v = 0;
    for (int t = 0; t < 4; ++t) {
      const int m = 4 * d + t;
      v |= c[2 * m] << (4 * t);
      v |= c[2 * m + 1] << (16 + 4 * t);
    }
    w[d] = v;
  }
}

void unplace_u4(const uint32_t* w, uint32_t* c) {
  for (int d = 0; d < 4; ++d)
    for (int t = 0; t < 4; ++t) {
      const int m = 4 * d + t;
      c[2 * m] = (w[d] >> (4 * t)) & 15u;
      c[2 * m + 1] = (w[d] >> (16 + 4 * t)) & 15u;
    }
}

constexpr int kU3Shift[5] = {0, 3, 6, 10, 13};

void place_u3(const uint32_t* c, uint32_t* w) {
  for (int d = 0; d < 3; ++d) {
    uint32_t v = 0;
    for (int t = 0; t < 5; ++t) {
      const int m = 5 * d + t;
      v |= c[2 * m] << kU3Shift[t];
      v |= c[2 * m + 1] << (16 + kU3Shift[t]);
    }
    // pair 15: one bit of each of its two codes per dword
    v |= ((c[30] >> d) & 1u) << 9;
    v |= ((c[31] >> d) & 1u) << 25;
    w[d] = v;
  }
}

void unplace_u3(const uint32_t* w, uint32_t* c) {
  for (int d = 0; d < 3; ++d)
    for (int t = 0; t < 5; ++t) {
      const int m = 5 * d + t;
      c[2 * m] = (w[d] >> kU3Shift[t]) & 7u;
      c[2 * m + 1] = (w[d] >> (16 + kU3Shift[t])) & 7u;
    }
  c[30] = c[31] = 0;
  for (int d = 0; d < 3; ++d) {
    c[30] |= ((w[d] >> 9) & 1u) << d;
    c[31] |= ((w[d] >> 25) & 1u) << d;
  }
}

void place_l4(const uint32_t* c, uint32_t* w) {
  for (int d = 0; d < 4; ++d) {
    uint32_t v = 0;
    for (int k = 0; k < 4; ++k) {
      const uint32_t a = c[8 * d + k], b = c[8 * d + 4 + k];
      const uint32_t byte = (a & 7u) | ((b & 7u) << 3) | ((a >> 3) << 6) | ((b >> 3) << 7);
      v |= byte << (8 * k);
    }
    w[d] = v;
  }
}

void unplace_l4(const uint32_t* w, uint32_t* c) {
  for (int d = 0; d < 4; ++d)
    for (int k = 0; k < 4; ++k) {
      const uint32_t byte = (w[d] >> (8 * k)) & 255u;
      c[8 * d + k] = (byte & 7u) | (((byte >> 6) & 1u) << 3);
      c[8 * d + 4 + k] = ((byte >> 3) & 7u) | (((byte >> 7) & 1u) << 3);
    }
}

void place_l3(const uint32_t* c, uint32_t* w) {
  for (int d = 0; d < 3; ++d) {
    uint32_t v = 0;
    for (int k = 0; k < 4; ++k) {
      uint32_t byte = (c[8 * d + k] & 7u) | ((c[8 * d + 4 + k] & 7u) << 3);
      if (d == 0) byte |= (c[24 + k] & 3u) << 6;
      if (d == 1) byte |= (c[28 + k] & 3u) << 6;
      if (d == 2) byte |= ((c[24 + k] >> 2) << 6) | ((c[28 + k] >> 2) << 7);
      v |= byte << (8 * k);
    }
    w[d] = v;
  }
}

void unplace_l3(const uint32_t* w, uint32_t* c) {
  for (int d = 0; d < 3; ++d)
    for (int k = 0; k < 4; ++k) {
      const uint32_t byte = (w[d] >> (8 * k)) & 255u;
      c[8 * d + k] = byte & 7u;
      c[8 * d + 4 + k] = (byte >> 3) & 7u;
    }
  for (int k = 0; k < 4; ++k) {
    const uint32_t b0 = (w[0] >> (8 * k)) & 255u, b1 = (w[1] >> (8 * k)) & 255u,
                   b2 = (w[2] >> (8 * k)) & 255u;
    c[24 + k] = ((b0 >> 6) & 3u) | (((b2 >> 6) & 1u) << 2);
    c[28 + k] = ((b1 >> 6) & 3u) | (((b2 >> 7) & 1u) << 2);
  }
}

void place_chunk(int bits, int format, const uint32_t* c, uint32_t* w) {
  if (format == QGEMV_FMT_UNIFORM)
    bits == 4 ? place_u4(c, w) : place_u3(c, w);
  else
    bits == 4 ? place_l4(c, w) : place_l3(c, w);
}

void unplace_chunk(int bits, int format, const uint32_t* w, uint32_t* c) {
  if (format == QGEMV_FMT_UNIFORM)
    bits == 4 ? unplace_u4(w, c) : unplace_u3(w, c);
  else
    bits == 4 ? unplace_l4(w, c) : unplace_l3(w, c);
}

}  // namespace

// ---------------------------------------------------------------------------
// Validation shared by the entry points
// ---------------------------------------------------------------------------
int qgemv_validate_shape(const qgemv_weights* w) {
  if (!w) return QGEMV_ERR_INVALID_ARG;
  if (w->M < 1 || w->K < 1 || w->nnz < 0) return QGEMV_ERR_INVALID_ARG;
  if (w->format == QGEMV_FMT_HPTQ) {
    if (w->group_size != kBlockK || w->K % kBlockK != 0 || w->K > kMaxK) return QGEMV_ERR_UNSUPPORTED;
    if (w->nnz != 0) return QGEMV_ERR_UNSUPPORTED;  // one grid for inliers and outliers, no CSR
    if (w->huff_nsym < 1 || w->huff_nsym > kHuffMaxSym) return QGEMV_ERR_UNSUPPORTED;
    if ((int64_t)w->M * w->K > ((int64_t)1 << 40)) return QGEMV_ERR_UNSUPPORTED;
    return QGEMV_OK;
  }
  if (w->bits != 3 && w->bits != 4) return QGEMV_ERR_UNSUPPORTED;
  if (w->format != QGEMV_FMT_UNIFORM && w->format != QGEMV_FMT_LUT && w->format != QGEMV_FMT_BPDQ)
    return QGEMV_ERR_UNSUPPORTED;
  if (w->K % kChunkCodes != 0 || w->K > kMaxK) return QGEMV_ERR_UNSUPPORTED;
  if (w->format == QGEMV_FMT_UNIFORM && w->group_size != 16) return QGEMV_ERR_UNSUPPORTED;
  if (w->format == QGEMV_FMT_BPDQ) {
    if (w->bits != 3) return QGEMV_ERR_UNSUPPORTED;
    if (w->group_size != 32 && w->group_size != 64 && w->group_size != 128) return QGEMV_ERR_UNSUPPORTED;
    if (w->K % w->group_size != 0) return QGEMV_ERR_UNSUPPORTED;
  }
  if (w->nnz > 0x1fffffffLL) return QGEMV_ERR_UNSUPPORTED;  // byte offsets of entries stay in int32
  if ((int64_t)w->M * w->K > ((int64_t)1 << 40)) return QGEMV_ERR_UNSUPPORTED;
  // the kernels address every section with 31-bit byte offsets
  const BlobHeader h = make_header(w->M, w->K, w->bits, w->format, w->group_size, w->nnz);
  if (h.total_bytes >= ((uint64_t)1 << 31)) return QGEMV_ERR_UNSUPPORTED;
  return QGEMV_OK;
}

// HPTQ: the canonical codewords of the code (lengths non-decreasing, integers
// ascending among equal lengths, Kraft sum <= 1), then every row decoded from
// the stream; q gets the integers [M][K].  Returns a status.
struct HuffCode {
  std::vector<uint32_t> code;  // canonical codeword of each entry
  int first[kHuffMaxLen + 1], count[kHuffMaxLen + 1], offset[kHuffMaxLen + 1];
};

// Number of second-level tables: the distinct kHuffBits-bit prefixes among
// codewords longer than kHuffBits, at least 1 (with no long codeword, one
// table of length-16 entries keeps a decoder that meets bits starting no
// codeword advancing by a bounded length).
static uint32_t hptq_nsub(const qgemv_weights* w, const HuffCode& hc) {
  uint32_t n = 0;
  int64_t last = -1;
  for (int k = 0; k < w->huff_nsym; ++k) {  // canonical order: prefixes ascend
    const int l = w->huff_len[k];
    if (l <= kHuffBits) continue;
    const int64_t pre = hc.code[k] >> (l - kHuffBits);
    if (pre != last) ++n;
    last = pre;
  }
  return n > 0 ? n : 1;
}

static int hptq_code(const qgemv_weights* w, HuffCode& hc) {
  const int n = w->huff_nsym;
  if (!w->huff_len || !w->huff_sym) return QGEMV_ERR_INVALID_ARG;
  double kraft = 0.0;
  for (int l = 0; l <= kHuffMaxLen; ++l) hc.first[l] = hc.count[l] = hc.offset[l] = 0;
  hc.code.assign(n, 0);
  uint32_t code = 0;
  for (int k = 0; k < n; ++k) {
    const int l = w->huff_len[k], q = w->huff_sym[k];
    if (l < 1 || l > kHuffMaxLen || q < -2048 || q > 2048) return QGEMV_ERR_INVALID_ARG;
    if (k > 0) {
      const int lp = w->huff_len[k - 1];
      if (l < lp || (l == lp && q <= w->huff_sym[k - 1])) return QGEMV_ERR_INVALID_ARG;
      code = (code + 1) << (l - lp);
    }
    hc.code[k] = code;
    if (hc.count[l]++ == 0) {
      hc.first[l] = (int)code;
      hc.offset[l] = k;
    }
    kraft += std::ldexp(1.0, -l);
  }
  if (kraft > 1.0) return QGEMV_ERR_INVALID_ARG;
  return QGEMV_OK;
}

static int hptq_decode(const qgemv_weights* w, const HuffCode& hc, std::vector<int16_t>& q) {
  const int64_t M = w->M, K = w->K;
  if (!w->codes || !w->row_bits || !w->scales) return QGEMV_ERR_INVALID_ARG;
  if (w->row_bits[0] != 0) return QGEMV_ERR_INVALID_ARG;
  q.assign((size_t)(M * K), 0);
  for (int64_t i = 0; i < M; ++i) {
    int64_t p = w->row_bits[i];
    const int64_t end = w->row_bits[i + 1];
    if (end < p) return QGEMV_ERR_INVALID_ARG;
    for (int64_t j = 0; j < K; ++j) {
      uint32_t c = 0;
      int l = 0, sym = -1;
      while (sym < 0) {
        if (p >= end || l >= kHuffMaxLen) return QGEMV_ERR_INVALID_ARG;
        c = (c << 1) | ((w->codes[p >> 3] >> (7 - (p & 7))) & 1u);
        ++p;
        ++l;
        if (hc.count[l] && c >= (uint32_t)hc.first[l] && c - (uint32_t)hc.first[l] < (uint32_t)hc.count[l])
          sym = hc.offset[l] + (int)(c - (uint32_t)hc.first[l]);
      }
      q[(size_t)(i * K + j)] = w->huff_sym[sym];
    }
    if (p != end) return QGEMV_ERR_INVALID_ARG;
  }
  const int64_t n = M * (K / kBlockK);
  for (int64_t i = 0; i < n; ++i)
    if (!half_finite(w->scales[i])) return QGEMV_ERR_INVALID_ARG;
  return QGEMV_OK;
}

// Words of the HPTQ code section: every block's chunks, padded to 16 bytes.
static uint64_t hptq_words(const qgemv_weights* w, const HuffCode& hc, const std::vector<int16_t>& q,
                           std::vector<uint32_t>* hidx, uint32_t* maxw) {
  const int M = w->M, K = w->K, nkb = K / kBlockK, tiles = (M + kTileRows - 1) / kTileRows;
  std::vector<int> len_of(4097, 0);
  for (int k = 0; k < w->huff_nsym; ++k) len_of[w->huff_sym[k] + 2048] = w->huff_len[k];
  uint64_t words = 0;
  *maxw = 0;
  if (hidx) hidx->assign((size_t)tiles * nkb + 1, 0);
  for (int t = 0; t < tiles; ++t)
    for (int b = 0; b < nkb; ++b) {
      if (hidx) (*hidx)[(size_t)t * nkb + b] = (uint32_t)words;
      uint64_t bits = 0;
      for (int r = 0; r < kTileRows; ++r) {
        const int row = t * kTileRows + r;
        if (row >= M) continue;
        for (int j = 0; j < kBlockK; ++j) bits += len_of[q[(size_t)row * K + b * kBlockK + j] + 2048];
      }
      const uint64_t bw = ((bits + 31) / 32 + 3) / 4 * 4;
      if (bw > *maxw) *maxw = (uint32_t)bw;
      words += bw;
    }
  if (hidx) (*hidx)[(size_t)tiles * nkb] = (uint32_t)words;
  return words;
}

static int validate_arrays(const qgemv_weights* w) {
  int st = qgemv_validate_shape(w);
  if (st) return st;
  if (w->format == QGEMV_FMT_HPTQ) {
    if (!w->row_ptr || w->row_ptr[0] != 0 || w->row_ptr[w->M] != 0) return QGEMV_ERR_MALFORMED_CSR;
    return QGEMV_OK;  // the code and the stream are checked while they are decoded
  }
  const int64_t M = w->M, K = w->K, nnz = w->nnz;
  if (!w->codes || !w->row_ptr) return QGEMV_ERR_INVALID_ARG;
  if (nnz > 0 && (!w->col_idx || !w->values)) return QGEMV_ERR_INVALID_ARG;
  const int L = (1 << w->bits) - 1;
  if (w->format == QGEMV_FMT_UNIFORM) {
    if (!w->scales || !w->zeros) return QGEMV_ERR_INVALID_ARG;
    const int64_t n = M * (K / w->group_size);
    for (int64_t i = 0; i < n; ++i) {
      if (!half_finite(w->scales[i])) return QGEMV_ERR_INVALID_ARG;
      if (std::fabs(half_to_float(w->scales[i])) * (float)L > 65504.0f) return QGEMV_ERR_UNSUPPORTED;
      const float z = half_to_float(w->zeros[i]);
      if (!(z >= 0.0f && z <= (float)L && z == std::floor(z))) return QGEMV_ERR_INVALID_ARG;
    }
  } else if (w->format == QGEMV_FMT_LUT) {
    if (!w->lut) return QGEMV_ERR_INVALID_ARG;
    const int64_t n = M << w->bits;
    for (int64_t i = 0; i < n; ++i)
      if (!half_finite(w->lut[i])) return QGEMV_ERR_INVALID_ARG;
  } else {
    if (!w->coefs) return QGEMV_ERR_INVALID_ARG;
    const int E = w->bits + 1;
    const int64_t n = M * (K / w->group_size);
    for (int64_t i = 0; i < n; ++i) {
      float span = 0.0f;  // largest |level| a code can reach
      for (int t = 0; t < E; ++t) {
        const uint16_t c = w->coefs[i * E + t];
        if (!half_finite(c)) return QGEMV_ERR_INVALID_ARG;
        span += std::fabs(half_to_float(c));
      }
      if (span > 65504.0f) return QGEMV_ERR_UNSUPPORTED;  // levels are split into FP16 parts
    }
  }
  if (w->row_ptr[0] != 0 || (int64_t)w->row_ptr[M] != nnz) return QGEMV_ERR_MALFORMED_CSR;
  for (int64_t i = 0; i < M; ++i) {
    const int32_t a = w->row_ptr[i], b = w->row_ptr[i + 1];
    if (b < a || a < 0 || (int64_t)b > nnz) return QGEMV_ERR_MALFORMED_CSR;
    for (int32_t p = a; p < b; ++p) {
      const int32_t c = w->col_idx[p];
      if (c < 0 || c >= K) return QGEMV_ERR_MALFORMED_CSR;
      if (p > a && c <= w->col_idx[p - 1]) return QGEMV_ERR_MALFORMED_CSR;
      if (!half_finite(w->values[p])) return QGEMV_ERR_INVALID_ARG;
    }
  }
  return QGEMV_OK;
}

void qgemv_set_hip_error(int e) { g_last_hip_error = e; }

extern "C" {

// The blob header of a validated descriptor (HPTQ: decodes the stream to size the code section).
static int header_of(const qgemv_weights* w, BlobHeader& h, HuffCode* hc_out = nullptr,
                     std::vector<int16_t>* q_out = nullptr) {
  int st = validate_arrays(w);
  if (st) return st;
  uint32_t words = 0, maxw = 0, nsub = 0;
  if (w->format == QGEMV_FMT_HPTQ) {
    HuffCode hc;
    std::vector<int16_t> q;
    if ((st = hptq_code(w, hc))) return st;
    nsub = hptq_nsub(w, hc);
    if ((st = hptq_decode(w, hc, q))) return st;
    const uint64_t nw = hptq_words(w, hc, q, nullptr, &maxw);
    if (nw >= ((uint64_t)1 << 29)) return QGEMV_ERR_UNSUPPORTED;
    words = (uint32_t)nw;
    if (hc_out) *hc_out = hc;
    if (q_out) q_out->swap(q);
  }
  h = make_header(w->M, w->K, w->bits, w->format, w->group_size, w->nnz, w->huff_nsym, words, maxw, nsub);
  if (h.total_bytes >= ((uint64_t)1 << 31)) return QGEMV_ERR_UNSUPPORTED;
  return QGEMV_OK;
}

int qgemv_packed_size(const qgemv_weights* w, size_t* bytes) {
  if (!bytes) return QGEMV_ERR_INVALID_ARG;
  BlobHeader h;
  const int st = header_of(w, h);
  if (st) return st;
  *bytes = (size_t)h.total_bytes;
  return QGEMV_OK;
}

// HPTQ repack: every block's chunks re-laid from the stream, the steps, the
// block and lane offsets and the decode tables (see qgemv_layout.h).
static void put_bits(uint32_t* words, uint64_t pos, uint32_t code, int len) {
  for (int i = 0; i < len; ++i) {
    const uint64_t p = pos + (uint64_t)i;
    words[p >> 5] |= ((code >> (len - 1 - i)) & 1u) << (31 - (p & 31));
  }
}

static int repack_hptq(const qgemv_weights* w, void* dst_host, size_t bytes) {
  BlobHeader h;
  HuffCode hc;
  std::vector<int16_t> q;
  const int st = header_of(w, h, &hc, &q);
  if (st) return st;
  if (bytes < h.total_bytes) return QGEMV_ERR_SIZE;
  uint8_t* blob = (uint8_t*)dst_host;
  std::memset(blob, 0, (size_t)h.total_bytes);
  std::memcpy(blob, &h, sizeof(h));
  const int M = w->M, K = w->K, nkb = h.nkb, tiles = h.tiles, n = w->huff_nsym;
  std::vector<uint32_t> cw(4097, 0);
  std::vector<int> cl(4097, 0);
  for (int k = 0; k < n; ++k) {
    cw[w->huff_sym[k] + 2048] = hc.code[k];
    cl[w->huff_sym[k] + 2048] = w->huff_len[k];
  }
  std::vector<uint32_t> hidx;
  uint32_t maxw;
  hptq_words(w, hc, q, &hidx, &maxw);
  uint32_t* words = (uint32_t*)(blob + h.off_codes);
  uint16_t* hlane = (uint16_t*)(blob + h.off_hlane);
  uint16_t* steps = (uint16_t*)(blob + h.off_meta);
  for (int t = 0; t < tiles; ++t)
    for (int b = 0; b < nkb; ++b) {
      const size_t blk = (size_t)t * nkb + b;
      const uint64_t base = (uint64_t)hidx[blk] * 32;
      uint32_t p = 0;
      for (int l = 0; l < 64; ++l) {
        hlane[blk * 64 + l] = (uint16_t)p;
        const int row = t * kTileRows + l % 16;
        if (row >= M) continue;
        for (int j = 0; j < kChunkCodes; ++j) {
          const int v = q[(size_t)row * K + b * kBlockK + 32 * (l / 16) + j] + 2048;
          put_bits(words, base + p, cw[v], cl[v]);
          p += (uint32_t)cl[v];
        }
      }
      for (int r = 0; r < kTileRows; ++r) {
        const int row = t * kTileRows + r;
        steps[blk * kTileRows + r] = row < M ? w->scales[(size_t)row * nkb + b] : 0;
      }
    }
  std::memcpy(blob + h.off_hidx, hidx.data(), 4 * hidx.size());
  int32_t* tab = (int32_t*)(blob + h.off_htab);
  int32_t* sub = tab + kHuffTable + 4 * 17;
  for (uint32_t i = 0; i < (uint32_t)kHuffSub * h.hsub; ++i) sub[i] = kHuffMaxLen;
  int64_t last = -1;
  int nsub = -1;
  for (int k = 0; k < n; ++k) {
    const int l = w->huff_len[k];
    const uint32_t e = ((uint32_t)int_to_half(w->huff_sym[k]) << 16) | (uint32_t)l;
    if (l <= kHuffBits) {
      const uint32_t lo = hc.code[k] << (kHuffBits - l);
      for (uint32_t s = 0; s < (1u << (kHuffBits - l)); ++s) tab[lo + s] = (int32_t)e;
      continue;
    }
    const uint32_t pre = hc.code[k] >> (l - kHuffBits);
    if ((int64_t)pre != last) {
      ++nsub;
      last = pre;
      tab[pre] = (int32_t)((uint32_t)(kHuffSub * nsub) << 16);
    }
    const uint32_t lo = (hc.code[k] << (kHuffMaxLen - l)) & (uint32_t)(kHuffSub - 1);
    for (uint32_t s = 0; s < (1u << (kHuffMaxLen - l)); ++s) sub[kHuffSub * nsub + lo + s] = (int32_t)e;
  }
  int32_t* slow = tab + kHuffTable;
  int32_t lim = 0;
  for (int l = 0; l <= kHuffMaxLen; ++l) {
    slow[l] = hc.first[l];
    slow[17 + l] = hc.count[l];
    slow[34 + l] = hc.offset[l];
    if (hc.count[l]) lim = (hc.first[l] + hc.count[l]) << (kHuffMaxLen - l);
    slow[51 + l] = lim;
  }
  std::memcpy(blob + h.off_hsym, w->huff_sym, 2 * (size_t)n);
  return QGEMV_OK;
}

int qgemv_repack(const qgemv_weights* w, void* dst_host, size_t bytes) {
  if (!dst_host) return QGEMV_ERR_INVALID_ARG;
  if (w && w->format == QGEMV_FMT_HPTQ) return repack_hptq(w, dst_host, bytes);
  const int st = validate_arrays(w);
  if (st) return st;
  const BlobHeader h = make_header(w->M, w->K, w->bits, w->format, w->group_size, w->nnz);
  if (bytes < h.total_bytes) return QGEMV_ERR_SIZE;
  uint8_t* blob = (uint8_t*)dst_host;
  std::memset(blob, 0, (size_t)h.total_bytes);
  std::memcpy(blob, &h, sizeof(h));

  const int M = w->M, K = w->K, bits = w->bits, Kp = h.Kp, nkb = h.nkb;
  const size_t row_bytes = (size_t)K * bits / 8;
  const int chunk_bytes = 4 * bits;
  std::vector<uint8_t> tile((size_t)kTileRows * Kp);   // canonical codes of one tile, zero padded
  uint32_t c[32], dw[4];
  for (int t = 0; t < h.tiles; ++t) {
    std::fill(tile.begin(), tile.end(), (uint8_t)0);
    for (int r = 0; r < kTileRows; ++r) {
      const int row = t * kTileRows + r;
      if (row >= M) break;
      canon_unpack_row(w->codes + (size_t)row * row_bytes, K, bits, tile.data() + (size_t)r * Kp);
    }
    for (int b = 0; b < nkb; ++b) {
      uint8_t* dst = blob + h.off_codes + ((size_t)t * nkb + b) * h.block_bytes;
      for (int l = 0; l < 64; ++l) {
        const uint8_t* src = tile.data() + (size_t)(l % 16) * Kp + b * kBlockK + 32 * (l / 16);
        for (int j = 0; j < 32; ++j) c[j] = src[j];
        place_chunk(bits, w->format, c, dw);
        std::memcpy(dst + (size_t)l * chunk_bytes, dw, chunk_bytes);
      }
    }
  }

  uint8_t* meta = blob + h.off_meta;
  if (w->format == QGEMV_FMT_UNIFORM) {
    // per (tile, K-block): z plane [16 rows][8 groups], then s plane [4 group pairs][16 rows][2]
    const int G = K / w->group_size;
    for (int t = 0; t < h.tiles; ++t)
      for (int b = 0; b < nkb; ++b) {
        uint16_t* zp = (uint16_t*)(meta + ((size_t)t * nkb + b) * h.meta_unit_bytes);
        uint16_t* sp = zp + kTileRows * 8;
        for (int r = 0; r < kTileRows; ++r) {
          const int row = t * kTileRows + r;
          for (int g = 0; g < 8; ++g) {
            const int gg = b * 8 + g;
            uint16_t sv = 0, zv = 0;
            if (row < M && gg < G) {
              sv = w->scales[(size_t)row * G + gg];
              zv = w->zeros[(size_t)row * G + gg];
            }
            zp[r * 8 + g] = zv;
            sp[(g / 2) * 32 + r * 2 + (g % 2)] = sv;
          }
        }
      }
  } else if (w->format == QGEMV_FMT_LUT) {
    const int E = 1 << bits;
    for (int i = 0; i < M; ++i)
      std::memcpy(meta + (size_t)i * h.meta_unit_bytes, w->lut + (size_t)i * E, 2 * (size_t)E);
  } else {
    // per (tile, K-block): [16 rows][128 / group groups][bits + 1] FP16
    const int gs = w->group_size, gpk = kBlockK / gs, G = K / gs, E = bits + 1;
    for (int t = 0; t < h.tiles; ++t)
      for (int b = 0; b < nkb; ++b) {
        uint16_t* cp = (uint16_t*)(meta + ((size_t)t * nkb + b) * h.meta_unit_bytes);
        for (int r = 0; r < kTileRows; ++r) {
          const int row = t * kTileRows + r;
          for (int g = 0; g < gpk; ++g) {
            const int gg = b * gpk + g;
            for (int e = 0; e < E; ++e)
              cp[(r * gpk + g) * E + e] = row < M && gg < G ? w->coefs[((size_t)row * G + gg) * E + e] : 0;
          }
        }
      }
  }

  std::memcpy(blob + h.off_rowptr, w->row_ptr, 4ull * ((size_t)M + 1));
  uint32_t* ent = (uint32_t*)(blob + h.off_entries);
  for (int64_t p = 0; p < w->nnz; ++p)
    ent[p] = (uint32_t)w->col_idx[p] | ((uint32_t)w->values[p] << 16);

  // The outliers again, grouped by (tile, K-block): a counting sort over the
  // rows in order keeps rows, then columns, ascending inside each group.
  const size_t nblocks = (size_t)h.tiles * nkb;
  int32_t* boff = (int32_t*)(blob + h.off_boff);
  uint32_t* bent = (uint32_t*)(blob + h.off_bent);
  for (int row = 0; row < M; ++row)
    for (int32_t p = w->row_ptr[row]; p < w->row_ptr[row + 1]; ++p)
      ++boff[(size_t)(row / kTileRows) * nkb + w->col_idx[p] / kBlockK + 1];
  for (size_t i = 0; i < nblocks; ++i) boff[i + 1] += boff[i];
  std::vector<int32_t> fill(boff, boff + nblocks);
  for (int row = 0; row < M; ++row)
    for (int32_t p = w->row_ptr[row]; p < w->row_ptr[row + 1]; ++p) {
      const int c = w->col_idx[p];
      const size_t i = (size_t)(row / kTileRows) * nkb + c / kBlockK;
      bent[fill[i]++] = (uint32_t)(c % kBlockK) | ((uint32_t)(row % kTileRows) << 7) | ((uint32_t)w->values[p] << 16);
    }
  return QGEMV_OK;
}

int qgemv_unpack_host(const void* blob_host, size_t bytes, uint8_t* codes_out, size_t codes_bytes) {
  if (!blob_host || !codes_out) return QGEMV_ERR_INVALID_ARG;
  if (bytes < sizeof(BlobHeader)) return QGEMV_ERR_SIZE;
  BlobHeader h;
  std::memcpy(&h, blob_host, sizeof(h));
  if (h.magic != kMagic || h.version != kVersion) return QGEMV_ERR_SIZE;
  if (h.format == QGEMV_FMT_HPTQ) return QGEMV_ERR_UNSUPPORTED;
  // Every field must be the one the repacker writes for the header's own
  // shape, so the loop below stays inside the blob.
  qgemv_weights shape{};
  shape.M = h.M;
  shape.K = h.K;
  shape.bits = h.bits;
  shape.format = h.format;
  shape.group_size = h.format == QGEMV_FMT_LUT ? 16 : h.group_size;
  shape.nnz = h.nnz;
  if (qgemv_validate_shape(&shape) != QGEMV_OK) return QGEMV_ERR_SIZE;
  const BlobHeader expect = make_header(h.M, h.K, h.bits, h.format, shape.group_size, h.nnz);
  if (std::memcmp(&expect, &h, sizeof(h)) != 0) return QGEMV_ERR_SIZE;
  if (h.total_bytes > bytes) return QGEMV_ERR_SIZE;
  if ((uint64_t)h.M * (uint64_t)h.K > codes_bytes) return QGEMV_ERR_SIZE;
  const uint8_t* blob = (const uint8_t*)blob_host;
  const int chunk_bytes = 4 * h.bits;
  uint32_t c[32], dw[4] = {0, 0, 0, 0};
  for (int t = 0; t < h.tiles; ++t)
    for (int b = 0; b < h.nkb; ++b)
      for (int l = 0; l < 64; ++l) {
        const int row = t * kTileRows + l % 16;
        if (row >= h.M) continue;
        std::memcpy(dw, blob + h.off_codes + ((size_t)t * h.nkb + b) * h.block_bytes + (size_t)l * chunk_bytes,
                    chunk_bytes);
        unplace_chunk(h.bits, h.format, dw, c);
        const int k0 = b * kBlockK + 32 * (l / 16);
        for (int j = 0; j < 32 && k0 + j < h.K; ++j) codes_out[(size_t)row * h.K + k0 + j] = (uint8_t)c[j];
      }
  return QGEMV_OK;
}

const char* qgemv_error_string(int status) {
  switch (status) {
    case QGEMV_OK: return "ok";
    case QGEMV_ERR_INVALID_ARG: return "invalid argument";
    case QGEMV_ERR_MALFORMED_CSR: return "malformed CSR (row_ptr/col_idx)";
    case QGEMV_ERR_UNSUPPORTED: return "unsupported bits/format/group/K/batch";
    case QGEMV_ERR_HIP: return "HIP runtime error";
    case QGEMV_ERR_SIZE: return "buffer too small or blob header mismatch";
    case QGEMV_ERR_SCRATCH: return "workspace needed exceeds the static scratch of qgemv_run_noalloc";
    default: return "unknown status";
  }
}

int qgemv_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
