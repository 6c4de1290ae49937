// host_sanitize_driver.cpp -- runs the library's host entry points
// (qgemv_packed_size, qgemv_repack, qgemv_unpack_host) on canonical arrays
// read from a case file, for an AddressSanitizer + UndefinedBehaviorSanitizer
// build of qgemv_host.cpp (test infrastructure; built with g++, no GPU code).
//
// Every array gets its own heap block of exactly the length the case file
// gives, so a read past the end of any input is reported.
//
// Case file: int64 M, K, bits, format, group_size, nnz, huff_nsym, flags;
// then 11 arrays, each an int64 byte length (0 = NULL) and the bytes, in the
// order codes, scales, zeros, lut, row_ptr, col_idx, values, coefs, huff_len,
// huff_sym, row_bits.
//
// usage: host_sanitize_driver CASE OUT_BLOB OUT_CODES
// Prints "packed_size <status> <bytes>", "repack <status>", "unpack <status>"
// and "header_fuzz <accepted> <rejected>"; writes the blob and the codes.

#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "../../include/qgemv.h"

namespace {

std::vector<unsigned char> slurp(const char* path) {
  std::vector<unsigned char> v;
  FILE* f = std::fopen(path, "rb");
  if (!f) return v;
  unsigned char buf[65536];
  size_t n;
  while ((n = std::fread(buf, 1, sizeof buf, f)) > 0) v.insert(v.end(), buf, buf + n);
  std::fclose(f);
  return v;
}

bool spit(const char* path, const void* p, size_t n) {
  FILE* f = std::fopen(path, "wb");
  if (!f) return false;
  const bool ok = n == 0 || std::fwrite(p, 1, n, f) == n;
  return std::fclose(f) == 0 && ok;
}

struct Reader {
  const std::vector<unsigned char>& d;
  size_t pos = 0;
  bool ok = true;
  int64_t i64() {
    int64_t v = 0;
    if (pos + 8 > d.size()) { ok = false; return 0; }
    std::memcpy(&v, d.data() + pos, 8);
    pos += 8;
    return v;
  }
  void* array() {  // exact-size heap copy, or NULL for length 0
    const int64_t n = i64();
    if (!ok || n < 0 || pos + (size_t)n > d.size()) { ok = false; return nullptr; }
    if (n == 0) return nullptr;
    void* p = std::malloc((size_t)n);
    std::memcpy(p, d.data() + pos, (size_t)n);
    pos += (size_t)n;
    return p;
  }
};

}  // namespace

int main(int argc, char** argv) {
  if (argc != 4) {
    std::fprintf(stderr, "usage: %s CASE OUT_BLOB OUT_CODES\n", argv[0]);
    return 2;
  }
  const std::vector<unsigned char> data = slurp(argv[1]);
  Reader r{data};
  qgemv_weights w{};
  w.M = (int32_t)r.i64();
  w.K = (int32_t)r.i64();
  w.bits = (int32_t)r.i64();
  w.format = (int32_t)r.i64();
  w.group_size = (int32_t)r.i64();
  w.nnz = r.i64();
  w.huff_nsym = (int32_t)r.i64();
  (void)r.i64();  // flags (unused)
  void* arrays[11];
  for (void*& a : arrays) a = r.array();
  if (!r.ok || r.pos != data.size()) {
    std::fprintf(stderr, "malformed case file\n");
    return 2;
  }
  w.codes = (const uint8_t*)arrays[0];
  w.scales = (const uint16_t*)arrays[1];
  w.zeros = (const uint16_t*)arrays[2];
  w.lut = (const uint16_t*)arrays[3];
  w.row_ptr = (const int32_t*)arrays[4];
  w.col_idx = (const int32_t*)arrays[5];
  w.values = (const uint16_t*)arrays[6];
  w.coefs = (const uint16_t*)arrays[7];
  w.huff_len = (const uint8_t*)arrays[8];
  w.huff_sym = (const int16_t*)arrays[9];
  w.row_bits = (const int64_t*)arrays[10];

  size_t bytes = 0;
  int st = qgemv_packed_size(&w, &bytes);
  std::printf("packed_size %d %zu\n", st, bytes);
  if (st == QGEMV_OK) {
    unsigned char* blob = (unsigned char*)std::malloc(bytes);
    // one byte short first: must be refused without writing past the buffer
    std::printf("repack_short %d\n", qgemv_repack(&w, blob, bytes - 1));
    st = qgemv_repack(&w, blob, bytes);
    std::printf("repack %d\n", st);
    if (st == QGEMV_OK && !spit(argv[2], blob, bytes)) return 3;
    if (st == QGEMV_OK && w.format != QGEMV_FMT_HPTQ) {
      const size_t n = (size_t)w.M * (size_t)w.K;
      unsigned char* codes = (unsigned char*)std::malloc(n);
      st = qgemv_unpack_host(blob, bytes, codes, n);
      std::printf("unpack %d\n", st);
      if (st == QGEMV_OK && !spit(argv[3], codes, n)) return 3;
      // every int32 word of the header set to a few other values: the call
      // must refuse or stay inside the blob and the output buffer
      int accepted = 0, rejected = 0;
      unsigned char* bad = (unsigned char*)std::malloc(bytes);
      const int32_t probes[] = {0, 1, -1, 3, 4, 16, 128, 4096, 1 << 20, 1 << 30};
      for (int word = 0; word < 64; ++word)
        for (int32_t v : probes) {
          std::memcpy(bad, blob, bytes);
          std::memcpy(bad + 4 * word, &v, 4);
          (qgemv_unpack_host(bad, bytes, codes, n) == QGEMV_OK ? accepted : rejected)++;
        }
      std::printf("header_fuzz %d %d\n", accepted, rejected);
      std::printf("unpack_truncated %d\n", qgemv_unpack_host(blob, bytes - 1, codes, n));
      std::free(bad);
      std::free(codes);
    }
    std::free(blob);
  }
  for (void* a : arrays) std::free(a);
  return 0;
}
