// qgemv_kernels.hip -- gfx950 kernels and the device side of the C ABI.
//
// The product runs on 16-row tiles.  In a batch-1 launch one workgroup owns
// one tile and its KS waves split the K-blocks of that tile:
//   * each lane streams the 32-code chunks of its row (16 B or 12 B per
//     K-block, 1 KiB / 768 B contiguous per wave load), through a ring of PF
//     K-blocks held in registers;
//   * it turns them into FP16 A operands -- v_perm byte lookups in the row's
//     table for LUT codes, a magic-number OR plus exact FP16 scaling for
//     uniform codes -- and issues 16x16x32 MFMAs against x read from LDS (B
//     operand, the same x in every column), fp32 accumulation;
//   * the row's CSR outliers are gathered from the same LDS copy of x and
//     reduced with a DPP wave sum;
//   * partial sums of the KS waves meet in LDS and are added in a fixed order,
//     so every output is written once, with no atomics, deterministically.
//
// Uniform codes: the group scale s is split into s_hi (s with the four low
// mantissa bits cleared) and s_lo = s - s_hi.  (q - z) * s_hi and (q - z) * s_lo
// are exact in FP16, so two MFMAs reproduce s * (q - z) * x without rounding
// the decoded weight.

#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>
#include <new>

#include "../../include/qgemv.h"
#include "qgemv_decode.h"
#include "qgemv_internal.h"
#include "qgemv_layout.h"

using namespace qgemv_layout;
using namespace qgemv_dev;

struct qgemv_plan {
  BlobHeader h;
  const uint8_t* blob;
};

namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ half8_t h8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  const u32x4_t v = {a, b, c, d};
  return __builtin_bit_cast(half8_t, v);
}

__device__ __forceinline__ floatx4_t mfma(half8_t a, half8_t b, floatx4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// FP16 pair (-(base + z), -(base + z)); exact for the small integers used here.
__device__ __forceinline__ uint32_t hsplat_neg_sum(uint32_t z_bits, float base) {
  const _Float16 z = __builtin_bit_cast(_Float16, (uint16_t)z_bits);
  const _Float16 c = (_Float16)(-base) - z;
  const uint16_t b = __builtin_bit_cast(uint16_t, c);
  return (uint32_t)b | ((uint32_t)b << 16);
}

__device__ __forceinline__ uint32_t hsplat(uint16_t b) { return (uint32_t)b | ((uint32_t)b << 16); }

// (1024 + k*q) pair -> (q - z) pair, exactly: h * (1/k) + (-(1024/k) - z).
__device__ __forceinline__ uint32_t to_qz(uint32_t h, uint32_t c, _Float16 inv_k) {
  return as_u32(as_h2(h) * (half2_t){inv_k, inv_k} + as_h2(c));
}

__device__ __forceinline__ uint32_t hmul(uint32_t a, uint32_t b) { return as_u32(as_h2(a) * as_h2(b)); }

// Scale split of one group: s_hi = s with the low 4 mantissa bits cleared, s_lo = s - s_hi.
__device__ __forceinline__ void scale_split(uint32_t st, uint32_t& shi2, uint32_t& slo2) {
  const uint16_t s = (uint16_t)(st & 0xFFFFu);
  const uint16_t hi = (uint16_t)(s & 0xFFF0u);
  const _Float16 lo = __builtin_bit_cast(_Float16, s) - __builtin_bit_cast(_Float16, hi);
  shi2 = hsplat(hi);
  slo2 = hsplat(__builtin_bit_cast(uint16_t, lo));
}

// Byte planes of a canonical FP16 table (pairs of entries per dword).
__device__ __forceinline__ void l4_planes(const uint32_t L[8], uint32_t t[8]) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    t[q] = perm(L[2 * q + 1], L[2 * q], 0x06040200u);
    t[4 + q] = perm(L[2 * q + 1], L[2 * q], 0x07050301u);
  }
}
__device__ __forceinline__ void l3_planes(const uint32_t L[4], uint32_t t[4]) {
  t[0] = perm(L[1], L[0], 0x06040200u);
  t[1] = perm(L[3], L[2], 0x06040200u);
  t[2] = perm(L[1], L[0], 0x07050301u);
  t[3] = perm(L[3], L[2], 0x07050301u);
}

template <int FMT, int BITS>
struct Fmt {
  static constexpr bool lut = FMT == QGEMV_FMT_LUT;
  static constexpr int tab_dw = lut ? (BITS == 4 ? 8 : 4) : 1;
  static constexpr int n_mfma = lut ? 4 : 8;   // per K-block
};

// Decode one lane chunk into MFMA A operands.
//   LUT:     a[i][0..3] for step i = 0..3
//   UNIFORM: a[i] = hi part, a[4 + i] = lo part
template <int FMT, int BITS>
__device__ __forceinline__ void decode_chunk(const uint32_t (&c)[BITS], const uint32_t (&st)[2],
                                             const uint32_t (&tab)[Fmt<FMT, BITS>::tab_dw],
                                             uint32_t (&a)[Fmt<FMT, BITS>::n_mfma][4]) {
  if constexpr (FMT == QGEMV_FMT_LUT && BITS == 4) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t sa, sb;
      l4_sel(c[i], sa, sb);
      l4_lookup(tab, sa, 0x40404040u, a[i][0], a[i][1]);
      l4_lookup(tab, sb, 0x10101010u, a[i][2], a[i][3]);
    }
  } else if constexpr (FMT == QGEMV_FMT_LUT && BITS == 3) {
    uint32_t sel[8];
    l3_sel(c[0], c[1], c[2], sel);
#pragma unroll
    for (int q = 0; q < 8; ++q) l3_lookup(tab, sel[q], a[q / 2][2 * (q % 2)], a[q / 2][2 * (q % 2) + 1]);
  } else {
    uint32_t shi[2], slo[2], cz[2][3];
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      scale_split(st[g], shi[g], slo[g]);
      const uint32_t zb = st[g] >> 16;
      cz[g][0] = hsplat_neg_sum(zb, 1024.f);
      cz[g][1] = hsplat_neg_sum(zb, BITS == 4 ? 64.f : 128.f);
      cz[g][2] = hsplat_neg_sum(zb, 16.f);
    }
    if constexpr (BITS == 4) {
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const int g = d / 2;
        uint32_t h[4];
        u4_slots(c[d], h);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const uint32_t qz = (t & 1) ? to_qz(h[t], cz[g][1], (_Float16)0.0625f) : to_qz(h[t], cz[g][0], (_Float16)1.0f);
          a[d][t] = hmul(qz, shi[g]);
          a[4 + d][t] = hmul(qz, slo[g]);
        }
      }
    } else {
      uint32_t h[3][5];
      u3_slots(c[0], h[0]);
      u3_slots(c[1], h[1]);
      u3_slots(c[2], h[2]);
      const uint32_t hs = u3_spare(c[0], c[1], c[2]);
#pragma unroll
      for (int m = 0; m < 16; ++m) {
        const int g = m < 8 ? 0 : 1;
        uint32_t qz;
        if (m == 15) {
          qz = to_qz(hs, cz[g][0], (_Float16)1.0f);
        } else {
          const int d = m / 5, t = m % 5;
          if (t == 0 || t == 3) qz = to_qz(h[d][t], cz[g][0], (_Float16)1.0f);
          else if (t == 2) qz = to_qz(h[d][t], cz[g][2], (_Float16)0.015625f);
          else qz = to_qz(h[d][t], cz[g][1], (_Float16)0.125f);
        }
        a[m / 4][m % 4] = hmul(qz, shi[g]);
        a[4 + m / 4][m % 4] = hmul(qz, slo[g]);
      }
    }
  }
}

typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRsrcWord3 = 0x00020000;  // raw buffer, 32-bit data format

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kRsrcWord3);
}

// Loads through a range-checked buffer resource: offsets past the range read 0 and touch no memory.
template <int BITS>
__device__ __forceinline__ void load_chunk(uint32_t (&c)[BITS], rsrc_t r, uint32_t off) {
  if constexpr (BITS == 4) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
    c[0] = v[0]; c[1] = v[1]; c[2] = v[2]; c[3] = v[3];
  } else {
    const auto v = __builtin_amdgcn_raw_buffer_load_b96(r, (int)off, 0, 0);
    c[0] = v[0]; c[1] = v[1]; c[2] = v[2];
  }
}
__device__ __forceinline__ void load_stats(uint32_t (&s)[2], rsrc_t r, uint32_t off) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0);
  s[0] = v[0];
  s[1] = v[1];
}

constexpr uint32_t kOutOfRange = 0x7FFFFFF0u;

// ---------------------------------------------------------------------------
// Batch 1.  One workgroup of 16 waves per CU owns the contiguous tile range
// [T0, T1) and splits its (tile, K-block) pairs -- tile-major, i.e. one
// contiguous stretch of the blob -- evenly over its waves.  A wave therefore
// streams one contiguous run of K-blocks through a ring of PF register slots,
// crossing a tile boundary at most a few times; at each crossing it parks its
// partial sums for the finished tile in LDS.  After the stream each wave sums
// the outliers of its rows, and after one barrier the partials of every tile
// are added in a fixed order: two barriers per launch, deterministic output.
// ---------------------------------------------------------------------------
constexpr int kWaves = 16;
constexpr int kCsrRows = 8;  // outlier rows per wave whose first entries are prefetched

template <int FMT, int BITS, int PF, int NE>
__global__ void __launch_bounds__(64 * kWaves)
k_b1(const uint8_t* __restrict__ codes, const uint32_t* __restrict__ meta, const int32_t* __restrict__ row_ptr,
     const uint32_t* __restrict__ entries, const uint16_t* __restrict__ x, float* __restrict__ y, int M, int K,
     int Kp, int nkb, int tiles, uint32_t codes_bytes, uint32_t meta_bytes, int nnz) {
  using F = Fmt<FMT, BITS>;
  constexpr int BB = 256 * BITS;
  extern __shared__ uint32_t lds[];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int T0 = (int)((int64_t)blockIdx.x * tiles / gridDim.x);
  const int T1 = (int)((int64_t)(blockIdx.x + 1) * tiles / gridDim.x);
  const int TW = T1 - T0;
  const int nblk = TW * nkb;
  const int g0 = T0 * nkb + w * nblk / kWaves;
  const int g1 = T0 * nkb + (w + 1) * nblk / kWaves;
  const int nrows = min(TW * 16, M - T0 * 16);  // real rows of the workgroup

  // LDS: x [Kp] fp16 | partials [TW][kWaves][16] | csr [TW*16] | row_ptr [TW*16+4] | LUT [TW*16][tab_dw]
  uint16_t* x_lds = (uint16_t*)lds;
  float* part = (float*)(lds + Kp / 2);
  float* csr = part + TW * kWaves * 16;
  int* rp_lds = (int*)(csr + TW * 16);
  uint32_t* lut_lds = (uint32_t*)(rp_lds + TW * 16 + 4);  // 16-byte aligned

  const rsrc_t rc = make_rsrc(codes, codes_bytes);
  const rsrc_t rs = make_rsrc(meta, F::lut ? 0u : meta_bytes);

  // The code ring goes out first; x, the row_ptr slice and the tables follow
  // and land in LDS while the ring is in flight.
  const uint32_t voff = (uint32_t)lane * 4 * BITS;
  const uint32_t soff = (uint32_t)lane * 8;
  uint32_t cb[PF][BITS];
  uint32_t sb[PF][2];
#pragma unroll
  for (int u = 0; u < PF; ++u) {
    const int g = g0 + u;
    load_chunk<BITS>(cb[u], rc, g < g1 ? (uint32_t)g * BB + voff : kOutOfRange);
    if constexpr (!F::lut) load_stats(sb[u], rs, g < g1 ? (uint32_t)g * 512 + soff : kOutOfRange);
    else sb[u][0] = sb[u][1] = 0;
  }
  {
    const rsrc_t rx = make_rsrc(x, (uint32_t)K * 2);
    for (int i = threadIdx.x; i < Kp / 8; i += 64 * kWaves)
      ((u32x4_t*)x_lds)[i] = __builtin_amdgcn_raw_buffer_load_b128(rx, i * 16, 0, 0);
    const rsrc_t rr = make_rsrc(row_ptr, (uint32_t)(M + 1) * 4);
    for (int i = threadIdx.x; i <= TW * 16; i += 64 * kWaves)
      rp_lds[i] = __builtin_amdgcn_raw_buffer_load_b32(rr, min(T0 * 16 + i, M) * 4, 0, 0);
    if constexpr (F::lut) {
      const rsrc_t rl = make_rsrc(meta, meta_bytes);
      const int n = TW * 16 * F::tab_dw / 4;  // 16-byte pieces
      for (int i = threadIdx.x; i < n; i += 64 * kWaves)
        ((u32x4_t*)lut_lds)[i] = __builtin_amdgcn_raw_buffer_load_b128(rl, (T0 * 16 * F::tab_dw / 4 + i) * 16, 0, 0);
    }
    for (int j = lane; j < TW * 16; j += 64) part[((j >> 4) * kWaves + w) * 16 + (j & 15)] = 0.f;
  }
  __syncthreads();

  // First NE*64 entries of each of this wave's outlier rows (rows w, w+16, ...).
  const rsrc_t re = make_rsrc(entries, (uint32_t)nnz * 4);
  uint32_t ent[kCsrRows][NE];
#pragma unroll
  for (int j = 0; j < kCsrRows; ++j) {
    const int r = w + 16 * j;
    const int p0 = r < nrows ? rp_lds[r] : 0;
    const int cnt = r < nrows ? rp_lds[r + 1] - p0 : 0;
#pragma unroll
    for (int k = 0; k < NE; ++k) {
      const int q = lane + 64 * k;
      ent[j][k] = __builtin_amdgcn_raw_buffer_load_b32(re, q < cnt ? (p0 + q) * 4 : (int)kOutOfRange, 0, 0);
    }
  }

  int tc = g0 / nkb;  // current tile
  int kb = g0 - tc * nkb;
  uint32_t tab[F::tab_dw];
  auto planes = [&]() {
    if constexpr (F::lut) {
      const uint32_t* L = lut_lds + ((tc - T0) * 16 + (lane & 15)) * F::tab_dw;
      uint32_t Lr[F::tab_dw];
#pragma unroll
      for (int i = 0; i < F::tab_dw; ++i) Lr[i] = L[i];
      if constexpr (BITS == 4) l4_planes(Lr, tab);
      else l3_planes(Lr, tab);
    } else {
      tab[0] = 0;
    }
  };
  planes();

  const uint16_t* xb = x_lds + 32 * (lane >> 4);
  floatx4_t acc = {0.f, 0.f, 0.f, 0.f};
  auto flush = [&]() {  // rows 4*(lane/16) .. +3 of the tile sit in lanes 0, 16, 32, 48
    if ((lane & 15) == 0) {
      float* sl = part + ((tc - T0) * kWaves + w) * 16 + 4 * (lane >> 4);
#pragma unroll
      for (int r = 0; r < 4; ++r) sl[r] = acc[r];
    }
    acc = (floatx4_t){0.f, 0.f, 0.f, 0.f};
  };
  for (int gi = g0; gi < g1; gi += PF) {
#pragma unroll
    for (int u = 0; u < PF; ++u) {
      const int g = gi + u;
      if (g < g1) {
        if (kb == nkb) {
          flush();
          kb = 0;
          ++tc;
          planes();
        }
        uint32_t am[F::n_mfma][4];
        decode_chunk<FMT, BITS>(cb[u], sb[u], tab, am);
        const uint16_t* xk = xb + kb * kBlockK;
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) {
          const half8_t bx = *(const half8_t*)(xk + 8 * s2);
          acc = mfma(h8(am[s2][0], am[s2][1], am[s2][2], am[s2][3]), bx, acc);
          if constexpr (!F::lut) acc = mfma(h8(am[4 + s2][0], am[4 + s2][1], am[4 + s2][2], am[4 + s2][3]), bx, acc);
        }
        ++kb;
      }
      const int gn = g + PF;
      load_chunk<BITS>(cb[u], rc, gn < g1 ? (uint32_t)gn * BB + voff : kOutOfRange);
      if constexpr (!F::lut) load_stats(sb[u], rs, gn < g1 ? (uint32_t)gn * 512 + soff : kOutOfRange);
    }
  }
  if (g1 > g0) flush();

  // Outliers of this wave's rows; entries past the prefetched ones are read
  // four wave-loads at a time.
  for (int j = 0; w + 16 * j < nrows; ++j) {
    const int r = w + 16 * j;
    const int p0 = rp_lds[r];
    const int cnt = rp_lds[r + 1] - p0;
    float sum = 0.f;
    int k0 = 0;
    if (j < kCsrRows) {
#pragma unroll
      for (int jj = 0; jj < kCsrRows; ++jj)
        if (jj == j) {
#pragma unroll
          for (int k = 0; k < NE; ++k)
            if (lane + 64 * k < cnt) {
              const uint32_t e = ent[jj][k];
              sum = dot2(e >> 16, (uint32_t)x_lds[e & 0xFFFFu], sum);
            }
        }
      k0 = NE;
    }
    for (int k = k0; 64 * k < cnt; k += 4) {
      uint32_t e4[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int q = lane + 64 * (k + i);
        e4[i] = __builtin_amdgcn_raw_buffer_load_b32(re, q < cnt ? (p0 + q) * 4 : (int)kOutOfRange, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (lane + 64 * (k + i) < cnt) sum = dot2(e4[i] >> 16, (uint32_t)x_lds[e4[i] & 0xFFFFu], sum);
    }
    sum = wave_sum(sum);
    if (lane == 0) csr[r] = sum;
  }
  __syncthreads();
  for (int r = threadIdx.x; r < nrows; r += 64 * kWaves) {
    const float* pr = part + (r >> 4) * kWaves * 16 + (r & 15);
    float v = 0.f;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) v += pr[ww * 16];
    y[T0 * 16 + r] = v + csr[r];
  }
}

// Debug: decode the blob's codes back to canonical order, one thread per 32-code chunk.
template <int FMT, int BITS>
__global__ void __launch_bounds__(256)
k_unpack(const uint8_t* __restrict__ codes, uint8_t* __restrict__ out, int M, int K, int nkb, int tiles) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)tiles * nkb * 64) return;
  const int l = (int)(idx % 64);
  const int64_t tb = idx / 64;
  const int b = (int)(tb % nkb), t = (int)(tb / nkb);
  const int row = t * 16 + (l & 15);
  if (row >= M) return;
  uint32_t w[4] = {0, 0, 0, 0};
  const uint32_t* src = (const uint32_t*)(codes + tb * 256 * BITS + l * 4 * BITS);
#pragma unroll
  for (int d = 0; d < BITS; ++d) w[d] = src[d];
  uint8_t c[32];
  if constexpr (FMT == QGEMV_FMT_UNIFORM && BITS == 4) {
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      uint32_t h[4];
      u4_slots(w[d], h);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int sh = (s & 1) ? 4 : 0;
        c[2 * (4 * d + s)] = (uint8_t)((h[s] & 0x3FFu) >> sh);
        c[2 * (4 * d + s) + 1] = (uint8_t)(((h[s] >> 16) & 0x3FFu) >> sh);
      }
    }
  } else if constexpr (FMT == QGEMV_FMT_UNIFORM && BITS == 3) {
    const int shk[5] = {0, 3, 6, 0, 3};
#pragma unroll
    for (int d = 0; d < 3; ++d) {
      uint32_t h[5];
      u3_slots(w[d], h);
#pragma unroll
      for (int s = 0; s < 5; ++s) {
        c[2 * (5 * d + s)] = (uint8_t)((h[s] & 0x3FFu) >> shk[s]);
        c[2 * (5 * d + s) + 1] = (uint8_t)(((h[s] >> 16) & 0x3FFu) >> shk[s]);
      }
    }
    const uint32_t hs = u3_spare(w[0], w[1], w[2]);
    c[30] = (uint8_t)(hs & 0x3FFu);
    c[31] = (uint8_t)((hs >> 16) & 0x3FFu);
  } else if constexpr (BITS == 4) {
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      uint32_t sa, sb;
      l4_sel(w[d], sa, sb);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t a = (sa >> (8 * k)) & 0xFFu, bb = (sb >> (8 * k)) & 0xFFu;
        c[8 * d + k] = (uint8_t)((a & 7u) | (((a >> 6) & 1u) << 3));
        c[8 * d + 4 + k] = (uint8_t)((bb & 7u) | (((bb >> 4) & 1u) << 3));
      }
    }
  } else {
    uint32_t sel[8];
    l3_sel(w[0], w[1], w[2], sel);
#pragma unroll
    for (int q = 0; q < 8; ++q)
#pragma unroll
      for (int k = 0; k < 4; ++k) c[4 * q + k] = (uint8_t)((sel[q] >> (8 * k)) & 0xFFu);
  }
  const int k0 = b * kBlockK + 32 * (l >> 4);
  if (k0 + 32 <= K) {
    uint4 v0, v1;
    std::memcpy(&v0, c, 16);
    std::memcpy(&v1, c + 16, 16);
    uint4* dst = (uint4*)(out + (size_t)row * K + k0);
    dst[0] = v0;
    dst[1] = v1;
  } else {
    for (int j = 0; j < 32 && k0 + j < K; ++j) out[(size_t)row * K + k0 + j] = c[j];
  }
}

// ---- launch plumbing --------------------------------------------------------
constexpr int kMaxGrid = 256;   // one workgroup per CU
constexpr int kMaxTilesPerWG = 32;

int b1_grid(const BlobHeader& h) {
  int g = h.tiles < kMaxGrid ? h.tiles : kMaxGrid;
  const int need = (h.tiles + kMaxTilesPerWG - 1) / kMaxTilesPerWG;
  return g > need ? g : need;
}

size_t b1_lds_bytes(const BlobHeader& h, int grid) {
  const size_t tw = (size_t)((h.tiles + grid - 1) / grid);
  const size_t tab = h.format == QGEMV_FMT_LUT ? (size_t)(2u << h.bits) : 0;
  return (size_t)h.Kp * 2 + tw * kWaves * 16 * 4 + tw * 16 * 4 + (tw * 16 + 4) * 4 + tw * 16 * tab;
}

template <int FMT, int BITS>
hipError_t launch_b1(const qgemv_plan* p, const uint16_t* x, float* y, hipStream_t st) {
  constexpr int PF = 8, NE = 2;
  const BlobHeader& h = p->h;
  const int grid = b1_grid(h);
  const size_t lds = b1_lds_bytes(h, grid);
  static bool attr_set = false;
  if (!attr_set) {
    const hipError_t e = hipFuncSetAttribute((const void*)k_b1<FMT, BITS, PF, NE>,
                                             hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const uint32_t codes_bytes = (uint32_t)((uint64_t)h.tiles * h.nkb * h.block_bytes);
  const uint32_t meta_bytes = (uint32_t)(h.off_rowptr - h.off_meta);
  hipLaunchKernelGGL((k_b1<FMT, BITS, PF, NE>), dim3(grid), dim3(64 * kWaves), lds, st, p->blob + h.off_codes,
                     (const uint32_t*)(p->blob + h.off_meta), (const int32_t*)(p->blob + h.off_rowptr),
                     (const uint32_t*)(p->blob + h.off_entries), x, y, h.M, h.K, h.Kp, h.nkb, h.tiles, codes_bytes,
                     meta_bytes, (int)h.nnz);
  return hipGetLastError();
}

template <int FMT, int BITS>
hipError_t launch_unpack(const qgemv_plan* p, uint8_t* out, hipStream_t st) {
  const BlobHeader& h = p->h;
  const int64_t n = (int64_t)h.tiles * h.nkb * 64;
  const int blocks = (int)((n + 255) / 256);
  hipLaunchKernelGGL((k_unpack<FMT, BITS>), dim3(blocks), dim3(256), 0, st, p->blob + h.off_codes, out, h.M, h.K,
                     h.nkb, h.tiles);
  return hipGetLastError();
}

int hip_status(hipError_t e) {
  if (e == hipSuccess) return QGEMV_OK;
  qgemv_set_hip_error((int)e);
  return QGEMV_ERR_HIP;
}

}  // namespace

extern "C" {

int qgemv_create(qgemv_handle* out, const qgemv_weights* shape, const void* packed_dev, size_t bytes) {
  if (!out || !shape || !packed_dev) return QGEMV_ERR_INVALID_ARG;
  *out = nullptr;
  const int st = qgemv_validate_shape(shape);
  if (st) return st;
  if ((uintptr_t)packed_dev % kAlign) return QGEMV_ERR_INVALID_ARG;
  const BlobHeader expect =
      make_header(shape->M, shape->K, shape->bits, shape->format, shape->group_size, shape->nnz);
  if (bytes < expect.total_bytes) return QGEMV_ERR_SIZE;
  BlobHeader got;
  const hipError_t e = hipMemcpy(&got, packed_dev, sizeof(got), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_status(e);
  if (std::memcmp(&got, &expect, sizeof(got)) != 0) return QGEMV_ERR_SIZE;
  qgemv_plan* p = new (std::nothrow) qgemv_plan{expect, (const uint8_t*)packed_dev};
  if (!p) return QGEMV_ERR_INVALID_ARG;
  *out = p;
  return QGEMV_OK;
}

int qgemv_run(qgemv_handle h, const void* x_dev, float* y_dev, int32_t batch, void* stream) {
  if (!h || !x_dev || !y_dev) return QGEMV_ERR_INVALID_ARG;
  if ((uintptr_t)x_dev % 16 || (uintptr_t)y_dev % 16) return QGEMV_ERR_INVALID_ARG;
  if (batch != 1 && batch != 8 && batch != 16) return QGEMV_ERR_UNSUPPORTED;
  if (batch != 1) return QGEMV_ERR_UNSUPPORTED;
  const hipStream_t st = (hipStream_t)stream;
  const uint16_t* x = (const uint16_t*)x_dev;
  hipError_t e;
  if (h->h.format == QGEMV_FMT_LUT)
    e = h->h.bits == 4 ? launch_b1<QGEMV_FMT_LUT, 4>(h, x, y_dev, st) : launch_b1<QGEMV_FMT_LUT, 3>(h, x, y_dev, st);
  else
    e = h->h.bits == 4 ? launch_b1<QGEMV_FMT_UNIFORM, 4>(h, x, y_dev, st)
                       : launch_b1<QGEMV_FMT_UNIFORM, 3>(h, x, y_dev, st);
  return hip_status(e);
}

int qgemv_debug_unpack(qgemv_handle h, uint8_t* codes_dev, void* stream) {
  if (!h || !codes_dev) return QGEMV_ERR_INVALID_ARG;
  if ((uintptr_t)codes_dev % 16) return QGEMV_ERR_INVALID_ARG;
  const hipStream_t st = (hipStream_t)stream;
  hipError_t e;
  if (h->h.format == QGEMV_FMT_LUT)
    e = h->h.bits == 4 ? launch_unpack<QGEMV_FMT_LUT, 4>(h, codes_dev, st)
                       : launch_unpack<QGEMV_FMT_LUT, 3>(h, codes_dev, st);
  else
    e = h->h.bits == 4 ? launch_unpack<QGEMV_FMT_UNIFORM, 4>(h, codes_dev, st)
                       : launch_unpack<QGEMV_FMT_UNIFORM, 3>(h, codes_dev, st);
  return hip_status(e);
}

int qgemv_destroy(qgemv_handle h) {
  delete h;
  return QGEMV_OK;
}

}  // extern "C"
