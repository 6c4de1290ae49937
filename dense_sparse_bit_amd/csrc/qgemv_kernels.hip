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
// partial sums for the finished tile in LDS.
//
// The outliers of the workgroup's rows are one contiguous run of CSR entries.
// Right after the prologue the waves copy that run (up to the LDS space left)
// from HBM straight into LDS with buffer-to-LDS loads, which complete in the
// background while the dense stream runs.  After the stream each wave sums
// the outliers of its rows from LDS, and the partials of every row are added
// in a fixed order: the output is deterministic.
// ---------------------------------------------------------------------------
constexpr int kWaves = 16;
constexpr uint32_t kVmcntZero = 0x0F70;  // s_waitcnt vmcnt(0), no wait on the other counters

template <int FMT, int BITS, int PF>
__global__ void __launch_bounds__(64 * kWaves)
k_b1(const uint8_t* __restrict__ codes, const uint32_t* __restrict__ meta, const int32_t* __restrict__ row_ptr,
     const uint32_t* __restrict__ entries, const uint16_t* __restrict__ x, float* __restrict__ y, int M, int K,
     int Kp, int nkb, int tiles, uint32_t codes_bytes, uint32_t meta_bytes, int nnz, int ent_cap) {
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
  //      | CSR entries [ent_cap]
  uint16_t* x_lds = (uint16_t*)lds;
  float* part = (float*)(lds + Kp / 2);
  float* csr = part + TW * kWaves * 16;
  int* rp_lds = (int*)(csr + TW * 16);
  uint32_t* lut_lds = (uint32_t*)(rp_lds + TW * 16 + 4);  // 16-byte aligned
  uint32_t* ent_lds = lut_lds + (F::lut ? TW * 16 * F::tab_dw : 0);

  const rsrc_t rc = make_rsrc(codes, codes_bytes);
  const rsrc_t rs = make_rsrc(meta, F::lut ? 0u : meta_bytes);
  const rsrc_t re = make_rsrc(entries, (uint32_t)nnz * 4);

  // Prologue: the code ring, then x, the row_ptr slice and the tables; all of
  // them are in flight together.
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
  const int E0 = row_ptr[T0 * 16];            // outliers of the workgroup: entries [E0, E1)
  const int E1 = row_ptr[T0 * 16 + nrows];
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

  // CSR entries [A0, A0 + ent_cap) of the workgroup's run go to LDS, 1 KiB per
  // wave instruction (16 bytes per lane); issued after the barrier so that
  // nothing waits on them before the stream ends.
  const int A0 = E0 & ~3;
  const int Acap = min(E1, A0 + ent_cap);
  {
    const int pieces = (Acap - A0 + 3) >> 2;
    for (int i = w; 64 * i < pieces; i += kWaves) {
      const int piece = 64 * i + lane;
      if (piece < pieces)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(re, (__attribute__((address_space(3))) void*)(ent_lds + 256 * i), 16,
                                                 (A0 + 4 * piece) * 4, 0, 0, 0);
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

  // Outliers: entries of the LDS run come from LDS, any beyond it from HBM.
  __builtin_amdgcn_s_waitcnt(kVmcntZero);
  __syncthreads();
  for (int r = w; r < nrows; r += kWaves) {
    const int p1 = rp_lds[r + 1];
    float sum = 0.f;
    for (int p = rp_lds[r] + lane; p < p1; p += 64) {
      const uint32_t e = p < Acap ? ent_lds[p - A0] : entries[p];
      sum = dot2(e >> 16, (uint32_t)x_lds[e & 0xFFFFu], sum);
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

// ---------------------------------------------------------------------------
// Batch 8 / 16.  The dequantized tile is the A operand and the activations
// are the B operand of the same 16x16x32 MFMA: column n of the product is
// batch row n, so one MFMA serves the whole batch (columns n >= batch read
// zeros).  One workgroup owns one tile; its waves split the tile's K-blocks.
// x is 4 KiB per K-block at batch 16 and comes from L2 through the register
// ring, next to the codes of the same K-block.  The dense kernel writes y;
// the outliers are added by k_csr_bn on the same stream.
// ---------------------------------------------------------------------------
template <int FMT, int BITS, int PF>
__global__ void __launch_bounds__(64 * kWaves)
k_bn(const uint8_t* __restrict__ codes, const uint32_t* __restrict__ meta, const uint16_t* __restrict__ x,
     float* __restrict__ y, int M, int K, int nkb, uint32_t codes_bytes, uint32_t meta_bytes, int B) {
  using F = Fmt<FMT, BITS>;
  constexpr int BB = 256 * BITS;
  __shared__ float part[kWaves][256];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nw = blockDim.x >> 6;
  const int t = blockIdx.x;
  const int b0 = w * nkb / nw, b1 = (w + 1) * nkb / nw;  // this wave's K-blocks of tile t
  const int g0 = t * nkb + b0, g1 = t * nkb + b1;

  const rsrc_t rc = make_rsrc(codes, codes_bytes);
  const rsrc_t rs = make_rsrc(meta, F::lut ? 0u : meta_bytes);
  const rsrc_t rx = make_rsrc(x, (uint32_t)B * (uint32_t)K * 2u);
  const uint32_t voff = (uint32_t)lane * 4 * BITS;
  const uint32_t soff = (uint32_t)lane * 8;
  const int n = lane & 15;
  // B operand of lane (n, q = lane / 16) for K-block kb: x[n][128 kb + 32 q .. +31], 64 bytes.
  const uint32_t xrow = n < B ? (uint32_t)n * (uint32_t)K * 2u + 64u * (uint32_t)(lane >> 4) : kOutOfRange;
  auto xoff = [&](int kb) -> uint32_t {
    return (xrow != kOutOfRange && 128 * kb + 32 * (lane >> 4) < K) ? xrow + 256u * (uint32_t)kb : kOutOfRange;
  };

  uint32_t cb[PF][BITS];
  uint32_t sb[PF][2];
  u32x4_t xr[PF][4];
  auto issue = [&](int u, int g) {
    const bool in = g < g1;
    load_chunk<BITS>(cb[u], rc, in ? (uint32_t)g * BB + voff : kOutOfRange);
    if constexpr (!F::lut) load_stats(sb[u], rs, in ? (uint32_t)g * 512 + soff : kOutOfRange);
    const uint32_t xo = in ? xoff(g - t * nkb) : kOutOfRange;
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2)
      xr[u][s2] = __builtin_amdgcn_raw_buffer_load_b128(rx, (int)(xo == kOutOfRange ? kOutOfRange : xo + 16u * s2), 0, 0);
  };
#pragma unroll
  for (int u = 0; u < PF; ++u) {
    if constexpr (F::lut) sb[u][0] = sb[u][1] = 0;
    issue(u, g0 + u);
  }
  uint32_t tab[F::tab_dw];
  if constexpr (F::lut) {
    const rsrc_t rl = make_rsrc(meta, meta_bytes);
    const uint32_t off = ((uint32_t)t * 16 + (lane & 15)) * (F::tab_dw * 4);
    uint32_t L[F::tab_dw];
    const u32x4_t v0 = __builtin_amdgcn_raw_buffer_load_b128(rl, (int)off, 0, 0);
    L[0] = v0[0]; L[1] = v0[1]; L[2] = v0[2]; L[3] = v0[3];
    if constexpr (BITS == 4) {
      const u32x4_t v1 = __builtin_amdgcn_raw_buffer_load_b128(rl, (int)(off + 16), 0, 0);
      L[4] = v1[0]; L[5] = v1[1]; L[6] = v1[2]; L[7] = v1[3];
      l4_planes(L, tab);
    } else {
      l3_planes(L, tab);
    }
  } else {
    tab[0] = 0;
  }

  floatx4_t acc = {0.f, 0.f, 0.f, 0.f};
  for (int gi = g0; gi < g1; gi += PF) {
#pragma unroll
    for (int u = 0; u < PF; ++u) {
      const int g = gi + u;
      if (g < g1) {
        uint32_t am[F::n_mfma][4];
        decode_chunk<FMT, BITS>(cb[u], sb[u], tab, am);
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) {
          const half8_t bx = __builtin_bit_cast(half8_t, xr[u][s2]);
          acc = mfma(h8(am[s2][0], am[s2][1], am[s2][2], am[s2][3]), bx, acc);
          if constexpr (!F::lut) acc = mfma(h8(am[4 + s2][0], am[4 + s2][1], am[4 + s2][2], am[4 + s2][3]), bx, acc);
        }
      }
      issue(u, g + PF);
    }
  }
  // acc: row 4*(lane/16) + r, batch column lane % 16
#pragma unroll
  for (int r = 0; r < 4; ++r) part[w][(4 * (lane >> 4) + r) * 16 + n] = acc[r];
  __syncthreads();
  for (int i = threadIdx.x; i < 256; i += blockDim.x) {
    const int m = i >> 4, c = i & 15, row = 16 * t + m;
    if (c < B && row < M) {
      float v = 0.f;
      for (int ww = 0; ww < nw; ++ww) v += part[ww][i];
      y[(size_t)c * M + row] = v;
    }
  }
}

// Outliers at batch 8 / 16: y[n][r] += sum_p value_p * x[n][col_p].  A
// workgroup owns a run of rows.  x is staged transposed in LDS, KC columns at
// a time, so one entry meets all batch rows in one place; lane (n, slot) of a
// wave takes batch row n of entry slot.  Every y element is updated by exactly
// one lane, after the dense kernel on the same stream: no atomics, fixed order.
template <int NB>
__global__ void __launch_bounds__(256)
k_csr_bn(const int32_t* __restrict__ row_ptr, const uint32_t* __restrict__ entries, const uint16_t* __restrict__ x,
         float* __restrict__ y, int M, int K, int B, int rows_per_wg, int KC) {
  constexpr int SL = 64 / NB;           // entry slots per wave instruction
  constexpr int kRowsPerWave = 8;
  extern __shared__ uint16_t xT[];      // [KC][NB]
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int n = lane % NB, sl = lane / NB;
  const int R0 = blockIdx.x * rows_per_wg;
  const int R1 = min(M, R0 + rows_per_wg);
  float acc[kRowsPerWave];
#pragma unroll
  for (int j = 0; j < kRowsPerWave; ++j) acc[j] = 0.f;
  for (int c0 = 0; c0 < K; c0 += KC) {
    const int kc = min(KC, K - c0);
    __syncthreads();
    for (int i = threadIdx.x; i < kc * NB; i += blockDim.x) {
      const int nn = i / kc, k = i - nn * kc;  // read x row-wise, write transposed
      xT[k * NB + nn] = nn < B ? x[(size_t)nn * K + c0 + k] : (uint16_t)0;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kRowsPerWave; ++j) {
      const int r = R0 + w + 4 * j;
      if (r < R1) {
        const int p1 = row_ptr[r + 1];
        for (int p = row_ptr[r] + sl; p < p1; p += SL) {
          const uint32_t e = entries[p];
          const int col = (int)(e & 0xFFFFu) - c0;
          if (col >= 0 && col < kc) acc[j] = dot2(e >> 16, (uint32_t)xT[col * NB + n], acc[j]);
        }
      }
    }
  }
#pragma unroll
  for (int j = 0; j < kRowsPerWave; ++j) {
    float v = acc[j];
    for (int o = NB; o < 64; o <<= 1) v += __shfl_xor(v, o);
    const int r = R0 + w + 4 * j;
    if (sl == 0 && r < R1 && n < B) y[(size_t)n * M + r] += v;
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

constexpr size_t kLdsBytes = 160 * 1024;
constexpr size_t kEntCapBytes = 64 * 1024;  // CSR entries staged per workgroup
constexpr size_t kCsrStageBytes = 64 * 1024;  // transposed x per staging pass of k_csr_bn

// LDS of everything but the staged CSR entries.
size_t b1_lds_fixed(const BlobHeader& h, int grid) {
  const size_t tw = (size_t)((h.tiles + grid - 1) / grid);
  const size_t tab = h.format == QGEMV_FMT_LUT ? (size_t)(2u << h.bits) : 0;
  return (size_t)h.Kp * 2 + tw * kWaves * 16 * 4 + tw * 16 * 4 + (tw * 16 + 4) * 4 + tw * 16 * tab;
}

template <int FMT, int BITS>
hipError_t launch_b1(const qgemv_plan* p, const uint16_t* x, float* y, hipStream_t st) {
  constexpr int PF = 8;
  const BlobHeader& h = p->h;
  const int grid = b1_grid(h);
  const size_t fixed = b1_lds_fixed(h, grid);
  size_t cap = kLdsBytes - fixed;
  if (cap > kEntCapBytes) cap = kEntCapBytes;
  cap &= ~(size_t)1023;  // whole 1 KiB wave loads
  static bool attr_set = false;
  if (!attr_set) {
    const hipError_t e = hipFuncSetAttribute((const void*)k_b1<FMT, BITS, PF>,
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsBytes);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const uint32_t codes_bytes = (uint32_t)((uint64_t)h.tiles * h.nkb * h.block_bytes);
  const uint32_t meta_bytes = (uint32_t)(h.off_rowptr - h.off_meta);
  hipLaunchKernelGGL((k_b1<FMT, BITS, PF>), dim3(grid), dim3(64 * kWaves), fixed + cap, st, p->blob + h.off_codes,
                     (const uint32_t*)(p->blob + h.off_meta), (const int32_t*)(p->blob + h.off_rowptr),
                     (const uint32_t*)(p->blob + h.off_entries), x, y, h.M, h.K, h.Kp, h.nkb, h.tiles, codes_bytes,
                     meta_bytes, (int)h.nnz, (int)(cap / 4));
  return hipGetLastError();
}

template <int FMT, int BITS>
hipError_t launch_bn(const qgemv_plan* p, const uint16_t* x, float* y, int B, hipStream_t st) {
  constexpr int PF = 3;
  const BlobHeader& h = p->h;
  int waves = h.nkb / 4;  // at least 4 K-blocks per wave
  waves = waves < 1 ? 1 : (waves > kWaves ? kWaves : waves);
  const uint32_t codes_bytes = (uint32_t)((uint64_t)h.tiles * h.nkb * h.block_bytes);
  const uint32_t meta_bytes = (uint32_t)(h.off_rowptr - h.off_meta);
  hipLaunchKernelGGL((k_bn<FMT, BITS, PF>), dim3(h.tiles), dim3(64 * waves), 0, st, p->blob + h.off_codes,
                     (const uint32_t*)(p->blob + h.off_meta), x, y, h.M, h.K, h.nkb, codes_bytes, meta_bytes, B);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || h.nnz == 0) return e;
  const int rows_per_wg = 4 * 8;  // 4 waves x 8 rows
  const int grid = (h.M + rows_per_wg - 1) / rows_per_wg;
  const int nb = B <= 8 ? 8 : 16;
  const int KC = (int)(kCsrStageBytes / (2 * nb));
  const size_t lds = (size_t)(KC < h.K ? KC : h.K) * nb * 2;
  const int32_t* rp = (const int32_t*)(p->blob + h.off_rowptr);
  const uint32_t* ent = (const uint32_t*)(p->blob + h.off_entries);
  if (nb == 8)
    hipLaunchKernelGGL((k_csr_bn<8>), dim3(grid), dim3(256), lds, st, rp, ent, x, y, h.M, h.K, B, rows_per_wg, KC);
  else
    hipLaunchKernelGGL((k_csr_bn<16>), dim3(grid), dim3(256), lds, st, rp, ent, x, y, h.M, h.K, B, rows_per_wg, KC);
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
  const hipStream_t st = (hipStream_t)stream;
  const uint16_t* x = (const uint16_t*)x_dev;
  const bool lut = h->h.format == QGEMV_FMT_LUT, b4 = h->h.bits == 4;
  hipError_t e;
  if (batch == 1) {
    if (lut) e = b4 ? launch_b1<QGEMV_FMT_LUT, 4>(h, x, y_dev, st) : launch_b1<QGEMV_FMT_LUT, 3>(h, x, y_dev, st);
    else e = b4 ? launch_b1<QGEMV_FMT_UNIFORM, 4>(h, x, y_dev, st) : launch_b1<QGEMV_FMT_UNIFORM, 3>(h, x, y_dev, st);
  } else {
    if (lut)
      e = b4 ? launch_bn<QGEMV_FMT_LUT, 4>(h, x, y_dev, batch, st) : launch_bn<QGEMV_FMT_LUT, 3>(h, x, y_dev, batch, st);
    else
      e = b4 ? launch_bn<QGEMV_FMT_UNIFORM, 4>(h, x, y_dev, batch, st)
             : launch_bn<QGEMV_FMT_UNIFORM, 3>(h, x, y_dev, batch, st);
  }
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
