// qgemv_kernels.hip -- gfx950 kernels and the device side of the C ABI.
//
// Batch-1 product (the hot path): one wave64 per output row at a time.
//   * Lane l of wave step s owns the 32-code chunk 64*s + l of the row, so a
//     wave step reads 64 contiguous chunks (768 B for 3-bit, 1 KiB for 4-bit)
//     with one 96/128-bit load per lane.  Every code byte is read once.
//   * The lane's 32 activations per step live in VGPRs for the whole kernel;
//     a copy of x in LDS serves the gathers of the outlier SpMV.
//   * Codes become FP16 pairs (magic-number OR for uniform codes, v_perm byte
//     lookups for LUT codes) and meet x in v_dot2_f32_f16 (fp32 accumulate).
//   * The row's CSR entries (prefetched with its codes) add into the same
//     fp32 partial; a DPP wave sum gives y[i], written once, no atomics.
//   * Each wave walks a contiguous block of rows with a ring of PF row buffers
//     in registers, so the loads of row r+PF are in flight while row r computes.

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

constexpr int kWavesPerBlock = 4;
constexpr int kBlock = kWavesPerBlock * 64;

__device__ __forceinline__ uint32_t hsplat_neg_sum(uint32_t z_bits, float base) {
  // FP16 pair (-(base + z), -(base + z)); exact for the small integers used here.
  const _Float16 z = __builtin_bit_cast(_Float16, (uint16_t)z_bits);
  const _Float16 c = (_Float16)(-base) - z;
  const uint16_t b = __builtin_bit_cast(uint16_t, c);
  return (uint32_t)b | ((uint32_t)b << 16);
}

// (1024 + k*q) pair -> (q - z) pair, exactly: h * (1/k) + (-(1024/k) - z).
__device__ __forceinline__ uint32_t to_qz(uint32_t h, uint32_t c, _Float16 inv_k) {
  const half2_t r = as_h2(h) * (half2_t){inv_k, inv_k} + as_h2(c);
  return as_u32(r);
}

__device__ __forceinline__ float h_lo_to_f(uint32_t v) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(v & 0xFFFFu));
}

template <int FMT, int BITS>
struct MetaDw {
  static constexpr int n = FMT == QGEMV_FMT_LUT ? (BITS == 4 ? 8 : 4) : 2;  // per lane per step for uniform
};

template <int FMT, int BITS, int S, int NE>
struct RowBuf {
  uint32_t c[S][BITS];                     // code dwords
  uint32_t m[FMT == QGEMV_FMT_LUT ? 1 : S][MetaDw<FMT, BITS>::n];  // LUT planes or group stats
  uint32_t e[NE];                          // CSR entries (col | value << 16)
  int p0, cnt;
};

template <int FMT, int BITS, int S, int NE>
__device__ __forceinline__ void issue_row(RowBuf<FMT, BITS, S, NE>& b, int r, int lane, int last_lanes,
                                          const uint8_t* __restrict__ codes,
                                          const uint32_t* __restrict__ meta,
                                          const uint32_t* __restrict__ entries, int row_bytes,
                                          int meta_row_dw, int p0, int p1) {
  const uint8_t* rowc = codes + (size_t)r * row_bytes;
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const int ch = s * 64 + lane;
    const bool act = (s < S - 1) || (lane < last_lanes);
    if constexpr (BITS == 4) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (act) v = *(const uint4*)(rowc + (size_t)ch * 16);
      b.c[s][0] = v.x; b.c[s][1] = v.y; b.c[s][2] = v.z; b.c[s][3] = v.w;
    } else {
      uint3 v = make_uint3(0, 0, 0);
      if (act) v = *(const uint3*)(rowc + (size_t)ch * 12);
      b.c[s][0] = v.x; b.c[s][1] = v.y; b.c[s][2] = v.z;
    }
    if constexpr (FMT == QGEMV_FMT_UNIFORM) {
      uint2 v = make_uint2(0, 0);
      if (act) v = *(const uint2*)(meta + (size_t)r * meta_row_dw + 2 * ch);
      b.m[s][0] = v.x; b.m[s][1] = v.y;
    }
  }
  if constexpr (FMT == QGEMV_FMT_LUT) {
    const uint4* mt = (const uint4*)(meta + (size_t)r * meta_row_dw);
    const uint4 a = mt[0];
    b.m[0][0] = a.x; b.m[0][1] = a.y; b.m[0][2] = a.z; b.m[0][3] = a.w;
    if constexpr (BITS == 4) {
      const uint4 c = mt[1];
      b.m[0][4] = c.x; b.m[0][5] = c.y; b.m[0][6] = c.z; b.m[0][7] = c.w;
    }
  }
  b.p0 = p0;
  b.cnt = p1 - p0;
#pragma unroll
  for (int k = 0; k < NE; ++k) {
    b.e[k] = 0;
    if (k * 64 < b.cnt && lane + k * 64 < b.cnt) b.e[k] = entries[p0 + k * 64 + lane];
  }
}

// Dense part of one row: sum over the lane's chunks of d * x.
template <int FMT, int BITS, int S, int NE>
__device__ __forceinline__ float dense_row(const RowBuf<FMT, BITS, S, NE>& b, const uint32_t (&xr)[S][16]) {
  float acc = 0.f;
#pragma unroll
  for (int s = 0; s < S; ++s) {
    if constexpr (FMT == QGEMV_FMT_LUT && BITS == 4) {
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        uint32_t sa, sb, p01, p23;
        l4_sel(b.c[s][d], sa, sb);
        l4_lookup(b.m[0], sa, 0x40404040u, p01, p23);
        acc = dot2(p01, xr[s][4 * d + 0], acc);
        acc = dot2(p23, xr[s][4 * d + 1], acc);
        l4_lookup(b.m[0], sb, 0x10101010u, p01, p23);
        acc = dot2(p01, xr[s][4 * d + 2], acc);
        acc = dot2(p23, xr[s][4 * d + 3], acc);
      }
    } else if constexpr (FMT == QGEMV_FMT_LUT && BITS == 3) {
      uint32_t sel[8];
      l3_sel(b.c[s][0], b.c[s][1], b.c[s][2], sel);
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        uint32_t p01, p23;
        l3_lookup(b.m[0], sel[q], p01, p23);
        acc = dot2(p01, xr[s][2 * q + 0], acc);
        acc = dot2(p23, xr[s][2 * q + 1], acc);
      }
    } else if constexpr (BITS == 4) {  // uniform, 4 bit
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        const uint32_t st = b.m[s][g];
        const uint32_t c1 = hsplat_neg_sum(st >> 16, 1024.f), c16 = hsplat_neg_sum(st >> 16, 64.f);
        float ga = 0.f;
#pragma unroll
        for (int dd = 0; dd < 2; ++dd) {
          const int d = 2 * g + dd;
          uint32_t h[4];
          u4_slots(b.c[s][d], h);
          ga = dot2(to_qz(h[0], c1, (_Float16)1.0f), xr[s][4 * d + 0], ga);
          ga = dot2(to_qz(h[1], c16, (_Float16)0.0625f), xr[s][4 * d + 1], ga);
          ga = dot2(to_qz(h[2], c1, (_Float16)1.0f), xr[s][4 * d + 2], ga);
          ga = dot2(to_qz(h[3], c16, (_Float16)0.0625f), xr[s][4 * d + 3], ga);
        }
        acc = fmaf(h_lo_to_f(st), ga, acc);
      }
    } else {  // uniform, 3 bit
      uint32_t h[3][5];
      u3_slots(b.c[s][0], h[0]);
      u3_slots(b.c[s][1], h[1]);
      u3_slots(b.c[s][2], h[2]);
      const uint32_t hs = u3_spare(b.c[s][0], b.c[s][1], b.c[s][2]);
      const _Float16 ik[5] = {(_Float16)1.0f, (_Float16)0.125f, (_Float16)0.015625f, (_Float16)1.0f,
                              (_Float16)0.125f};
      const float kb[5] = {1024.f, 128.f, 16.f, 1024.f, 128.f};
      float ga[2] = {0.f, 0.f};
      uint32_t cz[2][3];
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        const uint32_t zb = b.m[s][g] >> 16;
        cz[g][0] = hsplat_neg_sum(zb, 1024.f);
        cz[g][1] = hsplat_neg_sum(zb, 128.f);
        cz[g][2] = hsplat_neg_sum(zb, 16.f);
      }
      (void)kb;
#pragma unroll
      for (int d = 0; d < 3; ++d) {
#pragma unroll
        for (int t = 0; t < 5; ++t) {
          const int m = 5 * d + t;
          const int g = m < 8 ? 0 : 1;
          const int ci = (t == 0 || t == 3) ? 0 : (t == 2 ? 2 : 1);
          ga[g] = dot2(to_qz(h[d][t], cz[g][ci], ik[t]), xr[s][m], ga[g]);
        }
      }
      ga[1] = dot2(to_qz(hs, cz[1][0], (_Float16)1.0f), xr[s][15], ga[1]);
      acc = fmaf(h_lo_to_f(b.m[s][0]), ga[0], acc);
      acc = fmaf(h_lo_to_f(b.m[s][1]), ga[1], acc);
    }
  }
  return acc;
}

template <int FMT, int BITS, int S, int PF, int NE>
__global__ void __launch_bounds__(kBlock)
k_gemv_b1(const uint8_t* __restrict__ codes, const uint32_t* __restrict__ meta,
          const int32_t* __restrict__ row_ptr, const uint32_t* __restrict__ entries,
          const uint16_t* __restrict__ x, float* __restrict__ y, int M, int K, int row_bytes,
          int meta_row_dw, int last_lanes, int nwaves) {
  extern __shared__ uint32_t lds[];
  uint16_t* x_lds = (uint16_t*)lds;
  int32_t* rp_lds = (int32_t*)(lds + K / 2);

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6));
  const int wb0 = blockIdx.x * kWavesPerBlock;
  const int wb1 = min(nwaves, wb0 + kWavesPerBlock);
  const int rb0 = (int)((int64_t)wb0 * M / nwaves);
  const int rb1 = (int)((int64_t)wb1 * M / nwaves);
  const bool has_rows = wave < nwaves;
  const int r0 = has_rows ? (int)((int64_t)wave * M / nwaves) : 0;
  const int r1 = has_rows ? (int)((int64_t)(wave + 1) * M / nwaves) : 0;

  // Codes and metadata of the first PF rows: issued before anything else.
  RowBuf<FMT, BITS, S, NE> buf[PF];
#pragma unroll
  for (int u = 0; u < PF; ++u)
    if (r0 + u < r1) issue_row(buf[u], r0 + u, lane, last_lanes, codes, meta, entries, row_bytes, meta_row_dw, 0, 0);

  // Stage x and this block's row_ptr slice in LDS.
  for (int i = threadIdx.x; i < K / 8; i += kBlock) ((uint4*)x_lds)[i] = ((const uint4*)x)[i];
  for (int i = threadIdx.x; i <= rb1 - rb0; i += kBlock) rp_lds[i] = row_ptr[rb0 + i];

  // The lane's activations, as FP16 pairs, for all steps.
  uint32_t xr[S][16];
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const int ch = s * 64 + lane;
    const bool act = (s < S - 1) || (lane < last_lanes);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (act) v = ((const uint4*)(x + (size_t)ch * 32))[q];
      xr[s][4 * q + 0] = v.x; xr[s][4 * q + 1] = v.y; xr[s][4 * q + 2] = v.z; xr[s][4 * q + 3] = v.w;
    }
  }
  __syncthreads();
  if (!has_rows) return;

  // CSR entries of the first PF rows.
#pragma unroll
  for (int u = 0; u < PF; ++u) {
    const int r = r0 + u;
    if (r < r1) {
      const int p0 = __builtin_amdgcn_readfirstlane(rp_lds[r - rb0]);
      const int p1 = __builtin_amdgcn_readfirstlane(rp_lds[r - rb0 + 1]);
      buf[u].p0 = p0;
      buf[u].cnt = p1 - p0;
#pragma unroll
      for (int k = 0; k < NE; ++k) {
        buf[u].e[k] = 0;
        if (k * 64 < buf[u].cnt && lane + k * 64 < buf[u].cnt) buf[u].e[k] = entries[p0 + k * 64 + lane];
      }
    }
  }

  for (int base = r0; base < r1; base += PF) {
#pragma unroll
    for (int u = 0; u < PF; ++u) {
      const int r = base + u;
      if (r < r1) {
        float acc = dense_row<FMT, BITS, S, NE>(buf[u], xr);
        // outliers of this row
        const int cnt = buf[u].cnt;
#pragma unroll
        for (int k = 0; k < NE; ++k) {
          if (k * 64 < cnt && lane + k * 64 < cnt) {
            const uint32_t e = buf[u].e[k];
            acc = dot2(e >> 16, (uint32_t)x_lds[e & 0xFFFFu], acc);
          }
        }
        for (int k = NE; k * 64 < cnt; ++k) {
          if (lane + k * 64 < cnt) {
            const uint32_t e = entries[buf[u].p0 + k * 64 + lane];
            acc = dot2(e >> 16, (uint32_t)x_lds[e & 0xFFFFu], acc);
          }
        }
        const float tot = wave_sum(acc);
        if (lane == 0) y[r] = tot;
        // refill this buffer with row r + PF
        const int rn = r + PF;
        if (rn < r1) {
          const int p0 = __builtin_amdgcn_readfirstlane(rp_lds[rn - rb0]);
          const int p1 = __builtin_amdgcn_readfirstlane(rp_lds[rn - rb0 + 1]);
          issue_row(buf[u], rn, lane, last_lanes, codes, meta, entries, row_bytes, meta_row_dw, p0, p1);
        }
      }
    }
  }
}

// Debug: decode the blob's codes back to canonical order, one thread per 32-code chunk.
template <int FMT, int BITS>
__global__ void __launch_bounds__(kBlock)
k_unpack(const uint8_t* __restrict__ codes, uint8_t* __restrict__ out, int M, int K, int row_bytes) {
  const int chunks = K / 32;
  const int64_t idx = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  if (idx >= (int64_t)M * chunks) return;
  const int r = (int)(idx / chunks), ch = (int)(idx % chunks);
  const uint32_t* src = (const uint32_t*)(codes + (size_t)r * row_bytes + (size_t)ch * 4 * BITS);
  uint32_t w[4] = {0, 0, 0, 0};
#pragma unroll
  for (int d = 0; d < BITS; ++d) w[d] = src[d];
  uint8_t c[32];
  if constexpr (FMT == QGEMV_FMT_UNIFORM && BITS == 4) {
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      uint32_t h[4];
      u4_slots(w[d], h);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int sh = (t & 1) ? 4 : 0;
        c[2 * (4 * d + t)] = (uint8_t)((h[t] & 0x3FFu) >> sh);
        c[2 * (4 * d + t) + 1] = (uint8_t)(((h[t] >> 16) & 0x3FFu) >> sh);
      }
    }
  } else if constexpr (FMT == QGEMV_FMT_UNIFORM && BITS == 3) {
    const int shk[5] = {0, 3, 6, 0, 3};
#pragma unroll
    for (int d = 0; d < 3; ++d) {
      uint32_t h[5];
      u3_slots(w[d], h);
#pragma unroll
      for (int t = 0; t < 5; ++t) {
        c[2 * (5 * d + t)] = (uint8_t)((h[t] & 0x3FFu) >> shk[t]);
        c[2 * (5 * d + t) + 1] = (uint8_t)(((h[t] >> 16) & 0x3FFu) >> shk[t]);
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
        const uint32_t a = (sa >> (8 * k)) & 0xFFu, b = (sb >> (8 * k)) & 0xFFu;
        c[8 * d + k] = (uint8_t)((a & 7u) | (((a >> 6) & 1u) << 3));
        c[8 * d + 4 + k] = (uint8_t)((b & 7u) | (((b >> 4) & 1u) << 3));
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
  uint4* dst = (uint4*)(out + (size_t)r * K + (size_t)ch * 32);
  uint4 v0, v1;
  std::memcpy(&v0, c, 16);
  std::memcpy(&v1, c + 16, 16);
  dst[0] = v0;
  dst[1] = v1;
}

// ---- launch plumbing --------------------------------------------------------
struct LaunchShape {
  int nwaves, blocks, lds_bytes;
};

LaunchShape b1_shape(const BlobHeader& h, int waves_per_cu) {
  const int target = 256 * waves_per_cu;
  LaunchShape s;
  s.nwaves = h.M < target ? h.M : target;
  s.blocks = (s.nwaves + kWavesPerBlock - 1) / kWavesPerBlock;
  const int rows_per_wave = (h.M + s.nwaves - 1) / s.nwaves;
  s.lds_bytes = h.K * 2 + 4 * (rows_per_wave * kWavesPerBlock + 2);
  return s;
}

template <int FMT, int BITS, int S>
hipError_t launch_b1(const qgemv_plan* p, const uint16_t* x, float* y, hipStream_t st) {
  constexpr int PF = S <= 2 ? 3 : 2;
  constexpr int NE = S <= 2 ? 2 : 5;
  constexpr int WPC = S <= 2 ? 16 : 8;
  const BlobHeader& h = p->h;
  const LaunchShape ls = b1_shape(h, WPC);
  const int last_lanes = (h.K - (h.steps - 1) * kStepCodes) / kChunkCodes;
  hipLaunchKernelGGL((k_gemv_b1<FMT, BITS, S, PF, NE>), dim3(ls.blocks), dim3(kBlock), ls.lds_bytes, st,
                     p->blob + h.off_codes, (const uint32_t*)(p->blob + h.off_meta),
                     (const int32_t*)(p->blob + h.off_rowptr), (const uint32_t*)(p->blob + h.off_entries), x,
                     y, h.M, h.K, (int)h.row_bytes, (int)(h.meta_row_bytes / 4), last_lanes, ls.nwaves);
  return hipGetLastError();
}

template <int FMT, int BITS>
hipError_t launch_b1_steps(const qgemv_plan* p, const uint16_t* x, float* y, hipStream_t st) {
  switch (p->h.steps) {
    case 1: return launch_b1<FMT, BITS, 1>(p, x, y, st);
    case 2: return launch_b1<FMT, BITS, 2>(p, x, y, st);
    case 3: return launch_b1<FMT, BITS, 3>(p, x, y, st);
    case 4: return launch_b1<FMT, BITS, 4>(p, x, y, st);
    case 5: return launch_b1<FMT, BITS, 5>(p, x, y, st);
    case 6: return launch_b1<FMT, BITS, 6>(p, x, y, st);
    case 7: return launch_b1<FMT, BITS, 7>(p, x, y, st);
    case 8: return launch_b1<FMT, BITS, 8>(p, x, y, st);
    default: return hipErrorInvalidValue;
  }
}

template <int FMT, int BITS>
hipError_t launch_unpack(const qgemv_plan* p, uint8_t* out, hipStream_t st) {
  const BlobHeader& h = p->h;
  const int64_t n = (int64_t)h.M * (h.K / 32);
  const int blocks = (int)((n + kBlock - 1) / kBlock);
  hipLaunchKernelGGL((k_unpack<FMT, BITS>), dim3(blocks), dim3(kBlock), 0, st, p->blob + h.off_codes, out, h.M,
                     h.K, (int)h.row_bytes);
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
    e = h->h.bits == 4 ? launch_b1_steps<QGEMV_FMT_LUT, 4>(h, x, y_dev, st)
                       : launch_b1_steps<QGEMV_FMT_LUT, 3>(h, x, y_dev, st);
  else
    e = h->h.bits == 4 ? launch_b1_steps<QGEMV_FMT_UNIFORM, 4>(h, x, y_dev, st)
                       : launch_b1_steps<QGEMV_FMT_UNIFORM, 3>(h, x, y_dev, st);
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
