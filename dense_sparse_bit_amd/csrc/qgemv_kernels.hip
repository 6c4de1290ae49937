// qgemv_kernels.hip -- gfx950 kernels and the device side of the C ABI.
//
// The product runs on 16-row tiles (the M side of a 16x16x32 MFMA) and
// K-blocks of 128 codes.  Every kernel runs one workgroup of 16 waves per CU;
// a workgroup owns a contiguous range of tiles, whose (tile, K-block) pairs are
// one contiguous stretch of the blob.
//   * k_stream: batch 1, and batch 8 / 16 when x does not fit in LDS.  The
//     waves take chunks of consecutive K-blocks in order from an LDS counter;
//     each lane streams the 32-code chunk of its row (16 B or 12 B per
//     K-block, 1 KiB / 768 B contiguous per wave load) through a register
//     ring, turns it into FP16 A operands (v_perm byte lookups in the row's
//     table for LUT codes; exact (q - z) values for uniform codes) and issues
//     16x16x32 MFMAs with fp32 accumulation.  Batch 1 reads x from LDS;
//     batch 8 / 16 loads it from L2 next to the codes.
//   * k_xlds: batch 8 / 16 with x resident in LDS for the whole launch.
// The CSR outliers of a workgroup's rows are copied into LDS while the dense
// stream runs and gathered against x in LDS; every output is written once,
// with no atomics, and partial sums meet in a fixed order, so results are
// deterministic.
//
// Uniform codes, batch 1: the MFMA columns are the eight groups of a K-block
// (x masked per column), so each group's sum of (q - z) * x comes out
// separately and its scale is applied in fp32.  Batch 8 / 16: the group scale
// s is split into s_hi (s with the four low mantissa bits cleared) and
// s_lo = s - s_hi; (q - z) * s_hi and (q - z) * s_lo are exact in FP16, so two
// MFMAs reproduce s * (q - z) * x without rounding the decoded weight.

#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>
#include <mutex>
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
  int device;             // the device of the blob (current at create)
  void* ws = nullptr;     // workspace of the K-split batched kernel, allocated by the first batched run
  size_t ws_bytes = 0;
  std::mutex ws_mu;
};

// Workspace of qgemv_run_noalloc, for callers that cannot allocate device
// memory: one static array per device, zero at load, held until the process
// ends.  Host code uses only the address hipGetSymbolAddress returns for it
// on each device (g_scratch_dev), never the array's name.
constexpr size_t kScratchBytes = (size_t)16 << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

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
  static constexpr bool bpdq = FMT == QGEMV_FMT_BPDQ;  // 3-bit codes in the L3 placement
  static constexpr int tab_dw = lut ? (BITS == 4 ? 8 : 4) : 1;
  static constexpr int n_mfma = lut ? 4 : 8;   // per K-block, split-scale decode
};

// Uniform codes of one lane chunk as exact FP16 pairs (q - z): pair m holds
// chunk codes 2m, 2m+1.  zw holds the zero points of the chunk's two groups
// (codes 0-15 and 16-31) in its low and high half.
template <int BITS>
__device__ __forceinline__ void uniform_qz(const uint32_t (&c)[BITS], uint32_t zw, uint32_t (&qz)[16]) {
  uint32_t cz[2][3];
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    const uint32_t zb = g ? zw >> 16 : zw & 0xFFFFu;
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
      for (int t = 0; t < 4; ++t)
        qz[4 * d + t] = (t & 1) ? to_qz(h[t], cz[g][1], (_Float16)0.0625f) : to_qz(h[t], cz[g][0], (_Float16)1.0f);
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
      if (m == 15) {
        qz[m] = to_qz(hs, cz[g][0], (_Float16)1.0f);
      } else {
        const int d = m / 5, t = m % 5;
        if (t == 0 || t == 3) qz[m] = to_qz(h[d][t], cz[g][0], (_Float16)1.0f);
        else if (t == 2) qz[m] = to_qz(h[d][t], cz[g][2], (_Float16)0.015625f);
        else qz[m] = to_qz(h[d][t], cz[g][1], (_Float16)0.125f);
      }
    }
  }
}

// Decode one lane chunk into MFMA A operands.
//   LUT:     a[i][0..3] for step i = 0..3
//   UNIFORM: a[i] = s_hi * (q - z), a[4 + i] = s_lo * (q - z); st[g] = scale | zero << 16 of group g
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
  } else if constexpr (FMT == QGEMV_FMT_BPDQ) {
    // st = C0 | C1 << 16, C2 | C3 << 16: the chunk's group.  The 8 levels
    // C0 + C1 b0 + C2 b1 + C3 b2 are formed in fp32 and split into an FP16
    // part and the FP16 rest; both tables go through the 3-bit lookups, the
    // parts to a[0..3] and the rests to a[4..7] (two MFMAs per step).
    const float c0 = (float)__builtin_bit_cast(_Float16, (uint16_t)st[0]);
    const float c1 = (float)__builtin_bit_cast(_Float16, (uint16_t)(st[0] >> 16));
    const float c2 = (float)__builtin_bit_cast(_Float16, (uint16_t)st[1]);
    const float c3 = (float)__builtin_bit_cast(_Float16, (uint16_t)(st[1] >> 16));
    float L[8];
    L[0] = c0;
    L[1] = c0 + c1;
    L[2] = c0 + c2;
    L[3] = L[1] + c2;
    L[4] = c0 + c3;
    L[5] = L[1] + c3;
    L[6] = L[2] + c3;
    L[7] = L[3] + c3;
    uint32_t hi[4], lo[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const _Float16 h0 = (_Float16)L[2 * e], h1 = (_Float16)L[2 * e + 1];
      const _Float16 r0 = (_Float16)(L[2 * e] - (float)h0), r1 = (_Float16)(L[2 * e + 1] - (float)h1);
      hi[e] = (uint32_t)__builtin_bit_cast(uint16_t, h0) | ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
      lo[e] = (uint32_t)__builtin_bit_cast(uint16_t, r0) | ((uint32_t)__builtin_bit_cast(uint16_t, r1) << 16);
    }
    uint32_t th[4], tl[4];
    l3_planes(hi, th);
    l3_planes(lo, tl);
    uint32_t sel[8];
    l3_sel(c[0], c[1], c[2], sel);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      l3_lookup(th, sel[q], a[q / 2][2 * (q % 2)], a[q / 2][2 * (q % 2) + 1]);
      l3_lookup(tl, sel[q], a[4 + q / 2][2 * (q % 2)], a[4 + q / 2][2 * (q % 2) + 1]);
    }
  } else {
    uint32_t qz[16], shi[2], slo[2];
    uniform_qz<BITS>(c, (st[0] >> 16) | (st[1] & 0xFFFF0000u), qz);
    scale_split(st[0], shi[0], slo[0]);
    scale_split(st[1], shi[1], slo[1]);
#pragma unroll
    for (int m = 0; m < 16; ++m) {
      const int g = m < 8 ? 0 : 1;
      a[m / 4][m % 4] = hmul(qz[m], shi[g]);
      a[4 + m / 4][m % 4] = hmul(qz[m], slo[g]);
    }
  }
}

typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRsrcWord3 = 0x00020000;  // raw buffer, 32-bit data format

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kRsrcWord3);
}

// Cache policy of loads whose bytes are read once (codes, statistics,
// tables, CSR entries): non-temporal, which streams measurably faster from
// HBM than the default policy.  x, which every workgroup reads, keeps the
// default.
constexpr int kNonTemporal = 2;

// Loads through a range-checked buffer resource: offsets past the range read 0 and touch no memory.
template <int BITS>
__device__ __forceinline__ void load_chunk(uint32_t (&c)[BITS], rsrc_t r, uint32_t off) {
  if constexpr (BITS == 4) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kNonTemporal);
    c[0] = v[0]; c[1] = v[1]; c[2] = v[2]; c[3] = v[3];
  } else {
    const auto v = __builtin_amdgcn_raw_buffer_load_b96(r, (int)off, 0, kNonTemporal);
    c[0] = v[0]; c[1] = v[1]; c[2] = v[2];
  }
}
__device__ __forceinline__ void load_stats(uint32_t (&s)[2], rsrc_t r, uint32_t off) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, kNonTemporal);
  s[0] = v[0];
  s[1] = v[1];
}

constexpr uint32_t kOutOfRange = 0x7FFFFFF0u;

// LDS fetch-and-add whose wait sits in the same asm block.  Written out
// because the compiler, not knowing which LDS bytes an in-flight
// buffer-to-LDS copy writes, would otherwise drain every global load before
// an LDS atomic.
__device__ __forceinline__ int lds_fetch_add(int* p, int v) {
  const uint32_t addr = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) int*)p;
  int r;
  asm volatile("ds_add_rtn_u32 %0, %1, %2\n\ts_waitcnt lgkmcnt(0)" : "=v"(r) : "v"(addr), "v"(v) : "memory");
  return r;
}

// Plain LDS read and write of a flag another wave updates, addressed as LDS
// (a volatile generic pointer would become a flat access, whose wait also
// drains the wave's global loads).
__device__ __forceinline__ int lds_read_flag(const int* p) {
  const uint32_t addr = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const int*)p;
  int r;
  asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(r) : "v"(addr) : "memory");
  return r;
}
__device__ __forceinline__ void lds_write_flag(int* p, int v) {
  const uint32_t addr = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) int*)p;
  asm volatile("ds_write_b32 %0, %1" : : "v"(addr), "v"(v) : "memory");
}

// Workgroup barrier that orders LDS only: outstanding global loads keep
// running across it (a plain __syncthreads() would wait for them).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// ---------------------------------------------------------------------------
// The streaming kernel.  One workgroup of 16 waves per CU owns the contiguous
// tile range [T0, T1); its (tile, K-block) pairs, tile-major, are one
// contiguous stretch of the blob.  The waves take that stretch in chunks of
// PF consecutive K-blocks of one tile, in order, from an LDS counter, and
// stream each chunk through a ring of PF register slots (the next chunk's
// loads are issued as the current one is consumed).  Every chunk writes its
// partial sums to its own LDS slot; after the stream the slots of every output
// are added in chunk order, so the output does not depend on which wave took
// which chunk.
//
// Batch 1 (NB = 1): x sits in LDS and every lane reads its B operand from
// there (the same x in all 16 MFMA columns).  The outliers of the
// workgroup's rows are one contiguous run of CSR entries; after its first
// chunk each wave copies its share of that run (up to the LDS space left)
// from HBM straight into LDS with buffer-to-LDS loads, which land while the
// dense stream runs.  After the stream 16 lanes per row add the row's
// outliers and its chunk partials.
//
// Batch 8 / 16 (NB = batch), used when x does not fit in LDS: column n of the
// MFMA is batch row n.  x is 2 KiB or 4 KiB per K-block and comes from L2
// through the ring, next to the codes of the same K-block; partials are kept
// per batch column.  The outliers go through the MFMAs too: the ring also
// loads the outliers of each block (grouped by block in the blob), the wave
// scatters them into its own zeroed 16x128 FP16 tile in LDS, reads the tile
// back as four A operands and multiplies them with the block's x already in
// registers, then clears what it wrote.
// ---------------------------------------------------------------------------
constexpr int kWaves = 16;
constexpr uint32_t kVmcntZero = 0x0F70;  // s_waitcnt vmcnt(0), no wait on the other counters

template <int FMT, int BITS, int CH, int NR, int NB, bool XST>
__global__ void __launch_bounds__(64 * kWaves)
k_stream(const uint8_t* __restrict__ codes, const uint32_t* __restrict__ meta, const int32_t* __restrict__ row_ptr,
         const uint32_t* __restrict__ entries, const int32_t* __restrict__ boff, const uint32_t* __restrict__ bent,
         const uint16_t* __restrict__ x, float* __restrict__ y, int M, int K, int Kp, int nkb, int tiles,
         uint32_t codes_bytes, uint32_t meta_bytes, int nnz, int ent_cap, int gsz) {
  using F = Fmt<FMT, BITS>;
  constexpr int BB = 256 * BITS;
  constexpr bool B1 = NB == 1;
  constexpr int PF = CH * NR;  // ring slots: NR chunks of CH K-blocks in flight per wave
  static_assert(B1 || NR == 1, "batch NB keeps one chunk in flight");
  extern __shared__ uint32_t lds[];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int T0 = (int)((int64_t)blockIdx.x * tiles / gridDim.x);
  const int T1 = (int)((int64_t)(blockIdx.x + 1) * tiles / gridDim.x);
  const int TW = T1 - T0;
  // Each tile's K-blocks are cut into CPT chunks of up to CH consecutive
  // blocks; chunk q of the workgroup is chunk q % CPT of tile T0 + q / CPT.
  // The waves take chunks in order from an LDS counter: a wave that runs ahead
  // takes more, so all waves end together and the workgroup sweeps its stretch
  // of the blob front to back.  A wave keeps NR chunks in flight.  Each
  // chunk's partial sums go to the chunk's own LDS slot, so the result does
  // not depend on which wave took what.
  const int CPT = (nkb + CH - 1) / CH;
  const int nchunks = TW * CPT;
  // Chunk q: tile T0 + q / CPT, K-blocks kb0 .. kb0 + nv - 1, blob block index g0 of the first.
  struct Chunk {
    int q, t, kb0, g0, nv;
  };
  // Batch NB: each workgroup starts its tiles' K sweep at its own chunk, so
  // that the workgroups do not all read the same x lines from L2 at once.
  const int rot = B1 ? 0 : (int)(blockIdx.x % (unsigned)CPT);
  auto chunk_at = [&](int q) -> Chunk {
    Chunk k;
    k.q = q;
    k.t = q / CPT;
    int j = q - k.t * CPT + rot;
    if (j >= CPT) j -= CPT;
    k.kb0 = j * CH;
    k.g0 = (T0 + k.t) * nkb + k.kb0;
    k.nv = q < nchunks ? min(CH, nkb - k.kb0) : 0;
    return k;
  };
  const int nrows = min(TW * 16, M - T0 * 16);  // real rows of the workgroup

  // LDS, batch 1:  x [Kp+8] fp16 | part [TW*CPT][16] | row_ptr [TW*16+4] | LUT [TW*16][tab_dw] | CSR entries [ent_cap]
  //      batch NB: part [TW*CPT][16][NB] | block offsets [TW*nkb+1, padded] | LUT | outlier tiles [16 waves][16][128] FP16
  // (the counters sit in spare slots at the end of the row_ptr / offsets region)
  uint16_t* x_lds = (uint16_t*)lds;  // batch 1: x, then 16 zero bytes
  float* part = (float*)(lds + (B1 ? Kp / 2 + 4 : 0));
  int* rp_lds = (int*)(part + nchunks * 16 * NB);
  const int rp_n = B1 ? TW * 16 + 4 : ((TW * nkb + 6) & ~3);
  uint32_t* lut_lds = (uint32_t*)(rp_lds + rp_n);  // 16-byte aligned
  uint32_t* ent_lds = lut_lds + (F::lut ? TW * 16 * F::tab_dw : 0);  // batch 1
  uint16_t* otile = (uint16_t*)ent_lds + 2048 * w;  // batch NB: this wave's outlier tile, A-operand order
  // Batch NB with XST: this wave's x stage, [16 batch rows][16 pieces of 8
  // columns] FP16, piece c of row r at slot c ^ r, so that the row-contiguous
  // stores and the B-operand reads both spread over all banks.
  uint16_t* xstage = (uint16_t*)ent_lds + 2048 * (kWaves + w);

  const rsrc_t rc = make_rsrc(codes, codes_bytes);
  const rsrc_t rs = make_rsrc(meta, F::lut ? 0u : meta_bytes);
  const rsrc_t rx = make_rsrc(x, (uint32_t)NB * (uint32_t)K * 2u);

  // B operand of lane (n, q) = (lane % 16, lane / 16) for K-block kb, batch NB:
  // x[n][128 kb + 32 q .. +31], 64 bytes.
  const uint32_t xrow = (lane & 15) < NB ? (uint32_t)(lane & 15) * (uint32_t)K * 2u + 64u * (uint32_t)(lane >> 4)
                                         : kOutOfRange;
  const int xq = 32 * (lane >> 4);

  // Prologue: the ring first, then what goes to LDS; all of it is in flight together.
  const uint32_t voff = (uint32_t)lane * 4 * BITS;
  // Uniform statistics of a K-block (see qgemv_layout.h): the z pair of the
  // lane's two groups, and either the s pair (split-scale decode, batch NB) or
  // the scales of group lane % 16 for rows 4*(lane/16) .. +3 (batch 1).
  constexpr bool UG1 = B1 && FMT == QGEMV_FMT_UNIFORM;  // batch-1 uniform: MFMA columns are the K-block's groups
  constexpr int SBW = UG1 ? 5 : 2;
  const uint32_t zoff = (uint32_t)(lane & 15) * 16 + (uint32_t)(lane >> 4) * 4;
  const uint32_t spoff = 256 + (uint32_t)(lane >> 4) * 64 + (uint32_t)(lane & 15) * 4;
  const uint32_t sqoff = (lane & 15) < 8 ? 256 + (uint32_t)((lane & 15) >> 1) * 64 + (uint32_t)(lane >> 4) * 16
                                         : kOutOfRange;
  // BPDQ coefficients of a K-block: [16 rows][128/gsz groups][4] FP16; lane
  // (row lane % 16, columns 32*(lane/16) .. +31) takes its group's 8 bytes.
  const uint32_t cunit = 16384u / (uint32_t)gsz;
  const uint32_t coff = ((uint32_t)(lane & 15) * (128u / (uint32_t)gsz) + (uint32_t)(32 * (lane >> 4)) / (uint32_t)gsz) * 8u;
  // What goes to LDS is loaded first: the x slice (batch 1), the row_ptr
  // slice and the tables, at most 2 + 1 + 1 pieces per thread.  The code
  // ring is issued right behind, so storing the staged pieces waits for them
  // alone, and the barrier below (LDS only) lets the ring loads run on: each
  // wave starts decoding as soon as its first K-block lands.
  constexpr int kThreads = 64 * kWaves;
  u32x4_t xs[2];
  if constexpr (B1) {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int i = threadIdx.x + k * kThreads;
      xs[k] = __builtin_amdgcn_raw_buffer_load_b128(rx, i < Kp / 8 ? i * 16 : (int)kOutOfRange, 0, 0);
    }
  }
  const rsrc_t rr = make_rsrc(row_ptr, (uint32_t)(M + 1) * 4);
  const int rpn = B1 && threadIdx.x <= TW * 16 ? __builtin_amdgcn_raw_buffer_load_b32(
                                                     rr, min(T0 * 16 + (int)threadIdx.x, M) * 4, 0, 0)
                                               : 0;
  // The bounds [E0, E1) of the workgroup's outliers, in lanes 0 and 1 of
  // every wave: vector loads, which the LDS barrier below does not wait for
  // (scalar loads would hold it until they return).
  const int ev = B1 && lane < 2 ? __builtin_amdgcn_raw_buffer_load_b32(rr, (T0 * 16 + (lane ? nrows : 0)) * 4, 0, 0)
                                : 0;
  // Batch NB: the outlier offsets of the workgroup's blocks, for LDS (at most
  // 4 per thread; the host keeps TW * nkb below 4096).
  const rsrc_t rbo = make_rsrc(boff, (uint32_t)((uint64_t)tiles * nkb + 1) * 4);
  int bo[4] = {0, 0, 0, 0};
  if constexpr (!B1) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int i = (int)threadIdx.x + 1024 * k;
      bo[k] = __builtin_amdgcn_raw_buffer_load_b32(rbo, i <= TW * nkb ? (T0 * nkb + i) * 4 : (int)kOutOfRange, 0, 0);
    }
  }
  u32x4_t ls = {0u, 0u, 0u, 0u};
  const int lpieces = F::lut ? TW * 16 * F::tab_dw / 4 : 0;  // 16-byte pieces of the tables
  if constexpr (F::lut) {
    const rsrc_t rl = make_rsrc(meta, meta_bytes);
    ls = __builtin_amdgcn_raw_buffer_load_b128(
        rl, (int)threadIdx.x < lpieces ? (T0 * 16 * F::tab_dw / 4 + (int)threadIdx.x) * 16 : (int)kOutOfRange, 0, kNonTemporal);
  }

  uint32_t cb[PF][BITS];
  uint32_t sb[PF][SBW];
  u32x4_t xr[B1 ? 1 : PF][4];
  // Batch NB: the outliers of each ring slot's block, one per lane (up to 64;
  // more are read when the block is decoded), and their first index and count.
  uint32_t ent[B1 ? 1 : PF];
  int elo[B1 ? 1 : PF], ecnt[B1 ? 1 : PF];
  const rsrc_t rbe = make_rsrc(bent, (uint32_t)nnz * 4);
  auto issue_ent = [&](int u, int lo, int n) {
    if constexpr (!B1) {
      ent[u] = __builtin_amdgcn_raw_buffer_load_b32(rbe, lane < n ? (lo + lane) * 4 : (int)kOutOfRange, 0, kNonTemporal);
      elo[u] = lo;
      ecnt[u] = n;
    }
  };
  auto issue = [&](int u, int g) {  // g: blob block index, -1 for none
    const bool in = g >= 0;
    load_chunk<BITS>(cb[u], rc, in ? (uint32_t)g * BB + voff : kOutOfRange);
    if constexpr (F::bpdq) {
      const u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(rs, (int)(in ? (uint32_t)g * cunit + coff : kOutOfRange),
                                                             0, kNonTemporal);
      sb[u][0] = v[0];
      sb[u][1] = v[1];
    } else if constexpr (!F::lut) {
      const uint32_t mb = in ? (uint32_t)g * 512 : kOutOfRange;
      sb[u][0] = __builtin_amdgcn_raw_buffer_load_b32(rs, (int)(in ? mb + zoff : kOutOfRange), 0, kNonTemporal);
      if constexpr (UG1) {
        const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(
            rs, (int)(in && sqoff != kOutOfRange ? mb + sqoff : kOutOfRange), 0, kNonTemporal);
        sb[u][1] = v[0]; sb[u][2] = v[1]; sb[u][3] = v[2]; sb[u][4] = v[3];
      } else {
        sb[u][1] = __builtin_amdgcn_raw_buffer_load_b32(rs, (int)(in ? mb + spoff : kOutOfRange), 0, kNonTemporal);
      }
    } else {
      sb[u][0] = sb[u][1] = 0;
    }
    if constexpr (!B1 && XST) {
      // x of the K-block, batch rows 4 s2 .. 4 s2 + 3 per instruction, 256
      // contiguous bytes each: lane l takes row 4 s2 + l / 16, columns
      // 8 (l % 16) .. +7 (rows past NB are not loaded; their MFMA columns are
      // never stored).
      const int kbl = g - (g / nkb) * nkb;
      const bool ok = in && 128 * kbl + 8 * (lane & 15) < K;
#pragma unroll
      for (int s2 = 0; s2 < NB / 4; ++s2)
        xr[u][s2] = __builtin_amdgcn_raw_buffer_load_b128(
            rx, ok ? (int)((uint32_t)(4 * s2 + (lane >> 4)) * (uint32_t)K * 2u + 256u * (uint32_t)kbl + 16u * (uint32_t)(lane & 15))
                   : (int)kOutOfRange,
            0, 0);
    } else if constexpr (!B1) {
      const int kbl = g - (g / nkb) * nkb;
      const uint32_t xo = in && xrow != kOutOfRange && 128 * kbl + xq < K ? xrow + 256u * (uint32_t)kbl : kOutOfRange;
#pragma unroll
      for (int s2 = 0; s2 < 4; ++s2)
        xr[u][s2] = __builtin_amdgcn_raw_buffer_load_b128(rx, (int)(xo == kOutOfRange ? kOutOfRange : xo + 16u * s2),
                                                          0, 0);
    }
  };
  // The first chunk of wave w goes to ring half 0 now; the others come from
  // the counter once it is set up.
  Chunk ck[NR];
  ck[0] = chunk_at(w);
#pragma unroll
  for (int u = 0; u < CH; ++u) issue(u, u < ck[0].nv ? ck[0].g0 + u : -1);

  if constexpr (B1) {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int i = threadIdx.x + k * kThreads;
      if (i < Kp / 8) ((u32x4_t*)x_lds)[i] = xs[k];
    }
    if (threadIdx.x < 4) ((uint32_t*)(x_lds + Kp))[threadIdx.x] = 0u;
  }
  if constexpr (F::lut) {
    if ((int)threadIdx.x < lpieces) ((u32x4_t*)lut_lds)[threadIdx.x] = ls;
  }
  for (int j = threadIdx.x; j < nchunks * 16 * NB; j += kThreads) part[j] = 0.f;  // chunks past a short tile end
  if constexpr (!B1) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int i = (int)threadIdx.x + 1024 * k;
      if (i <= TW * nkb) rp_lds[i] = bo[k];
    }
    const u32x4_t z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int k = 0; k < 4; ++k) ((u32x4_t*)otile)[lane + 64 * k] = z;
  }
  int* chunk_ctr = rp_lds + rp_n - 2;  // a spare slot after the row_ptr slice / block offsets
  if (threadIdx.x == 0) *chunk_ctr = kWaves;
  lds_barrier();
  // Batch NB: the outlier offsets of a chunk's blocks (lane i: block i's start, i <= nv).
  auto chunk_offsets = [&](const Chunk& k) {
    return lane <= k.nv && k.nv > 0 ? rp_lds[k.g0 - T0 * nkb + lane] : 0;
  };
  if constexpr (!B1) {
    const int obv = chunk_offsets(ck[0]);
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      const int lo = __builtin_amdgcn_readlane(obv, u);
      issue_ent(u, lo, u < ck[0].nv ? __builtin_amdgcn_readlane(obv, u + 1) - lo : 0);
    }
  }

  // Batch 1: set-up the dense stream does not need, done by each wave after
  // its first chunk (or after the stream if it had none), when the row_ptr
  // values have long arrived: the row_ptr slice goes to LDS, and the CSR
  // entries [A0, A0 + ent_cap) of the workgroup's run are copied from HBM
  // straight into LDS, 1 KiB per wave instruction (16 bytes per lane).  Both
  // are first read after the barrier that ends the stream.
  int A0 = 0, Acap = 0;
  bool late_done = false;
  auto late_setup = [&]() {
    const int E0 = __builtin_amdgcn_readlane(ev, 0), E1 = __builtin_amdgcn_readlane(ev, 1);
    A0 = E0 & ~3;
    Acap = min(E1, A0 + ent_cap);
    if ((int)threadIdx.x <= TW * 16) rp_lds[threadIdx.x] = rpn;
    const rsrc_t re = make_rsrc(entries, (uint32_t)nnz * 4);
    const int pieces = (Acap - A0 + 3) >> 2;
    for (int i = w; 64 * i < pieces; i += kWaves) {
      const int piece = 64 * i + lane;
      if (piece < pieces)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(re, (__attribute__((address_space(3))) void*)(ent_lds + 256 * i), 16,
                                                 (A0 + 4 * piece) * 4, 0, 0, kNonTemporal);
    }
    late_done = true;
  };

  auto next_chunk = [&]() -> Chunk {
    int q = 0;
    if (lane == 0) q = lds_fetch_add(chunk_ctr, 1);
    return chunk_at(__builtin_amdgcn_readfirstlane(q));
  };
#pragma unroll
  for (int r = 1; r < NR; ++r) {
    ck[r] = next_chunk();
#pragma unroll
    for (int u = 0; u < CH; ++u) issue(r * CH + u, u < ck[r].nv ? ck[r].g0 + u : -1);
  }

  int tc = -1;  // tile whose table is in tab
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

  const uint16_t* xb = x_lds + xq;
  const int jn = (lane & 15) - 2 * (lane >> 4);  // batch-1 uniform: the step pair that feeds this lane's column
  const uint32_t sh = 16u * (uint32_t)(lane & 1);
  // Chunks are taken in increasing order, so once ck[0] is past the end every
  // later one is too.
  while (ck[0].q < nchunks) {
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const Chunk cur = ck[r];
      const Chunk nx = next_chunk();
      const int obv = B1 ? 0 : chunk_offsets(nx);
      const bool live = cur.q < nchunks;
      if (live && T0 + cur.t != tc) {
        tc = T0 + cur.t;
        planes();
      }
      floatx4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int u = 0; u < CH; ++u) {
        const int kb = cur.kb0 + u;
        const int sl = r * CH + u;
        if (u < cur.nv) {
          if constexpr (UG1) {
            // Batch-1 uniform: A = exact (q - z), B = x masked so that MFMA column n
            // sees only group n of the K-block (step s2 covers groups 2*(lane/16) +
            // s2/2 in lane group lane/16).  cg[i] = sum over group lane % 16 of
            // (q - z) x for row 4*(lane/16) + i; its scale is applied in fp32.
            uint32_t qz[16];
            uniform_qz<BITS>(cb[sl], sb[sl][0], qz);
            floatx4_t cg = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s2 = 0; s2 < 4; ++s2) {
              const bool on = (s2 >> 1) == jn;
              const half8_t bx = *(const half8_t*)(on ? xb + kb * kBlockK + 8 * s2 : x_lds + Kp);
              cg = mfma(h8(qz[4 * s2], qz[4 * s2 + 1], qz[4 * s2 + 2], qz[4 * s2 + 3]), bx, cg);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const _Float16 sc = __builtin_bit_cast(_Float16, (uint16_t)(sb[sl][1 + i] >> sh));
              acc[i] += (float)sc * cg[i];
            }
          } else {
            uint32_t am[F::n_mfma][4];
            if constexpr (F::lut || F::bpdq) {
              decode_chunk<FMT, BITS>(cb[sl], sb[sl], tab, am);
            } else {
              const uint32_t st[2] = {perm(sb[sl][0], sb[sl][1], 0x05040100u),
                                      perm(sb[sl][0], sb[sl][1], 0x07060302u)};
              decode_chunk<FMT, BITS>(cb[sl], st, tab, am);
            }
            u32x4_t xb4[4];  // batch NB: the B operands of the four steps
            if constexpr (!B1 && XST) {
#pragma unroll
              for (int s2 = 0; s2 < NB / 4; ++s2) {
                const int r = 4 * s2 + (lane >> 4);
                *(u32x4_t*)(xstage + 128 * r + 8 * ((lane & 15) ^ r)) = xr[sl][s2];
              }
              const int n = lane & 15, q = lane >> 4;
#pragma unroll
              for (int s2 = 0; s2 < 4; ++s2) xb4[s2] = *(const u32x4_t*)(xstage + 128 * n + 8 * ((4 * q + s2) ^ n));
            } else if constexpr (!B1) {
#pragma unroll
              for (int s2 = 0; s2 < 4; ++s2) xb4[s2] = xr[sl][s2];
            }
#pragma unroll
            for (int s2 = 0; s2 < 4; ++s2) {
              half8_t bx;
              if constexpr (B1) bx = *(const half8_t*)(xb + kb * kBlockK + 8 * s2);
              else bx = __builtin_bit_cast(half8_t, xb4[s2]);
              acc = mfma(h8(am[s2][0], am[s2][1], am[s2][2], am[s2][3]), bx, acc);
              if constexpr (!F::lut)
                acc = mfma(h8(am[4 + s2][0], am[4 + s2][1], am[4 + s2][2], am[4 + s2][3]), bx, acc);
            }
            if constexpr (!B1) {
              // The block's outliers: scattered into the wave's (zero) 16x128
              // tile in A-operand order, read back as four A operands and
              // multiplied with the block's x like the dense codes, then
              // cleared again.
              const int n = ecnt[sl];
              if (n > 0) {
                auto place = [&](uint32_t e) {
                  const uint32_t c = e & 127u, m = (e >> 7) & 15u;
                  return (((c >> 3) & 3u) * 64u + m + 16u * (c >> 5)) * 8u + (c & 7u);
                };
                uint32_t oa = 0;
                if (lane < n) {
                  oa = place(ent[sl]);
                  otile[oa] = (uint16_t)(ent[sl] >> 16);
                }
                for (int p = 64; p < n; p += 64)  // more than 64 in the block
                  if (lane + p < n) {
                    const uint32_t e = bent[elo[sl] + p + lane];
                    otile[place(e)] = (uint16_t)(e >> 16);
                  }
#pragma unroll
                for (int s2 = 0; s2 < 4; ++s2) {
                  const u32x4_t a = ((const u32x4_t*)otile)[s2 * 64 + lane];
                  acc = mfma(h8(a[0], a[1], a[2], a[3]), __builtin_bit_cast(half8_t, xb4[s2]), acc);
                }
                if (n <= 64) {
                  if (lane < n) otile[oa] = 0;
                } else {
                  const u32x4_t z = {0u, 0u, 0u, 0u};
#pragma unroll
                  for (int k = 0; k < 4; ++k) ((u32x4_t*)otile)[lane + 64 * k] = z;
                }
              }
            }
          }
        }
        issue(sl, u < nx.nv ? nx.g0 + u : -1);
        if constexpr (!B1) {
          const int lo = __builtin_amdgcn_readlane(obv, u);
          issue_ent(sl, lo, u < nx.nv ? __builtin_amdgcn_readlane(obv, u + 1) - lo : 0);
        }
      }
      if constexpr (UG1) {  // add the 8 groups (lanes 16j + 0..7) of every row
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float v = acc[i];
          v += dpp_mov<0xB1, 0xF>(v);   // quad_perm [1,0,3,2]
          v += dpp_mov<0x4E, 0xF>(v);   // quad_perm [2,3,0,1]
          v += dpp_mov<0x141, 0xF>(v);  // row_half_mirror
          acc[i] = v;
        }
      }
      // acc[r]: row 4*(lane/16) + r of the tile, batch column lane % 16
      if (live) {
        float* sl = part + cur.q * 16 * NB;
        if constexpr (B1) {
          if ((lane & 15) == 0)
#pragma unroll
            for (int i = 0; i < 4; ++i) sl[4 * (lane >> 4) + i] = acc[i];
        } else {
          if ((lane & 15) < NB)
#pragma unroll
            for (int i = 0; i < 4; ++i) sl[(4 * (lane >> 4) + i) * NB + (lane & 15)] = acc[i];
        }
      }
      ck[r] = nx;
    }
    if constexpr (B1) {
      if (!late_done) late_setup();
    }
  }
  if constexpr (B1) {
    if (!late_done) late_setup();
  }

  // Outliers: entries of the LDS run come from LDS, any beyond it from HBM.
  __builtin_amdgcn_s_waitcnt(kVmcntZero);
  __syncthreads();
  if constexpr (B1) {
    // One DPP row of 16 lanes per output row, four rows per wave at a time.
    // Lane j of a row takes every 16th outlier of the row and every 16th of
    // the row's chunk partials (chunk order j, j + 16, ...); four DPP steps
    // add the 16 lanes, and the row's output is written at once.
    const int sl = lane & 15;
    for (int r0 = 4 * w; r0 < nrows; r0 += 4 * kWaves) {
      const int r = r0 + (lane >> 4);
      float v = 0.f;
      if (r < nrows) {
        const int p0 = rp_lds[r], p1 = rp_lds[r + 1];
        const int pm = min(p1, Acap);  // [p0, pm) is in LDS, [max(p0, Acap), p1) only in HBM
        int p = p0 + sl;
        for (; p + 48 < pm; p += 64) {  // four outliers in flight
          uint32_t e[4], xv[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) e[u] = ent_lds[p + 16 * u - A0];
#pragma unroll
          for (int u = 0; u < 4; ++u) xv[u] = x_lds[e[u] & 0xFFFFu];
#pragma unroll
          for (int u = 0; u < 4; ++u) v = dot2(e[u] >> 16, xv[u], v);
        }
        {  // the last three or fewer, read together (masked reads stay in LDS)
          uint32_t e[3], xv[3];
#pragma unroll
          for (int u = 0; u < 3; ++u) e[u] = ent_lds[p + 16 * u < pm ? p + 16 * u - A0 : 0];
#pragma unroll
          for (int u = 0; u < 3; ++u) xv[u] = x_lds[p + 16 * u < pm ? e[u] & 0xFFFFu : 0u];
#pragma unroll
          for (int u = 0; u < 3; ++u) v = p + 16 * u < pm ? dot2(e[u] >> 16, xv[u], v) : v;
        }
        for (int p = max(p0, Acap) + sl; p < p1; p += 16) {
          const uint32_t e = entries[p];
          v = dot2(e >> 16, (uint32_t)x_lds[e & 0xFFFFu], v);
        }
        const float* ps = part + (r >> 4) * CPT * 16 + (r & 15);
        for (int j = sl; j < CPT; j += 16) v += ps[j * 16];
      }
      v += dpp_mov<0xB1, 0xF>(v);   // quad_perm [1,0,3,2]
      v += dpp_mov<0x4E, 0xF>(v);   // quad_perm [2,3,0,1]
      v += dpp_mov<0x141, 0xF>(v);  // row_half_mirror
      v += dpp_mov<0x140, 0xF>(v);  // row_mirror: every lane of the row holds the sum
      if (r < nrows && sl == 0) y[T0 * 16 + r] = v;
    }
  } else {
    for (int i = threadIdx.x; i < nrows * NB; i += 64 * kWaves) {
      const int r = i / NB, n = i % NB;
      const float* pr = part + (r >> 4) * CPT * 16 * NB + (r & 15) * NB + n;
      float v = 0.f;
      for (int j = 0; j < CPT; ++j) v += pr[j * 16 * NB];
      y[(size_t)n * M + T0 * 16 + r] = v;
    }
  }
}

// ---------------------------------------------------------------------------
// Batch 8 / 16 with x resident in LDS, for shapes whose x (NB * Kp * 2 bytes)
// fits next to the partial sums.  x is copied once into LDS as
// [Kp / 8][NB][8] FP16: the eight activations of batch row n at columns
// 8j .. 8j+7 are the 16 bytes at ((j * NB) + n) * 16.  That is one MFMA B
// operand piece, so each K-step of a K-block reads its B operand with one
// 16-byte LDS load per lane, and the outlier sums read their activations from
// the same copy.
//
// The workgroup's (tile, K-block) pairs, tile-major, are cut into 16
// contiguous runs, one per wave; a wave streams its run through a ring of R
// code slots and keeps one accumulator per tile it touches.  Wave v writes its
// sums for local tile t to partial slot v + t -- distinct for every (v, t) a
// run can touch, because the runs are ordered -- and each output adds the
// slots of the waves covering its tile in wave order, then the outliers, so
// the result does not depend on timing.
// ---------------------------------------------------------------------------
template <int FMT, int BITS, int NB, int R>
__global__ void __launch_bounds__(64 * kWaves)
k_xlds(const uint8_t* __restrict__ codes, const uint32_t* __restrict__ meta, const int32_t* __restrict__ row_ptr,
       const uint32_t* __restrict__ entries, const uint16_t* __restrict__ x, float* __restrict__ y, int M, int K,
       int Kp, int nkb, int tiles, uint32_t codes_bytes, uint32_t meta_bytes, int nnz, int ent_cap, int gsz) {
  using F = Fmt<FMT, BITS>;
  constexpr int BB = 256 * BITS;
  constexpr int NP = NB / 2;
  extern __shared__ uint32_t lds[];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int T0 = (int)((int64_t)blockIdx.x * tiles / gridDim.x);
  const int T1 = (int)((int64_t)(blockIdx.x + 1) * tiles / gridDim.x);
  const int TW = T1 - T0;
  const int nrows = min(TW * 16, M - T0 * 16);
  const int L = TW * nkb;  // (tile, K-block) pairs of the workgroup
  const int b0 = w * L / kWaves, b1 = (w + 1) * L / kWaves;  // this wave's run

  // LDS: xs [Kp/8][NB][8] FP16 | slots [TW+15][16][NB] | csr [TW*16][NB] | row_ptr [TW*16+1, padded]
  //      | runs [16][2] | group counter (padded) | LUT [TW*16][tab_dw] | CSR entries [ent_cap]
  uint16_t* xs = (uint16_t*)lds;
  float* slots = (float*)(lds + Kp * NB / 2);
  float* csr = slots + (TW + 15) * 16 * NB;
  int* rp_lds = (int*)(csr + TW * 16 * NB);
  int* runs = rp_lds + ((TW * 16 + 4) & ~3);
  int* group_ctr = runs + 2 * kWaves;  // CSR row groups taken
  uint32_t* lut_lds = (uint32_t*)(group_ctr + 4);  // 16-byte aligned
  uint32_t* ent_lds = lut_lds + (F::lut ? TW * 16 * F::tab_dw : 0);

  const rsrc_t rc = make_rsrc(codes, codes_bytes);
  const rsrc_t rs = make_rsrc(meta, F::lut ? 0u : meta_bytes);
  const rsrc_t rx = make_rsrc(x, (uint32_t)NB * (uint32_t)K * 2u);
  const rsrc_t rr = make_rsrc(row_ptr, (uint32_t)(M + 1) * 4);

  // Prologue.  Small loads first (row_ptr slice, outlier bounds, tables),
  // then x and the CSR run straight into LDS, then the code ring; all of it
  // has landed before the barrier, so no LDS copy is pending in the stream.
  const int rpn = threadIdx.x <= TW * 16 ? __builtin_amdgcn_raw_buffer_load_b32(
                                               rr, min(T0 * 16 + (int)threadIdx.x, M) * 4, 0, 0)
                                         : 0;
  const int ev = lane < 2 ? __builtin_amdgcn_raw_buffer_load_b32(rr, (T0 * 16 + (lane ? nrows : 0)) * 4, 0, 0) : 0;
  u32x4_t ls = {0u, 0u, 0u, 0u};
  const int lpieces = F::lut ? TW * 16 * F::tab_dw / 4 : 0;
  if constexpr (F::lut) {
    const rsrc_t rl = make_rsrc(meta, meta_bytes);
    ls = __builtin_amdgcn_raw_buffer_load_b128(
        rl, (int)threadIdx.x < lpieces ? (T0 * 16 * F::tab_dw / 4 + (int)threadIdx.x) * 16 : (int)kOutOfRange, 0,
        kNonTemporal);
  }
  // x: LDS piece i (16 bytes) is (j, n) = (i / NB, i % NB); columns past K read as 0.
  const int xpieces = Kp / 8 * NB;  // a multiple of 64
  for (int i = w; 64 * i < xpieces; i += kWaves) {
    const int piece = 64 * i + lane;
    const int j = piece / NB, n = piece % NB;
    const int off = 8 * j < K ? (n * K + 8 * j) * 2 : (int)kOutOfRange;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (__attribute__((address_space(3))) void*)(xs + 512 * i), 16, off, 0,
                                             0, 0);
  }
  const int E0 = __builtin_amdgcn_readlane(ev, 0), E1 = __builtin_amdgcn_readlane(ev, 1);
  const int A0 = E0 & ~3;  // entries [A0, Acap) of the workgroup's run are copied into LDS
  const int Acap = min(E1, A0 + ent_cap);
  {
    const rsrc_t re = make_rsrc(entries, (uint32_t)nnz * 4);
    const int pieces = (Acap - A0 + 3) >> 2;
    for (int i = w; 64 * i < pieces; i += kWaves) {
      const int piece = 64 * i + lane;
      if (piece < pieces)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(re, (__attribute__((address_space(3))) void*)(ent_lds + 256 * i), 16,
                                                 (A0 + 4 * piece) * 4, 0, 0, kNonTemporal);
    }
  }

  const uint32_t voff = (uint32_t)lane * 4 * BITS;
  const uint32_t zoff = (uint32_t)(lane & 15) * 16 + (uint32_t)(lane >> 4) * 4;
  const uint32_t spoff = 256 + (uint32_t)(lane >> 4) * 64 + (uint32_t)(lane & 15) * 4;
  const uint32_t cunit = 16384u / (uint32_t)gsz;  // BPDQ coefficients, as in k_stream
  const uint32_t coff = ((uint32_t)(lane & 15) * (128u / (uint32_t)gsz) + (uint32_t)(32 * (lane >> 4)) / (uint32_t)gsz) * 8u;
  uint32_t cb[R][BITS];
  uint32_t sb[R][2];
  auto issue = [&](int u, int b) {  // b: block of the workgroup, -1 for none
    const bool in = b >= 0;
    const uint32_t g = (uint32_t)(T0 * nkb + b);
    load_chunk<BITS>(cb[u], rc, in ? g * BB + voff : kOutOfRange);
    if constexpr (F::bpdq) {
      const u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(rs, (int)(in ? g * cunit + coff : kOutOfRange), 0,
                                                             kNonTemporal);
      sb[u][0] = v[0];
      sb[u][1] = v[1];
    } else if constexpr (!F::lut) {
      sb[u][0] = __builtin_amdgcn_raw_buffer_load_b32(rs, (int)(in ? g * 512 + zoff : kOutOfRange), 0, kNonTemporal);
      sb[u][1] = __builtin_amdgcn_raw_buffer_load_b32(rs, (int)(in ? g * 512 + spoff : kOutOfRange), 0, kNonTemporal);
    } else {
      sb[u][0] = sb[u][1] = 0;
    }
  };
  // x, the tables and the CSR run land before the code ring is issued, so
  // that they do not queue behind every CU's ring at the start.
  __builtin_amdgcn_s_waitcnt(kVmcntZero);
#pragma unroll
  for (int u = 0; u < R; ++u) issue(u, b0 + u < b1 ? b0 + u : -1);

  if ((int)threadIdx.x <= TW * 16) rp_lds[threadIdx.x] = rpn;
  if constexpr (F::lut) {
    if ((int)threadIdx.x < lpieces) ((u32x4_t*)lut_lds)[threadIdx.x] = ls;
  }
  if (threadIdx.x < kWaves) {  // tiles touched by each wave's run: [first, last], empty if first > last
    const int v = threadIdx.x;
    const int c0 = v * L / kWaves, c1 = (v + 1) * L / kWaves;
    runs[2 * v] = c1 > c0 ? c0 / nkb : 1;
    runs[2 * v + 1] = c1 > c0 ? (c1 - 1) / nkb : 0;
  }
  if (threadIdx.x == 0) *group_ctr = 0;
  __syncthreads();

  // The stream: this wave's run, tile by tile.
  int tl = b0 / nkb, kb = b0 - tl * nkb;  // local tile and K-block of the next block
  uint32_t tab[F::tab_dw];
  auto planes = [&]() {
    if constexpr (F::lut) {
      const uint32_t* Lt = lut_lds + (tl * 16 + (lane & 15)) * F::tab_dw;
      uint32_t Lr[F::tab_dw];
#pragma unroll
      for (int i = 0; i < F::tab_dw; ++i) Lr[i] = Lt[i];
      if constexpr (BITS == 4) l4_planes(Lr, tab);
      else l3_planes(Lr, tab);
    } else {
      tab[0] = 0;
    }
  };
  floatx4_t acc = {0.f, 0.f, 0.f, 0.f};
  auto flush = [&]() {  // acc[i]: row 4*(lane/16) + i of local tile tl, batch column lane % 16
    float* d = slots + (w + tl) * 16 * NB;
    if ((lane & 15) < NB)
#pragma unroll
      for (int i = 0; i < 4; ++i) d[(4 * (lane >> 4) + i) * NB + (lane & 15)] = acc[i];
  };
  if (b0 < b1) planes();
  const uint16_t* xb = xs + (4 * (lane >> 4) * NB + ((lane & 15) & (NB - 1))) * 8;
  for (int bb = b0; bb < b1; bb += R) {
#pragma unroll
    for (int u = 0; u < R; ++u) {
      const bool live = bb + u < b1;
      if (live) {
        if (kb == nkb) {
          flush();
          acc = (floatx4_t){0.f, 0.f, 0.f, 0.f};
          ++tl;
          kb = 0;
          planes();
        }
        uint32_t am[F::n_mfma][4];
        if constexpr (F::lut || F::bpdq) {
          decode_chunk<FMT, BITS>(cb[u], sb[u], tab, am);
        } else {
          const uint32_t st[2] = {perm(sb[u][0], sb[u][1], 0x05040100u), perm(sb[u][0], sb[u][1], 0x07060302u)};
          decode_chunk<FMT, BITS>(cb[u], st, tab, am);
        }
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) {
          const half8_t bx = *(const half8_t*)(xb + (16 * kb + s2) * NB * 8);
          acc = mfma(h8(am[s2][0], am[s2][1], am[s2][2], am[s2][3]), bx, acc);
          if constexpr (!F::lut) acc = mfma(h8(am[4 + s2][0], am[4 + s2][1], am[4 + s2][2], am[4 + s2][3]), bx, acc);
        }
        ++kb;
      }
      // Unconditional, so that every slot has the same loads behind it and
      // the waits stay per slot (a load past the run is out of range).
      issue(u, bb + u + R < b1 ? bb + u + R : -1);
    }
  }
  if (b0 < b1) flush();

  // Outliers, before the barrier: the waves that finish their runs first
  // (the arbiter favours older waves) take groups of four CSR rows from an
  // LDS counter.  Each DPP row of 16 lanes takes one CSR row; a lane takes
  // every 16th outlier of its row, reads the NB activations of the outlier's
  // column from xs and keeps NB partial sums, which four DPP steps add up
  // across the 16 lanes.  A row's sum is the same whichever wave takes it.
  {
    const int sl = lane & 15, rq = lane >> 4;
    for (;;) {
      int g = 0;
      if (lane == 0) g = lds_fetch_add(group_ctr, 1);
      g = __builtin_amdgcn_readfirstlane(g);
      if (4 * g >= nrows) break;
      const int r = 4 * g + rq;
      const bool real = r < nrows;
      const int p0 = real ? rp_lds[r] : 0, p1 = real ? rp_lds[r + 1] : 0;
      const int pm = min(p1, Acap);  // [p0, pm) is in LDS, [max(p0, Acap), p1) only in HBM
      float an[NB];
#pragma unroll
      for (int j = 0; j < NB; ++j) an[j] = 0.f;
      auto term = [&](uint32_t e) {
        const int c = (int)(e & 0xFFFFu);
        const uint16_t* xc = xs + (c >> 3) * NB * 8 + (c & 7);
        const uint32_t vlo = e >> 16, vhi = e & 0xFFFF0000u;
#pragma unroll
        for (int j = 0; j < NP; ++j) {
          const uint32_t pr = (uint32_t)xc[16 * j] | ((uint32_t)xc[16 * j + 8] << 16);
          an[2 * j] = dot2(vlo, pr, an[2 * j]);
          an[2 * j + 1] = dot2(vhi, pr, an[2 * j + 1]);
        }
      };
      for (int p = p0 + sl; p < pm; p += 16) term(ent_lds[p - A0]);
      int p = max(p0, Acap) + sl;
      for (; p + 48 < p1; p += 64) {  // four outliers from HBM in flight
        uint32_t e[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) e[u] = entries[p + 16 * u];
#pragma unroll
        for (int u = 0; u < 4; ++u) term(e[u]);
      }
      for (; p < p1; p += 16) term(entries[p]);
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        float v = an[j];
        v += dpp_mov<0xB1, 0xF>(v);   // quad_perm [1,0,3,2]
        v += dpp_mov<0x4E, 0xF>(v);   // quad_perm [2,3,0,1]
        v += dpp_mov<0x141, 0xF>(v);  // row_half_mirror
        v += dpp_mov<0x140, 0xF>(v);  // row_mirror: every lane of the row holds the sum
        an[j] = v;
      }
      if (real && sl == 0)
#pragma unroll
        for (int j = 0; j < NB; ++j) csr[r * NB + j] = an[j];
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < nrows * NB; i += 64 * kWaves) {
    const int r = i / NB, n = i % NB, t = r >> 4;
    // Every slot is read before the first add (slots past the runs are in
    // bounds and dropped by the select), so the reads overlap instead of
    // waiting one by one inside a branch.
    float s[kWaves];
#pragma unroll
    for (int u = 0; u < kWaves; ++u) s[u] = slots[((u + t) * 16 + (r & 15)) * NB + n];
    float v = 0.f;
#pragma unroll
    for (int u = 0; u < kWaves; ++u) v = runs[2 * u] <= t && t <= runs[2 * u + 1] ? v + s[u] : v;
    y[(size_t)n * M + T0 * 16 + r] = v + csr[i];
  }
}

// ---------------------------------------------------------------------------
// Batch 8 / 16 with K split across workgroups.
//
// At batch 8 and 16 one K-block of x (NB x 128 FP16: 2 or 4 KiB) outweighs
// the codes of a (tile, K-block) (768 B or 1 KiB), so a workgroup that owns
// whole tiles pulls all of x through its CU for only a few tiles.  Here
// workgroup b owns the tiles of group b % NG and the K-blocks [kb0, kb1) of
// split b / NG (S splits of the K-blocks): it copies its x slice once into LDS
// ([pieces of 8 columns][NB][8] FP16, one MFMA B-operand piece per 16 bytes)
// and uses it for all of its tiles.  Block indices go round-robin over the
// eight XCDs, so with NG a multiple of 8 the S workgroups of a group (block
// indices gi + NG s) run on one XCD.
//
// Inside the workgroup the waves take chunks of CH K-blocks of one tile in
// order from an LDS counter, as in k_stream, and each chunk writes its own
// partial slot.  The outliers of each (tile, K-block) go through the MFMAs
// with the block, as in k_stream: loaded from the block-grouped copy next to
// the codes, scattered into the wave's zeroed 16x128 FP16 tile in LDS, read
// back as four A operands and multiplied with the block's x.  Each output of
// the group then adds its tile's chunks in order.  The S splits meet in the
// workspace: each writes its [rows][NB] partial, and the last to arrive (a
// counter per group) adds the S partials in split order and writes y, so the
// result does not depend on timing.  Each arrival adds 8 / S to the counter,
// so the counter is a multiple of 8 between launches whatever plans used it,
// and the arrival that reaches the next multiple is the last: nothing needs
// clearing.
// ---------------------------------------------------------------------------
template <int FMT, int BITS, int NB, int CH>
__global__ void __launch_bounds__(64 * kWaves)
k_split(const uint8_t* __restrict__ codes, const uint32_t* __restrict__ meta, const int32_t* __restrict__ boff,
        const uint32_t* __restrict__ bent, const uint16_t* __restrict__ x, float* __restrict__ y,
        float* __restrict__ wpart, uint32_t* __restrict__ wctr, int M, int K, int nkb, int tiles,
        uint32_t codes_bytes, uint32_t meta_bytes, int nnz, int gsz, int S, int NG) {
  using F = Fmt<FMT, BITS>;
  constexpr int BB = 256 * BITS;
  extern __shared__ uint32_t lds[];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int gi = (int)(blockIdx.x % (unsigned)NG), si = (int)(blockIdx.x / (unsigned)NG);
  const int T0 = (int)((int64_t)gi * tiles / NG), T1 = (int)((int64_t)(gi + 1) * tiles / NG);
  const int TW = T1 - T0;
  const int kb0 = si * nkb / S, kb1 = (si + 1) * nkb / S, KB = kb1 - kb0;
  const int CPT = (KB + CH - 1) / CH;  // chunks per tile
  const int nchunks = TW * CPT;
  const int nrows = min(TW * 16, M - T0 * 16);
  const int OB = (KB + 4) & ~3;  // block outlier offsets staged per tile (KB + 1, padded)

  // LDS: xs [KB*16][NB][8] FP16 | part [nchunks][16][NB] | offsets [TW][OB] | counter, flag (4 ints)
  //      | LUT [TW*16][tab_dw] | outlier tiles [16 waves][16][128] FP16
  uint16_t* xs = (uint16_t*)lds;
  float* part = (float*)(lds + KB * 64 * NB);
  int* bo_lds = (int*)(part + nchunks * 16 * NB);
  int* chunk_ctr = bo_lds + TW * OB;
  int* last_flag = chunk_ctr + 1;
  uint32_t* lut_lds = (uint32_t*)(chunk_ctr + 4);  // 16-byte aligned
  uint16_t* otile = (uint16_t*)(lut_lds + (F::lut ? TW * 16 * F::tab_dw : 0)) + 2048 * w;

  const rsrc_t rc = make_rsrc(codes, codes_bytes);
  const rsrc_t rs = make_rsrc(meta, F::lut ? 0u : meta_bytes);
  const rsrc_t rx = make_rsrc(x, (uint32_t)NB * (uint32_t)K * 2u);
  const rsrc_t rbo = make_rsrc(boff, (uint32_t)((uint64_t)tiles * nkb + 1) * 4);
  const rsrc_t rbe = make_rsrc(bent, (uint32_t)nnz * 4);

  // Prologue: the block outlier offsets and the tables, then the x slice
  // straight into LDS, then the first chunk's code loads (below).
  int bo[2] = {0, 0};  // offsets of (local tile, block) pairs tid and tid + 1024
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int i = (int)threadIdx.x + 1024 * k, t = i / OB, j = i - t * OB;
    bo[k] = __builtin_amdgcn_raw_buffer_load_b32(
        rbo, t < TW && j <= KB ? ((T0 + t) * nkb + kb0 + j) * 4 : (int)kOutOfRange, 0, 0);
  }
  u32x4_t ls = {0u, 0u, 0u, 0u};
  const int lpieces = F::lut ? TW * 16 * F::tab_dw / 4 : 0;
  if constexpr (F::lut) {
    const rsrc_t rl = make_rsrc(meta, meta_bytes);
    ls = __builtin_amdgcn_raw_buffer_load_b128(
        rl, (int)threadIdx.x < lpieces ? (T0 * 16 * F::tab_dw / 4 + (int)threadIdx.x) * 16 : (int)kOutOfRange, 0,
        kNonTemporal);
  }
  const int xpieces = KB * 16 * NB;  // a multiple of 64
  for (int i = w; 64 * i < xpieces; i += kWaves) {
    const int piece = 64 * i + lane;
    const int j = piece / NB, n = piece % NB;
    const int col = kb0 * kBlockK + 8 * j;
    const int off = col < K ? (n * K + col) * 2 : (int)kOutOfRange;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (__attribute__((address_space(3))) void*)(xs + 512 * i), 16, off, 0,
                                             0, 0);
  }

  const uint32_t voff = (uint32_t)lane * 4 * BITS;
  const uint32_t zoff = (uint32_t)(lane & 15) * 16 + (uint32_t)(lane >> 4) * 4;
  const uint32_t spoff = 256 + (uint32_t)(lane >> 4) * 64 + (uint32_t)(lane & 15) * 4;
  const uint32_t cunit = 16384u / (uint32_t)gsz;  // BPDQ coefficients, as in k_stream
  const uint32_t coff =
      ((uint32_t)(lane & 15) * (128u / (uint32_t)gsz) + (uint32_t)(32 * (lane >> 4)) / (uint32_t)gsz) * 8u;
  uint32_t cb[CH][BITS];
  uint32_t sb[CH][2];
  uint32_t ent[CH];  // the block's outliers, one per lane (up to 64; more are read at decode)
  int elo[CH], ecnt[CH];
  auto issue = [&](int u, int g) {  // g: blob block index, -1 for none
    const bool in = g >= 0;
    load_chunk<BITS>(cb[u], rc, in ? (uint32_t)g * BB + voff : kOutOfRange);
    if constexpr (F::bpdq) {
      const u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(rs, (int)(in ? (uint32_t)g * cunit + coff : kOutOfRange),
                                                             0, kNonTemporal);
      sb[u][0] = v[0];
      sb[u][1] = v[1];
    } else if constexpr (!F::lut) {
      sb[u][0] = __builtin_amdgcn_raw_buffer_load_b32(rs, (int)(in ? (uint32_t)g * 512 + zoff : kOutOfRange), 0,
                                                      kNonTemporal);
      sb[u][1] = __builtin_amdgcn_raw_buffer_load_b32(rs, (int)(in ? (uint32_t)g * 512 + spoff : kOutOfRange), 0,
                                                      kNonTemporal);
    } else {
      sb[u][0] = sb[u][1] = 0;
    }
  };
  auto issue_ent = [&](int u, int lo, int n) {
    ent[u] = __builtin_amdgcn_raw_buffer_load_b32(rbe, lane < n ? (lo + lane) * 4 : (int)kOutOfRange, 0, kNonTemporal);
    elo[u] = lo;
    ecnt[u] = n;
  };
  // Chunk q: local tile q / CPT, K-blocks kb .. kb + nv - 1 of the split,
  // blob block g0 of the first, staged offsets at bo_lds[t * OB + kb - kb0].
  struct Chunk {
    int q, t, kb, g0, nv;
  };
  auto chunk_at = [&](int q) -> Chunk {
    Chunk k;
    k.q = q;
    k.t = q / CPT;
    k.kb = kb0 + (q - k.t * CPT) * CH;
    k.g0 = (T0 + k.t) * nkb + k.kb;
    k.nv = q < nchunks ? min(CH, kb1 - k.kb) : 0;
    return k;
  };
  // the outlier offsets of a chunk's blocks (lane i: block i's start, i <= nv)
  auto chunk_offsets = [&](const Chunk& k) {
    return lane <= k.nv && k.nv > 0 ? bo_lds[k.t * OB + k.kb - kb0 + lane] : 0;
  };
  // The first chunk's loads go out behind the staged ones; the wait below
  // covers the staged loads alone (they were issued first and complete in
  // order), so the ring runs on across the barrier.
  Chunk ck = chunk_at(w);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int u = 0; u < CH; ++u) issue(u, u < ck.nv ? ck.g0 + u : -1);
  __builtin_amdgcn_sched_barrier(0);
  constexpr int kRing = CH * (F::lut ? 1 : F::bpdq ? 2 : 3);  // vector loads per ring fill
  static_assert(kRing < 64, "vmcnt holds 6 bits");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (kRing & 15) | ((kRing >> 4) << 14));

#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int i = (int)threadIdx.x + 1024 * k;
    if (i < TW * OB) bo_lds[i] = bo[k];
  }
  if constexpr (F::lut) {
    if ((int)threadIdx.x < lpieces) ((u32x4_t*)lut_lds)[threadIdx.x] = ls;
  }
  {
    const u32x4_t z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int k = 0; k < 4; ++k) ((u32x4_t*)otile)[lane + 64 * k] = z;
  }
  if (threadIdx.x == 0) *chunk_ctr = kWaves;
  lds_barrier();
  {
    const int obv = chunk_offsets(ck);
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      const int lo = __builtin_amdgcn_readlane(obv, u);
      issue_ent(u, lo, u < ck.nv ? __builtin_amdgcn_readlane(obv, u + 1) - lo : 0);
    }
  }
  auto next_chunk = [&]() -> Chunk {
    int q = 0;
    if (lane == 0) q = lds_fetch_add(chunk_ctr, 1);
    return chunk_at(__builtin_amdgcn_readfirstlane(q));
  };

  int tc = -1;  // local tile whose table is in tab
  uint32_t tab[F::tab_dw];
  auto planes = [&]() {
    if constexpr (F::lut) {
      const uint32_t* L = lut_lds + (tc * 16 + (lane & 15)) * F::tab_dw;
      uint32_t Lr[F::tab_dw];
#pragma unroll
      for (int i = 0; i < F::tab_dw; ++i) Lr[i] = L[i];
      if constexpr (BITS == 4) l4_planes(Lr, tab);
      else l3_planes(Lr, tab);
    } else {
      tab[0] = 0;
    }
  };
  // B operand of lane (n, q) = (lane % 16, lane / 16), step s2 of K-block kb:
  // x[n][128 kb + 32 q + 8 s2 .. +7], piece 16 (kb - kb0) + 4 q + s2 of the slice.
  const uint16_t* xb = xs + (4 * (lane >> 4) * NB + ((lane & 15) & (NB - 1))) * 8;
  while (ck.q < nchunks) {
    const Chunk nx = next_chunk();
    const int obv = chunk_offsets(nx);
    if (ck.t != tc) {
      tc = ck.t;
      planes();
    }
    floatx4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      if (u < ck.nv) {
        uint32_t am[F::n_mfma][4];
        if constexpr (F::lut || F::bpdq) {
          decode_chunk<FMT, BITS>(cb[u], sb[u], tab, am);
        } else {
          const uint32_t st[2] = {perm(sb[u][0], sb[u][1], 0x05040100u), perm(sb[u][0], sb[u][1], 0x07060302u)};
          decode_chunk<FMT, BITS>(cb[u], st, tab, am);
        }
        const int kbl = ck.kb + u - kb0;
        half8_t bx[4];
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) {
          bx[s2] = *(const half8_t*)(xb + (16 * kbl + s2) * NB * 8);
          acc = mfma(h8(am[s2][0], am[s2][1], am[s2][2], am[s2][3]), bx[s2], acc);
          if constexpr (!F::lut)
            acc = mfma(h8(am[4 + s2][0], am[4 + s2][1], am[4 + s2][2], am[4 + s2][3]), bx[s2], acc);
        }
        // The block's outliers: scattered into the wave's zero 16x128 tile
        // in A-operand order, multiplied with the block's x like the dense
        // codes, then cleared.
        const int n = ecnt[u];
        if (n > 0) {
          auto place = [&](uint32_t e) {
            const uint32_t c = e & 127u, m = (e >> 7) & 15u;
            return (((c >> 3) & 3u) * 64u + m + 16u * (c >> 5)) * 8u + (c & 7u);
          };
          uint32_t oa = 0;
          if (lane < n) {
            oa = place(ent[u]);
            otile[oa] = (uint16_t)(ent[u] >> 16);
          }
          for (int p = 64; p < n; p += 64)  // more than 64 in the block
            if (lane + p < n) {
              const uint32_t e = bent[elo[u] + p + lane];
              otile[place(e)] = (uint16_t)(e >> 16);
            }
#pragma unroll
          for (int s2 = 0; s2 < 4; ++s2) {
            const u32x4_t av = ((const u32x4_t*)otile)[s2 * 64 + lane];
            acc = mfma(h8(av[0], av[1], av[2], av[3]), bx[s2], acc);
          }
          if (n <= 64) {
            if (lane < n) otile[oa] = 0;
          } else {
            const u32x4_t z = {0u, 0u, 0u, 0u};
#pragma unroll
            for (int k = 0; k < 4; ++k) ((u32x4_t*)otile)[lane + 64 * k] = z;
          }
        }
      }
      issue(u, u < nx.nv ? nx.g0 + u : -1);
      const int lo = __builtin_amdgcn_readlane(obv, u);
      issue_ent(u, lo, u < nx.nv ? __builtin_amdgcn_readlane(obv, u + 1) - lo : 0);
    }
    // acc[i]: row 4*(lane/16) + i of the chunk's tile, batch column lane % 16
    float* sl = part + ck.q * 16 * NB;
    if ((lane & 15) < NB)
#pragma unroll
      for (int i = 0; i < 4; ++i) sl[(4 * (lane >> 4) + i) * NB + (lane & 15)] = acc[i];
    ck = nx;
  }
  __builtin_amdgcn_s_waitcnt(kVmcntZero);
  __syncthreads();

  // Each output (row r, batch column n) adds its tile's chunk partials in
  // chunk order; a thread takes four batch columns of one row (16 bytes).
  const bool split = S > 1;
  constexpr int kSc1 = 16;  // cache policy: device-coherent (bypass the XCD's non-coherent L2 copy)
  const rsrc_t rw = make_rsrc(wpart, (uint32_t)((uint64_t)S * tiles * 16 * NB * 4));
  const uint32_t wbase = (uint32_t)((si * tiles + T0) * 16 * NB) * 4u;  // this split's partials of the group
  for (int i = threadIdx.x; i < nrows * NB / 4; i += 64 * kWaves) {
    const int r = i / (NB / 4), n4 = 4 * (i - r * (NB / 4));
    const float* ps = part + (r >> 4) * CPT * 16 * NB + (r & 15) * NB + n4;
    floatx4_t v = {0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < CPT; ++j) v += *(const floatx4_t*)(ps + j * 16 * NB);
    if (split) {
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), rw, (int)(wbase + 16u * (uint32_t)i), 0,
                                             kSc1);
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k) y[(size_t)(n4 + k) * M + T0 * 16 + r] = v[k];
    }
  }
  if (!split) return;

  // The splits meet.  The partials went out as device-coherent stores; each
  // thread waits until its stores are acknowledged, and after the barrier
  // one thread counts the workgroup's arrival.  The last of the S reads the S
  // partials with device-coherent loads, after its count returned, and adds
  // them in split order.  No L2 write-back or invalidate is needed.
  __builtin_amdgcn_s_waitcnt(kVmcntZero);
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t add = 8u / (uint32_t)S;
    const uint32_t old = __hip_atomic_fetch_add(wctr + gi, add, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *last_flag = ((old + add) & 7u) == 0u;
  }
  __syncthreads();
  if (!*last_flag) return;
  for (int i = threadIdx.x; i < nrows * NB / 4; i += 64 * kWaves) {
    const int r = i / (NB / 4), n4 = 4 * (i - r * (NB / 4));
    u32x4_t pv[8];
#pragma unroll
    for (int s2 = 0; s2 < 8; ++s2)
      pv[s2] = __builtin_amdgcn_raw_buffer_load_b128(
          rw, s2 < S ? (int)((uint32_t)((s2 * tiles + T0) * 16 * NB) * 4u + 16u * (uint32_t)i) : (int)kOutOfRange, 0,
          kSc1);
    floatx4_t v = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s2 = 0; s2 < 8; ++s2)
      if (s2 < S) v += __builtin_bit_cast(floatx4_t, pv[s2]);
#pragma unroll
    for (int k = 0; k < 4; ++k) y[(size_t)(n4 + k) * M + T0 * 16 + r] = v[k];
  }
}

// ---------------------------------------------------------------------------
// Batch 1, 4-bit LUT codes: pair tables in LDS.
//
// A byte of an L4 chunk holds two codes, A (chunk column k) and B (column
// 4 + k).  For each row the workgroup builds a 256-entry table that maps a
// byte value to the FP16 pair (LUT[A], LUT[B]), so one 4-byte LDS read
// decodes two codes.  The four K-groups of the MFMA A operand carry four
// different tiles: lane l holds row l % 16 of tile 4g + l / 16 of the
// workgroup (g = table region, at most two), so each lane reads its own
// row's table.  The table of lane l sits at byte 4l of every 256-byte line
// and line b holds byte value b, so the 64 lanes of a read always fall in 64
// different banks, and one v_perm forms the address (4l, code byte, region)
// straight from the code dword.  Column t of the B operand carries x only in
// K-group t and zeros elsewhere, so MFMA column t sums the rows of tile t.
//
// x sits in LDS with each group of 8 columns in pair order (0,4,1,5,2,6,3,7),
// the order in which the pair reads fill an A operand.  The work is cut into
// units of one 256-byte quarter of a (tile, K-block) piece for each of the 4
// tiles of a region; the units, region-major, are cut into 16 contiguous
// runs, one per wave, and wave v writes its sums for region g to partial slot
// v + g (distinct, because the runs are ordered).  Every output adds the slots
// of the waves covering its region in wave order, then its outliers, so the
// result does not depend on timing.
// ---------------------------------------------------------------------------
template <int R>
__global__ void __launch_bounds__(64 * kWaves)
k_pair(const uint8_t* __restrict__ codes, const uint32_t* __restrict__ meta, const int32_t* __restrict__ row_ptr,
       const uint32_t* __restrict__ entries, const uint16_t* __restrict__ x, float* __restrict__ y, int M, int K,
       int Kp, int nkb, int tiles, uint32_t meta_bytes) {
  extern __shared__ uint32_t lds[];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int T0 = (int)((int64_t)blockIdx.x * tiles / gridDim.x);
  const int T1 = (int)((int64_t)(blockIdx.x + 1) * tiles / gridDim.x);
  const int TW = T1 - T0;  // at most 8
  const int G = (TW + 3) >> 2;  // table regions
  const int nrows = min(TW * 16, M - T0 * 16);
  const int P = 4 * nkb;  // units per region
  const int U = G * P;
  auto run_bound = [&](int v) { return v * U / kWaves; };
  const int u0 = run_bound(w), u1 = run_bound(w + 1);  // this wave's run

  // LDS: tables [G][256 byte values][64 lanes] | xs [Kp] FP16, pair order | slots [16 + G][4 tiles][16 rows]
  //      | csr [TW*16] | row_ptr [TW*16+1, padded] | group counter
  uint16_t* xs = (uint16_t*)(lds + G * 16384);
  float* slots = (float*)(lds + G * 16384 + Kp / 2);
  float* csr = slots + (kWaves + G) * 64;
  int* rp_lds = (int*)(csr + TW * 16);
  int* group_ctr = rp_lds + ((TW * 16 + 4) & ~3);

  // Prologue.  What goes to LDS is loaded first and waited for before the
  // code ring is issued, so that these few loads do not queue behind every
  // CU's ring at the start; the barrier (LDS only) then lets the ring loads
  // run on into the stream.
  const rsrc_t rr = make_rsrc(row_ptr, (uint32_t)(M + 1) * 4);
  const int rpn = threadIdx.x <= TW * 16 ? __builtin_amdgcn_raw_buffer_load_b32(
                                               rr, min(T0 * 16 + (int)threadIdx.x, M) * 4, 0, 0)
                                         : 0;
  // Table entries of byte values 16w .. 16w+15 for lane column `lane` of each
  // region: A runs over LUT entries 8*bit2(w) .. +7 (one 16-byte piece), B
  // over the two entries of LUT dword (w & 3) | 4*bit3(w).
  const rsrc_t rl = make_rsrc(meta, meta_bytes);
  u32x4_t la[2];
  uint32_t lb[2];
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    const int tile = T0 + 4 * g + (lane >> 4);
    const bool has = g < G && tile < T1;
    const uint32_t rowb = (uint32_t)(tile * 16 + (lane & 15)) * 32u;
    la[g] = __builtin_amdgcn_raw_buffer_load_b128(rl, (int)(has ? rowb + 16u * ((w >> 2) & 1) : kOutOfRange), 0,
                                                  kNonTemporal);
    lb[g] = __builtin_amdgcn_raw_buffer_load_b32(
        rl, (int)(has ? rowb + 4u * (uint32_t)((w & 3) | 4 * ((w >> 3) & 1)) : kOutOfRange), 0, kNonTemporal);
  }
  // x: 8-column pieces tid and tid + 1024 (Kp <= 16384); columns past K read as 0.
  const rsrc_t rx = make_rsrc(x, (uint32_t)K * 2u);
  const int xpieces = Kp / 8;
  u32x4_t xv[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int piece = (int)threadIdx.x + 1024 * k;
    xv[k] = __builtin_amdgcn_raw_buffer_load_b128(rx, piece < xpieces ? piece * 16 : (int)kOutOfRange, 0, 0);
  }
  __builtin_amdgcn_sched_barrier(0);  // keep the ring loads behind the staged ones
  __builtin_amdgcn_s_waitcnt(kVmcntZero);  // the staged loads have landed
  asm volatile("" ::"v"(la[0]), "v"(lb[0]), "v"(la[1]), "v"(lb[1]), "v"(xv[0]), "v"(xv[1]));
  // The code ring.  Unit v: region g = v / P, quarter-block v % P; lanes of
  // tiles past T1 fall outside the resource and read 0.
  const rsrc_t rc = make_rsrc(codes, (uint32_t)T1 * (uint32_t)nkb * 1024u);
  const uint32_t lb0 = (uint32_t)((T0 + (lane >> 4)) * nkb) * 1024u + (uint32_t)(lane & 15) * 16u;
  auto uoff = [&](int v) -> uint32_t {
    if (v >= u1) return kOutOfRange;
    const int g = v >= P ? 1 : 0;
    return lb0 + (uint32_t)(g * P) * 1024u + (uint32_t)(v - g * P) * 256u;
  };
  u32x4_t ring[R];
#pragma unroll
  for (int s = 0; s < R; ++s) ring[s] = __builtin_amdgcn_raw_buffer_load_b128(rc, (int)uoff(u0 + s), 0, kNonTemporal);

  // x in pair order: (0,4,1,5,2,6,3,7) in each 8-column group.  A piece past
  // x goes to the first 16 bytes after it (partial slot 0, which is written
  // before it is read); unconditional stores keep the x loads ahead of the ring.
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int piece = (int)threadIdx.x + 1024 * k;
    const u32x4_t v = xv[k];
    const u32x4_t o = {perm(v[2], v[0], 0x05040100u), perm(v[2], v[0], 0x07060302u), perm(v[3], v[1], 0x05040100u),
                       perm(v[3], v[1], 0x07060302u)};
    ((u32x4_t*)xs)[min(piece, xpieces)] = o;
  }
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    if (g < G) {
      uint32_t* tg = lds + g * 16384 + 16 * w * 64 + lane;
      const uint32_t a[4] = {la[g][0], la[g][1], la[g][2], la[g][3]};
#pragma unroll
      for (int i = 0; i < 16; ++i)
        tg[64 * i] = perm(lb[g], a[(i & 7) >> 1], ((i & 1) ? 0x0302u : 0x0100u) | ((i & 8) ? 0x07060000u : 0x05040000u));
    }
  }
  if ((int)threadIdx.x <= TW * 16) rp_lds[threadIdx.x] = rpn;
  if (threadIdx.x == 0) *group_ctr = 0;
  lds_barrier();

  // The stream.
  const int tq = lane >> 4, mq = lane & 15;
  const bool on = mq == tq;  // B-operand lanes that carry x
  floatx4_t acc = {0.f, 0.f, 0.f, 0.f};
  half8_t bx = {0, 0, 0, 0, 0, 0, 0, 0};
  int gc = u0 >= P ? 1 : 0;
  auto flush = [&]() {  // acc[i]: row 4*(lane/16) + i of tile lane % 16 of region gc
    float* d = slots + (w + gc) * 64;
    if (mq < 4)
#pragma unroll
      for (int i = 0; i < 4; ++i) d[mq * 16 + 4 * tq + i] = acc[i];
  };
  for (int uu = u0; uu < u1; uu += R) {
#pragma unroll
    for (int s = 0; s < R; ++s) {
      const int v = uu + s;
      if (v < u1) {
        const int g = v >= P ? 1 : 0;
        if (g != gc) {
          flush();
          acc = (floatx4_t){0.f, 0.f, 0.f, 0.f};
          gc = g;
        }
        const uint32_t base = ((uint32_t)g << 16) | ((uint32_t)lane << 2);
        const half8_t* xp = (const half8_t*)(xs + 32 * (v - g * P));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          uint32_t a[4];
#pragma unroll
          for (int k = 0; k < 4; ++k)
            a[k] = *(const uint32_t*)((const uint8_t*)lds + perm(ring[s][i], base, 0x0C020400u + ((uint32_t)k << 8)));
          if (on) bx = xp[i];
          acc = mfma(h8(a[0], a[1], a[2], a[3]), bx, acc);
        }
      }
      // Unconditional, so that every slot has the same loads behind it (a
      // load past the run is out of range).
      ring[s] = __builtin_amdgcn_raw_buffer_load_b128(rc, (int)uoff(v + R), 0, kNonTemporal);
    }
  }
  if (u0 < u1) flush();

  // Outliers, before the barrier, by the waves that finish first: groups of
  // four CSR rows from an LDS counter, one DPP row of 16 lanes per CSR row,
  // a lane taking every 16th outlier of its row from HBM, four at a time;
  // four DPP steps add the 16 lanes.  A row's sum is the same whichever wave
  // takes it.
  {
    const int sl = lane & 15, rq = lane >> 4;
    for (;;) {
      int gi = 0;
      if (lane == 0) gi = lds_fetch_add(group_ctr, 1);
      gi = __builtin_amdgcn_readfirstlane(gi);
      if (4 * gi >= nrows) break;
      const int r = 4 * gi + rq;
      const bool real = r < nrows;
      const int p0 = real ? rp_lds[r] : 0, p1 = real ? rp_lds[r + 1] : 0;
      float v = 0.f;
      auto term = [&](uint32_t e) {
        const uint32_t c = e & 0xFFFFu;
        const uint32_t pc = (c & ~7u) | ((c & 3u) << 1) | ((c >> 2) & 1u);  // pair-order position
        v = dot2(e >> 16, (uint32_t)xs[pc], v);
      };
      int p = p0 + sl;
      for (; p + 48 < p1; p += 64) {  // four outliers in flight
        uint32_t e[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) e[u] = entries[p + 16 * u];
#pragma unroll
        for (int u = 0; u < 4; ++u) term(e[u]);
      }
      for (; p < p1; p += 16) term(entries[p]);
      v += dpp_mov<0xB1, 0xF>(v);   // quad_perm [1,0,3,2]
      v += dpp_mov<0x4E, 0xF>(v);   // quad_perm [2,3,0,1]
      v += dpp_mov<0x141, 0xF>(v);  // row_half_mirror
      v += dpp_mov<0x140, 0xF>(v);  // row_mirror: every lane of the row holds the sum
      if (real && sl == 0) csr[r] = v;
    }
  }
  __syncthreads();
  for (int r = threadIdx.x; r < nrows; r += 64 * kWaves) {
    const int g = r >> 6;  // local row r = 64 g + 16 t + m
    float s[kWaves];  // all reads first, then the adds in wave order
#pragma unroll
    for (int u = 0; u < kWaves; ++u) s[u] = slots[(u + g) * 64 + (r & 63)];
    float v = 0.f;
#pragma unroll
    for (int u = 0; u < kWaves; ++u) {
      const int c0 = run_bound(u), c1 = run_bound(u + 1);
      v = c0 < c1 && c0 < (g + 1) * P && c1 > g * P ? v + s[u] : v;
    }
    y[T0 * 16 + r] = v + csr[r];
  }
}

// ---------------------------------------------------------------------------
// HPTQ, batch 1: prefix-coded integers on one grid.
//
// A (tile, K-block) block holds its 64 lanes' 32-codeword chunks as one bit
// sequence (qgemv_layout.h).  A wave takes the blocks of its run G at a
// time: it copies their words into G LDS buffers and decodes the G chunks of
// each lane side by side, so that the G chains of dependent LDS reads hide
// one another's latency.  For each pair of codewords (at most 32 bits) a
// chain funnel-shifts the two words at its bit position into a 32-bit
// window.  The window's top 8 bits index the first-level table, which gives
// the FP16 integer and the length of the codeword they start with; the
// table is held once per lane (entry e of lane l at e * 64 + l), so that a
// wave's 64 reads fall in 64 distinct banks.  A longer codeword's 8-bit
// prefix names a 256-entry second-level table, indexed by the next 8 bits;
// where those tables do not fit in LDS, the length is the shortest l whose
// 16-bit left-justified prefix lies below the end of the canonical
// codewords of length l, and the integer one more read.  The integers are
// exact in FP16; every 8 codewords of a chunk are the A operand of one MFMA
// against x, and each row's step scales the block's sums in fp32.  The
// blocks of a workgroup are cut into 16 runs, one per wave, with a partial
// slot per (wave, tile) as in k_xlds, and the outputs add the slots in wave
// order.  The next G blocks' first 1 KiB of code words, lane offsets and
// steps are loaded while the current ones are decoded.
// ---------------------------------------------------------------------------
constexpr int kHuffMaxBlockWords = 64 * kChunkCodes * kHuffMaxLen / 32;  // a block's largest code
constexpr int kHuffPad = 20;  // words a chain may read past its chunk's start word, and past the block
constexpr int kHuffMaxSub = 64;  // second-level tables held in LDS (64 KiB)
constexpr int kHuffLongLens = kHuffMaxLen - kHuffBits;  // lengths a second-level step decodes
static_assert(kHuffBits == 8, "the first-level address takes the window's top byte");
static_assert(kWaves == 16 && kHuffTable * 16 == 4 * 1024 && kMaxK / 8 <= 2 * 1024 &&
                  kHuffMaxSub * kHuffSub / 4 <= 4 * 1024,
              "the prologue stages x, the tables and the second-level tables in fixed rounds of 1024 threads");

template <int G, bool SUB, int NB>
__global__ void __launch_bounds__(64 * kWaves)
k_huff(const uint32_t* __restrict__ words, const uint16_t* __restrict__ steps, const uint32_t* __restrict__ hidx,
       const uint16_t* __restrict__ hlane, const int32_t* __restrict__ htab, const int16_t* __restrict__ hsym,
       const uint16_t* __restrict__ x, float* __restrict__ y, int M, int K, int nkb, int tiles, int nsym,
       uint32_t nwords, int bufw, int nsub) {
  extern __shared__ uint32_t lds[];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int T0 = (int)((int64_t)blockIdx.x * tiles / gridDim.x);
  const int T1 = (int)((int64_t)(blockIdx.x + 1) * tiles / gridDim.x);
  const int TW = T1 - T0;
  const int nrows = min(TW * 16, M - T0 * 16);
  const int L = TW * nkb;
  const int b0 = w * L / kWaves, b1 = (w + 1) * L / kWaves;  // this wave's run

  // LDS: first-level table [kHuffTable][64] (static, at address 0: entry e of
  //      lane l at e * 64 + l, so that a wave's 64 reads fall in 64 banks)
  //      | xs [K] FP16 (batch 1) | aux | slots [TW+15][16 rows][NB]
  //      | block word offsets hidx[T0 * nkb .. T1 * nkb] (padded) | code buffers [16][G][bufw];
  //      aux: the second-level tables [nsub][kHuffSub] (SUB), else the
  //      integers [nsym] FP16 (padded).  At batch 8/16 x stays in L2.
  __shared__ uint32_t tab[kHuffTable * 64];
  const int xsw = NB == 1 ? K / 2 : 0;
  uint16_t* xs = (uint16_t*)lds;
  uint32_t* aux = lds + xsw;
  uint16_t* syms = (uint16_t*)aux;
  const int auxw = SUB ? kHuffSub * nsub : ((nsym + 1) / 2 + 3) / 4 * 4;
  float* slots = (float*)(aux + auxw);
  uint32_t* hl = (uint32_t*)(slots + (TW + 15) * 16 * NB);
  const int bofs = xsw + auxw + (TW + 15) * 16 * NB + ((L + 4) & ~3) + w * G * bufw;  // in lds, in words
  uint32_t* buf = lds + bofs;

  // Prologue: every load first, then the LDS stores, so the latencies overlap.
  // x: pieces tid, tid + 1024 (K <= 16384); first-level entries (i >> 4) for
  // pieces i = tid + 1024 k, k < 4; second-level pieces tid + 1024 k (nsub <= 64).
  const int tid = (int)threadIdx.x;
  u32x4_t xv[2], av[4];
  uint32_t tv[4];
  const u32x4_t* asrc = (const u32x4_t*)(htab + kHuffTable + 4 * 17);
#pragma unroll
  for (int k = 0; k < 2; ++k)
    if (NB == 1 && tid + 1024 * k < K / 8) xv[k] = ((const u32x4_t*)x)[tid + 1024 * k];
#pragma unroll
  for (int k = 0; k < 4; ++k) tv[k] = (uint32_t)htab[(tid + 1024 * k) >> 4];
#pragma unroll
  for (int k = 0; k < 4; ++k)
    if (SUB && tid + 1024 * k < nsub * (kHuffSub / 4)) av[k] = asrc[tid + 1024 * k];
  const uint32_t hv = tid <= L ? hidx[T0 * nkb + tid] : 0u;
#pragma unroll
  for (int k = 0; k < 2; ++k)
    if (NB == 1 && tid + 1024 * k < K / 8) ((u32x4_t*)xs)[tid + 1024 * k] = xv[k];
#pragma unroll
  for (int k = 0; k < 4; ++k) ((u32x4_t*)tab)[tid + 1024 * k] = (u32x4_t){tv[k], tv[k], tv[k], tv[k]};
#pragma unroll
  for (int k = 0; k < 4; ++k)
    if (SUB && tid + 1024 * k < nsub * (kHuffSub / 4)) ((u32x4_t*)aux)[tid + 1024 * k] = av[k];
  if (tid <= L) hl[tid] = hv;
  for (int i = tid + 1024; i <= L; i += 64 * kWaves) hl[i] = hidx[T0 * nkb + i];  // runs past 1024 blocks
  if (!SUB)
    for (int i = tid; i < nsym; i += 64 * kWaves) syms[i] = __builtin_bit_cast(uint16_t, (_Float16)(float)hsym[i]);

  // Codewords longer than the first-level index, lengths kHuffBits+1 .. 16,
  // without second-level tables: per length the left-justified end of its
  // codewords, and the index in syms of a codeword c of that length minus c.
  // The length of a long codeword is the shortest whose end lies above the
  // prefix.
  __shared__ int32_t lcl[2 * kHuffLongLens];  // ends, then index offsets
  if (!SUB && threadIdx.x < kHuffLongLens) {
    const int l = kHuffBits + 1 + threadIdx.x;
    lcl[threadIdx.x] = htab[kHuffTable + 51 + l];
    lcl[kHuffLongLens + threadIdx.x] = htab[kHuffTable + 34 + l] - htab[kHuffTable + l];
  }
  auto long_code = [&](uint32_t win) -> uint32_t {
    const uint32_t p16 = win >> (32 - kHuffMaxLen);
    uint32_t len = kHuffMaxLen;
    int d = lcl[2 * kHuffLongLens - 1];
#pragma unroll
    for (int k = kHuffLongLens - 2; k >= 0; --k) {
      const bool in = p16 < (uint32_t)lcl[k];
      len = in ? (uint32_t)(kHuffBits + 1 + k) : len;
      d = in ? lcl[kHuffLongLens + k] : d;
    }
    const uint32_t idx = min((uint32_t)((int)(p16 >> (kHuffMaxLen - len)) + d), (uint32_t)(nsym - 1));
    return ((uint32_t)syms[idx] << 16) | len;
  };
  const uint32_t lane4 = (uint32_t)lane * 4u;
  const rsrc_t rw = make_rsrc(words, nwords * 4u);
  // batch 8/16: lane l's B operand is batch row l % 16 (zero past NB), columns
  // 32 (l / 16) + 8i .. +7 of the K-block; rows past NB read out of range
  const rsrc_t rxb = make_rsrc(x, NB == 1 ? 0u : (uint32_t)(NB * K) * 2u);
  const int xrow = NB > 1 && (lane & 15) < NB ? (lane & 15) * K : -1;
  constexpr int XP = NB == 1 ? 1 : 2;  // x pieces in flight per chain
  u32x4_t pre[G], xq[G][XP];
  int xk[G];  // the chain's K offset in x (its block's first column of this lane)
  uint32_t lbn[G], stn0[G], stn1[G];
#pragma unroll
  for (int c = 0; c < G; ++c) {
    pre[c] = (u32x4_t){0u, 0u, 0u, 0u};
    lbn[c] = stn0[c] = stn1[c] = 0u;
  }
  // per block: first 1 KiB of words, lane offset, steps of rows 4*(lane/16) .. +3;
  // the block offsets come from LDS once the prologue's barrier has passed
  auto prefetch = [&](int r0, bool first) {
#pragma unroll
    for (int c = 0; c < G; ++c) {
      const int bb = r0 + c;
      if (bb < b1) {
        const int g = T0 * nkb + bb;
        const uint32_t wo = first ? hidx[g] : __builtin_amdgcn_readfirstlane(hl[bb]);
        pre[c] = __builtin_amdgcn_raw_buffer_load_b128(rw, (int)((wo + 4u * (uint32_t)lane) * 4u), 0, kNonTemporal);
        lbn[c] = hlane[(size_t)g * 64 + lane];
        const uint32_t* sp = (const uint32_t*)(steps + (size_t)g * 16 + 4 * (lane >> 4));
        stn0[c] = sp[0];
        stn1[c] = sp[1];
      }
    }
  };
  prefetch(b0, true);
  __syncthreads();

  floatx4_t acc = {0.f, 0.f, 0.f, 0.f};
  int tl = b0 / nkb;
  auto flush = [&]() {  // acc[i]: row 4*(lane/16) + i of local tile tl, batch row lane % 16
    if constexpr (NB == 1) {
      if ((lane & 15) == 0)
#pragma unroll
        for (int i = 0; i < 4; ++i) slots[(w + tl) * 16 + 4 * (lane >> 4) + i] = acc[i];
    } else {
      if ((lane & 15) < NB)
#pragma unroll
        for (int i = 0; i < 4; ++i) slots[((w + tl) * 16 + 4 * (lane >> 4) + i) * NB + (lane & 15)] = acc[i];
    }
  };
  const int sl = 32 * (lane >> 4);
  const uint32_t cap = (uint32_t)(bufw - kHuffPad);
  for (int r0 = b0; r0 < b1; r0 += G) {
    uint32_t lb[G], st0[G], st1[G];
#pragma unroll
    for (int c = 0; c < G; ++c) {
      const int bb = r0 + c;
      uint32_t* bc = buf + c * bufw;
      lb[c] = 0u;
      if (bb < b1) {
        const int t = bb / nkb;
        const uint32_t wo = __builtin_amdgcn_readfirstlane(hl[bb]);
        const uint32_t nw = min(__builtin_amdgcn_readfirstlane(hl[bb + 1]) - wo, cap);  // a multiple of 4
        // the block's words: the first 1 KiB from the prefetch, any more now
        if (4 * lane < (int)nw) ((u32x4_t*)bc)[lane] = pre[c];
        for (uint32_t i = 256u + 4u * (uint32_t)lane; i < nw; i += 256u)
          *(u32x4_t*)(bc + i) = __builtin_amdgcn_raw_buffer_load_b128(rw, (int)((wo + i) * 4u), 0, kNonTemporal);
        if (T0 * 16 + t * 16 + (lane & 15) < M) lb[c] = min(lbn[c], 32u * cap);
      }
      st0[c] = stn0[c];
      st1[c] = stn1[c];
      if constexpr (NB > 1) {  // pieces 0 and 1 from L2 now, piece i + 2 after MFMA i
        xk[c] = xrow < 0 || bb >= b1 ? -1 : xrow + (bb - (bb / nkb) * nkb) * kBlockK + 32 * (lane >> 4);
#pragma unroll
        for (int i = 0; i < XP; ++i)
          xq[c][i] = __builtin_amdgcn_raw_buffer_load_b128(rxb, xk[c] < 0 ? (int)kOutOfRange : (xk[c] + 8 * i) * 2, 0, 0);
      }
    }
    prefetch(r0 + G, false);

    // decode the G chunks of this lane, 32 codewords each, side by side; every
    // 8 codewords of a chunk are one MFMA A operand.  Each pair of codewords
    // (at most 32 bits) is the 32-bit window at the chunk's bit position: with
    // p = position + 31, the words p/32 - 1 and p/32 funnel-shifted right by
    // -position mod 32.  A chain keeps np = ~p: the shift is np mod 32, and
    // p/32 = ~(np >> 5) with an arithmetic shift.  Rows past M decode whatever
    // their lanes read; their sums are never stored.
    uint32_t qh[G][4];
    floatx4_t blk[G];
    uint32_t np[G];
#pragma unroll
    for (int c = 0; c < G; ++c) {
      blk[c] = (floatx4_t){0.f, 0.f, 0.f, 0.f};
      np[c] = ~(lb[c] + 31u);
    }
#pragma unroll
    for (int j = 0; j < 32; j += 2) {
      uint32_t win[G], e[2][G];
#pragma unroll
      for (int c = 0; c < G; ++c) {
        const int k = (bofs + c * bufw - 2) - ((int)np[c] >> 5);
        win[c] = __builtin_amdgcn_alignbit(lds[k], lds[k + 1], np[c]);
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
#pragma unroll
        for (int c = 0; c < G; ++c)  // byte address: lane * 4 | top window byte << 8
          e[u][c] = *(const uint32_t*)((const char*)tab + perm(win[c], lane4, 0x0C0C0700u));
#pragma unroll
        for (int c = 0; c < G; ++c)
          if ((e[u][c] & 255u) == 0u) {
            if (SUB)  // the second-level table of these 8 bits, indexed by the next 8
              e[u][c] = aux[(e[u][c] >> 16) + ((win[c] >> (32 - kHuffMaxLen)) & (uint32_t)(kHuffSub - 1))];
            else
              e[u][c] = long_code(win[c]);
          }
        if (u == 0)
#pragma unroll
          for (int c = 0; c < G; ++c) win[c] <<= (e[0][c] & 31u);
      }
#pragma unroll
      for (int c = 0; c < G; ++c) {
        np[c] -= e[0][c] & 0xffffu;
        np[c] -= e[1][c] & 0xffffu;
        qh[c][(j / 2) & 3] = __builtin_amdgcn_perm(e[1][c], e[0][c], 0x07060302u);
        if ((j & 7) == 6) {
          half8_t bx;
          if constexpr (NB == 1) {
            const int bb = r0 + c, kb = bb - (bb / nkb) * nkb;
            bx = *(const half8_t*)(xs + kb * kBlockK + sl + j - 6);
          } else {
            bx = __builtin_bit_cast(half8_t, xq[c][(j >> 3) & 1]);
          }
          blk[c] = mfma(h8(qh[c][0], qh[c][1], qh[c][2], qh[c][3]), bx, blk[c]);
          if constexpr (NB > 1)
            if ((j >> 3) + 2 < 4)
              xq[c][(j >> 3) & 1] = __builtin_amdgcn_raw_buffer_load_b128(
                  rxb, xk[c] < 0 ? (int)kOutOfRange : (xk[c] + 8 * ((j >> 3) + 2)) * 2, 0, 0);
        }
      }
    }

#pragma unroll
    for (int c = 0; c < G; ++c) {
      const int bb = r0 + c;
      if (bb < b1) {
        const int t = bb / nkb;
        if (t != tl) {
          flush();
          acc = (floatx4_t){0.f, 0.f, 0.f, 0.f};
          tl = t;
        }
        acc[0] += (float)__builtin_bit_cast(_Float16, (uint16_t)st0[c]) * blk[c][0];
        acc[1] += (float)__builtin_bit_cast(_Float16, (uint16_t)(st0[c] >> 16)) * blk[c][1];
        acc[2] += (float)__builtin_bit_cast(_Float16, (uint16_t)st1[c]) * blk[c][2];
        acc[3] += (float)__builtin_bit_cast(_Float16, (uint16_t)(st1[c] >> 16)) * blk[c][3];
      }
    }
  }
  if (b0 < b1) flush();
  __syncthreads();
  for (int i = threadIdx.x; i < nrows * NB; i += 64 * kWaves) {
    const int r = NB == 1 ? i : i / NB, n = NB == 1 ? 0 : i - r * NB, t = r >> 4;
    float v = 0.f;
    for (int u = 0; u < kWaves; ++u) {
      const int c0 = u * L / kWaves, c1 = (u + 1) * L / kWaves;
      if (c0 < c1 && c0 / nkb <= t && t <= (c1 - 1) / nkb) v += slots[((u + t) * 16 + (r & 15)) * NB + n];
    }
    y[n * M + T0 * 16 + r] = v;
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
constexpr int kMaxGrid = 256;  // one workgroup per CU
constexpr size_t kLdsBytes = 160 * 1024;
constexpr size_t kEntCapBytes = 64 * 1024;  // CSR entries staged per workgroup, at most
constexpr size_t kOneWorkgroupLds = kLdsBytes / 2 + 1024;

// LDS per tile of a workgroup.  Batch 1: chunk partials, row_ptr entries,
// table.  Batch NB: chunk partials, block outlier offsets, table.
size_t stream_lds_per_tile(const BlobHeader& h, int nb, int ch) {
  const size_t cpt = (size_t)((h.nkb + ch - 1) / ch);
  const size_t tab = h.format == QGEMV_FMT_LUT ? (size_t)(2u << h.bits) : 0;
  return nb == 1 ? cpt * 16 * 4 + 16 * 4 + 16 * tab : cpt * 16 * nb * 4 + (size_t)h.nkb * 4 + 16 * tab;
}

// LDS besides the per-tile parts and the CSR entries: batch 1, x with 16 zero
// bytes and the spare row_ptr slots; batch NB, offset padding and the 16
// waves' 4 KiB outlier tiles (and 4 KiB x stages with xst).
size_t stream_lds_extra(const BlobHeader& h, int nb, bool xst) {
  return nb == 1 ? (size_t)h.Kp * 2 + 16 + 16 : 32 + (size_t)kWaves * 4096 * (xst ? 2 : 1);
}

// One workgroup per CU, more when the per-tile LDS of 256 workgroups would
// not fit (batch 1 keeps at least 16 KiB for CSR entries) or, for batch NB,
// a workgroup's block offsets would exceed 4096.
int stream_grid(const BlobHeader& h, int nb, int ch, bool xst) {
  const size_t keep = nb == 1 ? 16 * 1024 : 0;
  if (stream_lds_extra(h, nb, xst) + keep >= kLdsBytes) return 1 << 30;
  size_t max_tw = (kLdsBytes - stream_lds_extra(h, nb, xst) - keep) / stream_lds_per_tile(h, nb, ch);
  if (max_tw > 32) max_tw = 32;
  if (nb > 1 && max_tw > (size_t)(4095 / h.nkb)) max_tw = (size_t)(4095 / h.nkb);
  if (max_tw < 1) max_tw = 1;
  int g = h.tiles < kMaxGrid ? h.tiles : kMaxGrid;
  const int need = (int)((h.tiles + max_tw - 1) / max_tw);
  return g > need ? g : need;
}

size_t stream_lds_fixed(const BlobHeader& h, int grid, int nb, int ch, bool xst) {
  const size_t tw = (size_t)((h.tiles + grid - 1) / grid);
  return stream_lds_extra(h, nb, xst) + tw * stream_lds_per_tile(h, nb, ch);
}

// Batch NB stages x through LDS (contiguous loads) when the stages fit beside
// the per-tile parts without needing more workgroups.
bool stream_xst(const BlobHeader& h, int nb, int ch) {
  if (nb == 1) return false;
  const int g = stream_grid(h, nb, ch, true);
  return g == stream_grid(h, nb, ch, false) && stream_lds_fixed(h, g, nb, ch, true) <= kLdsBytes;
}

template <int FMT, int BITS, int NB, bool XST, int CH>
hipError_t launch_stream_x(const qgemv_plan* p, const uint16_t* x, float* y, hipStream_t st) {
  constexpr int NR = 1;                // chunks in flight per wave
  const BlobHeader& h = p->h;
  const int grid = stream_grid(h, NB, CH, XST);
  const size_t fixed = stream_lds_fixed(h, grid, NB, CH, XST);
  if (fixed > kLdsBytes) return hipErrorInvalidValue;
  // Batch 1 gives the rest of LDS (up to 64 KiB) to the CSR entries.
  size_t cap = 0;
  if (NB == 1) {
    cap = kLdsBytes - fixed;
    if (cap > kEntCapBytes) cap = kEntCapBytes;
    cap &= ~(size_t)1023;  // whole 1 KiB wave loads
  }
  size_t lds = fixed + cap;
  // More than half of LDS keeps a second workgroup off the CU: one per CU.
  if (lds < kOneWorkgroupLds) lds = kOneWorkgroupLds;
  // once per instantiation (thread-safe static initialisation)
  static const hipError_t attr = hipFuncSetAttribute((const void*)k_stream<FMT, BITS, CH, NR, NB, XST>,
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsBytes);
  if (attr != hipSuccess) return attr;
  const uint32_t codes_bytes = (uint32_t)((uint64_t)h.tiles * h.nkb * h.block_bytes);
  const uint32_t meta_bytes = (uint32_t)(h.off_rowptr - h.off_meta);
  hipLaunchKernelGGL((k_stream<FMT, BITS, CH, NR, NB, XST>), dim3(grid), dim3(64 * kWaves), lds, st, p->blob + h.off_codes,
                     (const uint32_t*)(p->blob + h.off_meta), (const int32_t*)(p->blob + h.off_rowptr),
                     (const uint32_t*)(p->blob + h.off_entries), (const int32_t*)(p->blob + h.off_boff),
                     (const uint32_t*)(p->blob + h.off_bent), x, y, h.M, h.K, h.Kp, h.nkb, h.tiles, codes_bytes,
                     meta_bytes, (int)h.nnz, (int)(cap / 4), h.group_size > 0 ? h.group_size : 16);
  return hipGetLastError();
}

template <int FMT, int BITS, int NB>
hipError_t launch_stream(const qgemv_plan* p, const uint16_t* x, float* y, hipStream_t st) {
  if constexpr (NB == 1) {
    // K-blocks per chunk at batch 1: single blocks when a workgroup holds one
    // tile (its 16 waves then share the tile's blocks more finely) and for
    // BPDQ codes, whose decode keeps a wave longest per block; pairs
    // otherwise.
    const bool one = FMT == QGEMV_FMT_BPDQ || (p->h.tiles + stream_grid(p->h, 1, 2, false) - 1) /
                                                      stream_grid(p->h, 1, 2, false) <= 1;
    return one ? launch_stream_x<FMT, BITS, NB, false, 1>(p, x, y, st)
               : launch_stream_x<FMT, BITS, NB, false, 2>(p, x, y, st);
  } else {
    return stream_xst(p->h, NB, 3) ? launch_stream_x<FMT, BITS, NB, true, 3>(p, x, y, st)
                                   : launch_stream_x<FMT, BITS, NB, false, 3>(p, x, y, st);
  }
}

// LDS of the x-resident batched kernel apart from the CSR entries: x, partial
// slots, CSR sums, row_ptr slice, run table and CSR group count, tables.
size_t xlds_fixed(const BlobHeader& h, int grid, int nb) {
  const size_t tw = (size_t)((h.tiles + grid - 1) / grid);
  const size_t tab = h.format == QGEMV_FMT_LUT ? (size_t)(2u << h.bits) : 0;
  return (size_t)h.Kp * nb * 2 + (tw + 15) * 16 * nb * 4 + tw * 16 * nb * 4 + ((tw * 16 + 4) & ~(size_t)3) * 4 +
         (2 * kWaves + 4) * 4 + tw * 16 * tab;
}

// One workgroup per CU, more when a workgroup would get over 32 tiles (the
// row_ptr slice is staged by one thread per row).
int xlds_grid(const BlobHeader& h) {
  const int g = h.tiles < kMaxGrid ? h.tiles : kMaxGrid;
  const int need = (h.tiles + 31) / 32;
  return g > need ? g : need;
}

// The x-resident kernel runs when workgroups get two or more tiles (x is
// then reused across tiles; with one tile per workgroup loading x next to the
// codes is faster) and x and the partials leave at least 1 KiB of LDS.
bool xlds_fits(const BlobHeader& h, int nb) {
  return h.tiles > xlds_grid(h) && xlds_fixed(h, xlds_grid(h), nb) + 1024 <= kLdsBytes;
}

template <int FMT, int BITS, int NB>
hipError_t launch_xlds(const qgemv_plan* p, const uint16_t* x, float* y, hipStream_t st) {
  // code ring slots per wave: 4 for 4-bit codes (1 KiB per block), 3 for 3-bit
  constexpr int R = BITS == 4 ? 4 : 3;
  const BlobHeader& h = p->h;
  const int grid = xlds_grid(h);
  const size_t fixed = xlds_fixed(h, grid, NB);
  size_t cap = kLdsBytes - fixed;  // CSR entries staged in LDS
  if (cap > kEntCapBytes) cap = kEntCapBytes;
  cap &= ~(size_t)1023;  // whole 1 KiB wave copies
  size_t lds = fixed + cap;
  if (lds < kOneWorkgroupLds) lds = kOneWorkgroupLds;
  static const hipError_t attr = hipFuncSetAttribute((const void*)k_xlds<FMT, BITS, NB, R>,
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsBytes);
  if (attr != hipSuccess) return attr;
  const uint32_t codes_bytes = (uint32_t)((uint64_t)h.tiles * h.nkb * h.block_bytes);
  const uint32_t meta_bytes = (uint32_t)(h.off_rowptr - h.off_meta);
  hipLaunchKernelGGL((k_xlds<FMT, BITS, NB, R>), dim3(grid), dim3(64 * kWaves), lds, st, p->blob + h.off_codes,
                     (const uint32_t*)(p->blob + h.off_meta), (const int32_t*)(p->blob + h.off_rowptr),
                     (const uint32_t*)(p->blob + h.off_entries), x, y, h.M, h.K, h.Kp, h.nkb, h.tiles, codes_bytes,
                     meta_bytes, (int)h.nnz, (int)(cap / 4), h.group_size > 0 ? h.group_size : 16);
  return hipGetLastError();
}

// Pair-table kernel (4-bit LUT codes, batch 1): at most 8 tiles per
// workgroup, so that the tables fit in two 64 KiB regions.
int pair_grid(const BlobHeader& h) {
  const int g = h.tiles < kMaxGrid ? h.tiles : kMaxGrid;
  const int need = (h.tiles + 7) / 8;
  return g > need ? g : need;
}

// LDS of the pair-table kernel: tables, x, partial slots, CSR sums, row_ptr
// slice and the CSR group counter.
size_t pair_lds(const BlobHeader& h, int grid) {
  const size_t tw = (size_t)((h.tiles + grid - 1) / grid);
  const size_t regions = (tw + 3) / 4;
  return regions * 65536 + (size_t)h.Kp * 2 + (kWaves + regions) * 64 * 4 + tw * 16 * 4 +
         ((tw * 16 + 4) & ~(size_t)3) * 4 + 16;
}

bool pair_fits(const BlobHeader& h) {
  return h.format == QGEMV_FMT_LUT && h.bits == 4 && h.Kp <= 16384 && pair_lds(h, pair_grid(h)) <= kLdsBytes;
}

hipError_t launch_pair(const qgemv_plan* p, const uint16_t* x, float* y, hipStream_t st) {
  constexpr int R = 4;  // code ring slots per wave
  const BlobHeader& h = p->h;
  const int grid = pair_grid(h);
  size_t lds = pair_lds(h, grid);
  if (lds < kOneWorkgroupLds) lds = kOneWorkgroupLds;
  static const hipError_t attr =
      hipFuncSetAttribute((const void*)k_pair<R>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsBytes);
  if (attr != hipSuccess) return attr;
  const uint32_t meta_bytes = (uint32_t)(h.off_rowptr - h.off_meta);
  hipLaunchKernelGGL((k_pair<R>), dim3(grid), dim3(64 * kWaves), lds, st, p->blob + h.off_codes,
                     (const uint32_t*)(p->blob + h.off_meta), (const int32_t*)(p->blob + h.off_rowptr),
                     (const uint32_t*)(p->blob + h.off_entries), x, y, h.M, h.K, h.Kp, h.nkb, h.tiles, meta_bytes);
  return hipGetLastError();
}

// K-split batched kernel.  S splits of the K-blocks times NG tile groups
// (NG a multiple of 8 when it can be, so that a group's splits share an
// XCD), chunks of CH K-blocks.  LDS: x slice, chunk partials, staged block
// outlier offsets, counters, tables, and the 16 waves' 4 KiB outlier tiles.
struct SplitCfg {
  int S, NG, CH;
  size_t lds;
};

size_t split_lds(const BlobHeader& h, int nb, int S, int NG, int CH) {
  const size_t tw = (size_t)((h.tiles + NG - 1) / NG);
  const size_t kbm = (size_t)((h.nkb + S - 1) / S);
  const size_t cpt = (kbm + CH - 1) / CH;
  const size_t ob = (kbm + 4) & ~(size_t)3;
  const size_t tab = h.format == QGEMV_FMT_LUT ? (size_t)(2u << h.bits) : 0;  // table bytes per row
  return kbm * 256 * nb + tw * cpt * 16 * nb * 4 + tw * ob * 4 + 16 + tw * 16 * tab + (size_t)kWaves * 4096;
}

// The first (S, CH) in order of preference that fits: S = 4 keeps a quarter
// of x per CU with one read-back per group of four; S = 8 for long K.
// Single-block chunks where their partials fit (more chunks per wave, so the
// older waves of a SIMD take more of them), larger chunks otherwise.  The
// staged offsets of a workgroup must fit two per thread.
bool split_config(const BlobHeader& h, int nb, SplitCfg& c) {
  // Uniform codes only: LUT and BPDQ decodes are bound by the VALU, not by x.
  if (h.format != QGEMV_FMT_UNIFORM) return false;
  for (int S : {4, 8, 2}) {
    if (S > h.nkb) continue;
    int NG = h.tiles < kMaxGrid / S ? h.tiles : kMaxGrid / S;
    if (NG >= 8) NG &= ~7;
    const int tw = (h.tiles + NG - 1) / NG, kbm = (h.nkb + S - 1) / S;
    if (tw * ((kbm + 4) & ~3) > 2 * 64 * kWaves) continue;
    for (int CH : {1, 2, 4, 8}) {
      const size_t lds = split_lds(h, nb, S, NG, CH);
      if (lds > kLdsBytes) continue;
      c.S = S;
      c.NG = NG;
      c.CH = CH;
      c.lds = lds < kOneWorkgroupLds ? kOneWorkgroupLds : lds;
      return true;
    }
  }
  return false;
}

// Workspace of the K-split kernel: 1 KiB of counters (one per tile group),
// then the partials [S][tiles * 16][nb] fp32.
constexpr size_t kSplitCtrBytes = 1024;
size_t split_ws_bytes(const BlobHeader& h, int nb, const SplitCfg& c) {
  return kSplitCtrBytes + (size_t)c.S * h.tiles * 16 * nb * 4;
}

template <int FMT, int BITS, int NB, int CH>
hipError_t launch_split_ch(const qgemv_plan* p, const SplitCfg& c, const uint16_t* x, float* y, void* ws,
                           hipStream_t st) {
  const BlobHeader& h = p->h;
  static const hipError_t attr = hipFuncSetAttribute((const void*)k_split<FMT, BITS, NB, CH>,
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsBytes);
  if (attr != hipSuccess) return attr;
  const uint32_t codes_bytes = (uint32_t)((uint64_t)h.tiles * h.nkb * h.block_bytes);
  const uint32_t meta_bytes = (uint32_t)(h.off_rowptr - h.off_meta);
  hipLaunchKernelGGL((k_split<FMT, BITS, NB, CH>), dim3(c.NG * c.S), dim3(64 * kWaves), c.lds, st,
                     p->blob + h.off_codes, (const uint32_t*)(p->blob + h.off_meta),
                     (const int32_t*)(p->blob + h.off_boff), (const uint32_t*)(p->blob + h.off_bent), x, y,
                     (float*)((uint8_t*)ws + kSplitCtrBytes), (uint32_t*)ws, h.M, h.K, h.nkb, h.tiles, codes_bytes,
                     meta_bytes, (int)h.nnz, h.group_size > 0 ? h.group_size : 16, c.S, c.NG);
  return hipGetLastError();
}

template <int FMT, int BITS, int NB>
hipError_t launch_split(const qgemv_plan* p, const SplitCfg& c, const uint16_t* x, float* y, void* ws,
                        hipStream_t st) {
  if (c.CH == 1) return launch_split_ch<FMT, BITS, NB, 1>(p, c, x, y, ws, st);
  return c.CH == 2   ? launch_split_ch<FMT, BITS, NB, 2>(p, c, x, y, ws, st)
         : c.CH == 4 ? launch_split_ch<FMT, BITS, NB, 4>(p, c, x, y, ws, st)
                     : launch_split_ch<FMT, BITS, NB, 8>(p, c, x, y, ws, st);
}

// HPTQ: one workgroup per CU over its tile range; G = 3 blocks decoded side
// by side per wave where their buffers fit in LDS and their registers fit
// without spilling, else fewer.  Long codewords
// go through the second-level tables where they fit in LDS, else through the
// canonical search.  x sits in LDS at batch 1 and is read from L2 at 8/16.
template <int G, bool SUB, int NB>
hipError_t launch_huff_g(const qgemv_plan* p, const uint16_t* x, float* y, int grid, size_t lds, int bufw,
                         hipStream_t st) {
  const BlobHeader& h = p->h;
  static const hipError_t attr =
      hipFuncSetAttribute((const void*)k_huff<G, SUB, NB>, hipFuncAttributeMaxDynamicSharedMemorySize,
                          (int)(kLdsBytes - (size_t)kHuffTable * 64 * 4 - 64));
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL((k_huff<G, SUB, NB>), dim3(grid), dim3(64 * kWaves), lds, st,
                     (const uint32_t*)(p->blob + h.off_codes), (const uint16_t*)(p->blob + h.off_meta),
                     (const uint32_t*)(p->blob + h.off_hidx), (const uint16_t*)(p->blob + h.off_hlane),
                     (const int32_t*)(p->blob + h.off_htab), (const int16_t*)(p->blob + h.off_hsym), x, y, h.M, h.K,
                     h.nkb, h.tiles, h.hsym, h.hwords, bufw, (int)h.hsub);
  return hipGetLastError();
}

template <int NB>
hipError_t launch_huff_nb(const qgemv_plan* p, const uint16_t* x, float* y, hipStream_t st) {
  const BlobHeader& h = p->h;
  const int grid = h.tiles < kMaxGrid ? h.tiles : kMaxGrid;
  const size_t tw = (size_t)((h.tiles + grid - 1) / grid);
  const int bufw = (int)((h.hmaxw + kHuffPad + 3) / 4 * 4);
  const size_t table = (size_t)kHuffTable * 64 * 4 + 64;  // static LDS
  for (int sub = 1; sub >= 0; --sub) {
    const size_t aux =
        sub ? (size_t)kHuffSub * h.hsub * 4 : (size_t)(((h.hsym + 1) / 2 + 3) / 4 * 4) * 4;
    if (sub && h.hsub > (uint32_t)kHuffMaxSub) continue;
    const size_t fixed = (NB == 1 ? (size_t)h.K * 2 : 0) + aux + (tw + 15) * 16 * NB * 4 +
                         ((tw * (size_t)h.nkb + 4) & ~(size_t)3) * 4;
    // three chains spill registers at batch 16, and with the canonical search at batch 8
    for (int g = NB == 1 || (NB == 8 && sub) ? 3 : 2; g >= 1; --g) {
      size_t lds = fixed + (size_t)kWaves * g * bufw * 4;
      if (lds + table > kLdsBytes) continue;
      if (lds + table < kOneWorkgroupLds) lds = kOneWorkgroupLds - table;
      if (g == 3) {
        if constexpr (NB == 1)
          return sub ? launch_huff_g<3, true, NB>(p, x, y, grid, lds, bufw, st)
                     : launch_huff_g<3, false, NB>(p, x, y, grid, lds, bufw, st);
        else if constexpr (NB == 8)
          return launch_huff_g<3, true, NB>(p, x, y, grid, lds, bufw, st);
      }
      if (sub)
        return g == 2 ? launch_huff_g<2, true, NB>(p, x, y, grid, lds, bufw, st)
                      : launch_huff_g<1, true, NB>(p, x, y, grid, lds, bufw, st);
      return g == 2 ? launch_huff_g<2, false, NB>(p, x, y, grid, lds, bufw, st)
                    : launch_huff_g<1, false, NB>(p, x, y, grid, lds, bufw, st);
    }
  }
  return hipErrorInvalidValue;
}

hipError_t launch_huff(const qgemv_plan* p, const uint16_t* x, float* y, int batch, hipStream_t st) {
  return batch == 1   ? launch_huff_nb<1>(p, x, y, st)
         : batch == 8 ? launch_huff_nb<8>(p, x, y, st)
                      : launch_huff_nb<16>(p, x, y, st);
}

// ws: the K-split workspace for this batch (split_ws_bytes), or null to use
// the kernels that need none.
template <int FMT, int BITS>
hipError_t launch_run(const qgemv_plan* p, const uint16_t* x, float* y, int batch, void* ws, hipStream_t st) {
  if (batch == 1) {
    if (FMT == QGEMV_FMT_LUT && BITS == 4 && pair_fits(p->h)) return launch_pair(p, x, y, st);
    return launch_stream<FMT, BITS, 1>(p, x, y, st);
  }
  SplitCfg c;
  if (ws && split_config(p->h, batch, c))
    return batch == 8 ? launch_split<FMT, BITS, 8>(p, c, x, y, ws, st) : launch_split<FMT, BITS, 16>(p, c, x, y, ws, st);
  if (batch == 8)
    return xlds_fits(p->h, 8) ? launch_xlds<FMT, BITS, 8>(p, x, y, st) : launch_stream<FMT, BITS, 8>(p, x, y, st);
  return xlds_fits(p->h, 16) ? launch_xlds<FMT, BITS, 16>(p, x, y, st) : launch_stream<FMT, BITS, 16>(p, x, y, st);
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

// ---------------------------------------------------------------------------
// Streaming-read probe (measurement only, none of the method's arithmetic):
// reads `bytes` (a multiple of 16, at most 1 GiB) once with 16-byte
// non-temporal buffer loads, four in flight per lane, and XORs the dwords it
// read into one word per thread.  Thread t reads the 16-byte pieces t,
// t + T, t + 2T, ... (T threads in the grid), so sink[t] is the XOR of those
// pieces' dwords.  It gives the read ceiling the GEMV kernels are held against.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256)
k_read_probe(const uint8_t* __restrict__ src, uint32_t bytes, uint32_t* __restrict__ sink) {
  const rsrc_t r = make_rsrc(src, bytes);
  const uint32_t t = blockIdx.x * 256u + threadIdx.x, step = gridDim.x * 256u * 16u;
  uint32_t acc = 0;
  for (uint32_t i = t * 16u; i < bytes; i += 4u * step) {
    u32x4_t v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint32_t o = i + (uint32_t)u * step;
      v[u] = __builtin_amdgcn_raw_buffer_load_b128(r, (int)(o < bytes ? o : kOutOfRange), 0, kNonTemporal);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  sink[t] = acc;
}

int hip_status(hipError_t e) {
  if (e == hipSuccess) return QGEMV_OK;
  qgemv_set_hip_error((int)e);
  return QGEMV_ERR_HIP;
}

// Bytes of K-split workspace a plan's batched runs need (0 if none).
size_t plan_ws_need(const qgemv_plan* p) {
  size_t need = 0;
  for (int nb : {8, 16}) {
    SplitCfg c;
    if (split_config(p->h, nb, c)) {
      const size_t b = split_ws_bytes(p->h, nb, c);
      if (b > need) need = b;
    }
  }
  return need;
}

// The plan's workspace, allocated on the plan's device by its first batched
// run: counters cleared (in stream order, before the first use), partials
// left as they are (every launch writes the partials it reads).  A run under
// stream capture cannot allocate it and fails instead.
int plan_workspace(qgemv_plan* p, hipStream_t st, void** ws) {
  *ws = nullptr;
  const size_t need = plan_ws_need(p);
  if (need == 0) return QGEMV_OK;
  std::lock_guard<std::mutex> lock(p->ws_mu);
  if (!p->ws) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    hipError_t e = hipStreamIsCapturing(st, &cs);
    if (e != hipSuccess) return hip_status(e);
    if (cs != hipStreamCaptureStatusNone) return QGEMV_ERR_INVALID_ARG;
    int cur = 0;
    e = hipGetDevice(&cur);
    if (e != hipSuccess) return hip_status(e);
    if (cur != p->device && (e = hipSetDevice(p->device)) != hipSuccess) return hip_status(e);
    void* mem = nullptr;
    e = hipMalloc(&mem, need);
    if (e == hipSuccess) e = hipMemsetAsync(mem, 0, kSplitCtrBytes, st);
    if (cur != p->device) (void)hipSetDevice(cur);
    if (e != hipSuccess) {
      if (mem) (void)hipFree(mem);
      return hip_status(e);
    }
    p->ws = mem;
    p->ws_bytes = need;
  }
  *ws = p->ws;
  return QGEMV_OK;
}

// Device address of `scratch` on device dev, looked up once per device with
// that device current.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices];

int scratch_address(int dev, void** out) {
  *out = nullptr;
  if (dev < 0 || dev >= kMaxDevices) return QGEMV_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    int cur = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return hip_status(e);
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return hip_status(e);
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (cur != dev) (void)hipSetDevice(cur);
    if (e != hipSuccess) return hip_status(e);
    if (!ptr) return QGEMV_ERR_HIP;
    g_scratch_dev[dev] = ptr;
  }
  *out = g_scratch_dev[dev];
  return QGEMV_OK;
}

hipError_t launch_format(const qgemv_plan* p, const uint16_t* x, float* y, int batch, void* ws, hipStream_t st) {
  const bool b4 = p->h.bits == 4;
  if (p->h.format == QGEMV_FMT_HPTQ) return launch_huff(p, x, y, batch, st);
  if (p->h.format == QGEMV_FMT_LUT)
    return b4 ? launch_run<QGEMV_FMT_LUT, 4>(p, x, y, batch, ws, st) : launch_run<QGEMV_FMT_LUT, 3>(p, x, y, batch, ws, st);
  if (p->h.format == QGEMV_FMT_BPDQ) return launch_run<QGEMV_FMT_BPDQ, 3>(p, x, y, batch, ws, st);
  return b4 ? launch_run<QGEMV_FMT_UNIFORM, 4>(p, x, y, batch, ws, st)
            : launch_run<QGEMV_FMT_UNIFORM, 3>(p, x, y, batch, ws, st);
}

}  // namespace

extern "C" {

int qgemv_create(qgemv_handle* out, const qgemv_weights* shape, const void* packed_dev, size_t bytes) {
  if (!out || !shape || !packed_dev) return QGEMV_ERR_INVALID_ARG;
  *out = nullptr;
  const int st = qgemv_validate_shape(shape);
  if (st) return st;
  if ((uintptr_t)packed_dev % kAlign) return QGEMV_ERR_INVALID_ARG;
  const bool hptq = shape->format == QGEMV_FMT_HPTQ;
  BlobHeader expect =
      make_header(shape->M, shape->K, shape->bits, shape->format, shape->group_size, shape->nnz, shape->huff_nsym, 0);
  if (bytes < expect.total_bytes) return QGEMV_ERR_SIZE;
  BlobHeader got;
  const hipError_t e = hipMemcpy(&got, packed_dev, sizeof(got), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_status(e);
  if (hptq) {  // the code section's size comes from the stream, so from the blob
    if (got.hmaxw % 4 || got.hmaxw > (uint32_t)kHuffMaxBlockWords || got.hmaxw > got.hwords) return QGEMV_ERR_SIZE;
    if (got.hsub < 1 || got.hsub > (uint32_t)shape->huff_nsym) return QGEMV_ERR_SIZE;
    expect = make_header(shape->M, shape->K, shape->bits, shape->format, shape->group_size, shape->nnz,
                         shape->huff_nsym, got.hwords, got.hmaxw, got.hsub);
    if (bytes < expect.total_bytes) return QGEMV_ERR_SIZE;
  }
  if (std::memcmp(&got, &expect, sizeof(got)) != 0) return QGEMV_ERR_SIZE;
  int dev = 0;
  const hipError_t de = hipGetDevice(&dev);
  if (de != hipSuccess) return hip_status(de);
  qgemv_plan* p = new (std::nothrow) qgemv_plan{expect, (const uint8_t*)packed_dev, dev};
  if (!p) return QGEMV_ERR_INVALID_ARG;
  *out = p;
  return QGEMV_OK;
}

int qgemv_run(qgemv_handle h, const void* x_dev, float* y_dev, int32_t batch, void* stream) {
  if (!h || !x_dev || !y_dev) return QGEMV_ERR_INVALID_ARG;
  if ((uintptr_t)x_dev % 16 || (uintptr_t)y_dev % 16) return QGEMV_ERR_INVALID_ARG;
  if (batch != 1 && batch != 8 && batch != 16) return QGEMV_ERR_UNSUPPORTED;
  const hipStream_t st = (hipStream_t)stream;
  void* ws = nullptr;
  if (batch > 1) {
    const int stw = plan_workspace(h, st, &ws);
    if (stw != QGEMV_OK) return stw;
  }
  return hip_status(launch_format(h, (const uint16_t*)x_dev, y_dev, batch, ws, st));
}

int qgemv_run_noalloc(qgemv_handle h, const void* x_dev, float* y_dev, int32_t batch, void* stream) {
  if (!h || !x_dev || !y_dev) return QGEMV_ERR_INVALID_ARG;
  if ((uintptr_t)x_dev % 16 || (uintptr_t)y_dev % 16) return QGEMV_ERR_INVALID_ARG;
  if (batch != 1 && batch != 8 && batch != 16) return QGEMV_ERR_UNSUPPORTED;
  void* ws = nullptr;
  SplitCfg c;
  if (batch > 1 && split_config(h->h, batch, c)) {
    if (split_ws_bytes(h->h, batch, c) > kScratchBytes) return QGEMV_ERR_SCRATCH;
    const int sts = scratch_address(h->device, &ws);
    if (sts != QGEMV_OK) return sts;
  }
  return hip_status(launch_format(h, (const uint16_t*)x_dev, y_dev, batch, ws, (hipStream_t)stream));
}

int qgemv_debug_unpack(qgemv_handle h, uint8_t* codes_dev, void* stream) {
  if (!h || !codes_dev) return QGEMV_ERR_INVALID_ARG;
  if (h->h.format == QGEMV_FMT_HPTQ) return QGEMV_ERR_UNSUPPORTED;
  if ((uintptr_t)codes_dev % 16) return QGEMV_ERR_INVALID_ARG;
  const hipStream_t st = (hipStream_t)stream;
  hipError_t e;
  if (h->h.format == QGEMV_FMT_LUT || h->h.format == QGEMV_FMT_BPDQ)  // BPDQ codes use the L3 placement
    e = h->h.bits == 4 ? launch_unpack<QGEMV_FMT_LUT, 4>(h, codes_dev, st)
                       : launch_unpack<QGEMV_FMT_LUT, 3>(h, codes_dev, st);
  else
    e = h->h.bits == 4 ? launch_unpack<QGEMV_FMT_UNIFORM, 4>(h, codes_dev, st)
                       : launch_unpack<QGEMV_FMT_UNIFORM, 3>(h, codes_dev, st);
  return hip_status(e);
}

int qgemv_read_probe(const void* src_dev, uint64_t bytes, uint32_t* sink_dev, int32_t sink_words, void* stream) {
  if (!src_dev || !sink_dev || (uintptr_t)src_dev % 16 || (uintptr_t)sink_dev % 4) return QGEMV_ERR_INVALID_ARG;
  if (bytes == 0 || bytes % 16 || bytes > (1ull << 30) || sink_words < 256) return QGEMV_ERR_INVALID_ARG;
  const int grid = sink_words / 256 < 1024 ? sink_words / 256 : 1024;
  hipLaunchKernelGGL(k_read_probe, dim3(grid), dim3(256), 0, (hipStream_t)stream, (const uint8_t*)src_dev,
                     (uint32_t)bytes, sink_dev);
  return hip_status(hipGetLastError());
}

int qgemv_destroy(qgemv_handle h) {
  if (h && h->ws) (void)hipFree(h->ws);
  delete h;
  return QGEMV_OK;
}

}  // extern "C"
