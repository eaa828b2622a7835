// sa_device.h — device-side helpers for the gfx950 Sketch Attention kernels:
// vector types, MFMA wrappers and the ragged tile/chunk lookups.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sa_layout.h"

namespace sa {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float float16v __attribute__((ext_vector_type(16)));
typedef float float2v __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Word 3 of a gfx9 buffer resource for raw (unformatted) 32-bit data.  With
// stride 0 the hardware drops stores and returns zeros for loads at byte
// offsets at or beyond the resource's record count.
constexpr int kBufferRsrcWord3 = 0x00020000;

// D = A(32x16) * B(16x32) + C on the matrix cores, fp16 operands, fp32 sums.
// Lane l holds row (l % 32) of A and column (l % 32) of B, 8 contraction
// elements each from half (l / 32) of the 16; the same element slot pairs up
// in A and B, so any consistent assignment of contraction indices to slots is
// valid.  Result: lane l, register r holds C[8*(r/4) + 4*(l/32) + r%4][l % 32].
__device__ __forceinline__ float16v mfma32x32x16(half8 a, half8 b, float16v c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// Row of the 32x32 accumulator held in register r by lane half g.
__device__ __forceinline__ int acc_row(int r, int g) { return 8 * (r >> 2) + 4 * g + (r & 3); }

// Workgroup barrier for LDS only: this wave's LDS operations are complete,
// then s_barrier.  Global loads and stores (direct-to-LDS loads included) stay
// in flight; a language-level barrier also fences global memory and so waits
// for every outstanding load of the wave, prefetches included.  Data that a
// direct-to-LDS load writes is visible to other waves after the issuing wave's
// own vmcnt wait and then this barrier.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Row pitch of a padded fp16 token tile in LDS: 2d + 16 bytes (token t's
// 16-byte chunk c at t * pitch + 16 c; the extra chunk shifts consecutive
// rows by 4 of the 64 banks).
template <int D>
constexpr int tile_pitch() { return (D / 8 + 1) * 16; }

// Token held by pass 2's GEMM1 operand row m (m = 16 kk + 8 h + 4 g + e in
// bits): 16 kk + 4 e + 2 g + h.  GEMM1's accumulator rows are GEMM2's
// contraction order, so the 4 tokens of one transposing read of GEMM2's
// operand lie 4 rows apart in LDS, which with the padded pitch keeps every
// read conflict-free.
__device__ __forceinline__ int tau(int m) {
  return (m & 16) | ((m & 3) << 2) | (((m >> 2) & 1) << 1) | ((m >> 3) & 1);
}

// 32-bit LDS address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// GEMM2's B operands from one padded fp16 token tile in LDS (row pitch
// tile_pitch<D>()), with the gfx950 transposing read ds_read_b64_tr_b16:
// within each group of 16 lanes, destination lane i receives element i % 4 of
// the 4-element vectors that source lanes i/4, i/4 + 4, i/4 + 8, i/4 + 12
// address.  `addr` is the tile's LDS address plus the lane's offset (source
// lane i16 of 16-lane group gh, lane half g: row 4 (i16 / 4) + 2 g, column
// 16 gh + 4 (i16 % 4)); hb[kk][dt] = the reads at rows + 16 kk (lo) and
// + 16 kk + 1 (hi), columns + 32 dt.  Written with its wait in one asm
// block: while direct loads into LDS are in flight, the compiler puts a wait
// for every outstanding vector-memory operation (all prefetches) in front of
// the builtin form of this read.
template <int D>
__device__ __forceinline__ void tile_tr_reads(uint32_t addr, half8 (&hb)[2][D / 32]) {
  static_assert(D == 128 || D == 64, "d = 64 or 128");
  if constexpr (D == 128) {
    static_assert(tile_pitch<128>() == 272, "offsets below: 16 kk 272 + 64 dt (+ 272)");
    s16x4 r0, r1, r2, r3, r4, r5, r6, r7, r8, r9, r10, r11, r12, r13, r14, r15;
    asm volatile(
        "ds_read_b64_tr_b16 %0, %16\n\t"
        "ds_read_b64_tr_b16 %1, %16 offset:272\n\t"
        "ds_read_b64_tr_b16 %2, %16 offset:64\n\t"
        "ds_read_b64_tr_b16 %3, %16 offset:336\n\t"
        "ds_read_b64_tr_b16 %4, %16 offset:128\n\t"
        "ds_read_b64_tr_b16 %5, %16 offset:400\n\t"
        "ds_read_b64_tr_b16 %6, %16 offset:192\n\t"
        "ds_read_b64_tr_b16 %7, %16 offset:464\n\t"
        "ds_read_b64_tr_b16 %8, %16 offset:4352\n\t"
        "ds_read_b64_tr_b16 %9, %16 offset:4624\n\t"
        "ds_read_b64_tr_b16 %10, %16 offset:4416\n\t"
        "ds_read_b64_tr_b16 %11, %16 offset:4688\n\t"
        "ds_read_b64_tr_b16 %12, %16 offset:4480\n\t"
        "ds_read_b64_tr_b16 %13, %16 offset:4752\n\t"
        "ds_read_b64_tr_b16 %14, %16 offset:4544\n\t"
        "ds_read_b64_tr_b16 %15, %16 offset:4816\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3), "=&v"(r4), "=&v"(r5), "=&v"(r6), "=&v"(r7), "=&v"(r8),
          "=&v"(r9), "=&v"(r10), "=&v"(r11), "=&v"(r12), "=&v"(r13), "=&v"(r14), "=&v"(r15)
        : "v"(addr));
    const s16x4 r[16] = {r0, r1, r2, r3, r4, r5, r6, r7, r8, r9, r10, r11, r12, r13, r14, r15};
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const s16x4 lo = r[8 * kk + 2 * dt], hi = r[8 * kk + 2 * dt + 1];
        hb[kk][dt] = __builtin_bit_cast(half8, s16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
      }
  } else {
    static_assert(tile_pitch<64>() == 144, "offsets below: 16 kk 144 + 64 dt (+ 144)");
    s16x4 r0, r1, r2, r3, r4, r5, r6, r7;
    asm volatile(
        "ds_read_b64_tr_b16 %0, %8\n\t"
        "ds_read_b64_tr_b16 %1, %8 offset:144\n\t"
        "ds_read_b64_tr_b16 %2, %8 offset:64\n\t"
        "ds_read_b64_tr_b16 %3, %8 offset:208\n\t"
        "ds_read_b64_tr_b16 %4, %8 offset:2304\n\t"
        "ds_read_b64_tr_b16 %5, %8 offset:2448\n\t"
        "ds_read_b64_tr_b16 %6, %8 offset:2368\n\t"
        "ds_read_b64_tr_b16 %7, %8 offset:2512\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3), "=&v"(r4), "=&v"(r5), "=&v"(r6), "=&v"(r7)
        : "v"(addr));
    const s16x4 r[8] = {r0, r1, r2, r3, r4, r5, r6, r7};
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int dt = 0; dt < 2; ++dt) {
        const s16x4 lo = r[4 * kk + 2 * dt], hi = r[4 * kk + 2 * dt + 1];
        hb[kk][dt] = __builtin_bit_cast(half8, s16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
      }
  }
}

// Half of tile_tr_reads: the B operands of one contraction step kk, read
// at `addr` = the tile's LDS address + the lane's offset + 16 kk rows
// (hb[dt] = hb[kk][dt] of tile_tr_reads).  Same wait-inside-the-asm rule.
template <int D>
__device__ __forceinline__ void tile_tr_reads_kk(uint32_t addr, half8 (&hb)[D / 32]) {
  static_assert(D == 128 || D == 64, "d = 64 or 128");
  if constexpr (D == 128) {
    s16x4 r0, r1, r2, r3, r4, r5, r6, r7;
    asm volatile(
        "ds_read_b64_tr_b16 %0, %8\n\t"
        "ds_read_b64_tr_b16 %1, %8 offset:272\n\t"
        "ds_read_b64_tr_b16 %2, %8 offset:64\n\t"
        "ds_read_b64_tr_b16 %3, %8 offset:336\n\t"
        "ds_read_b64_tr_b16 %4, %8 offset:128\n\t"
        "ds_read_b64_tr_b16 %5, %8 offset:400\n\t"
        "ds_read_b64_tr_b16 %6, %8 offset:192\n\t"
        "ds_read_b64_tr_b16 %7, %8 offset:464\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3), "=&v"(r4), "=&v"(r5), "=&v"(r6), "=&v"(r7)
        : "v"(addr));
    const s16x4 r[8] = {r0, r1, r2, r3, r4, r5, r6, r7};
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      const s16x4 lo = r[2 * dt], hi = r[2 * dt + 1];
      hb[dt] = __builtin_bit_cast(half8, s16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
    }
  } else {
    s16x4 r0, r1, r2, r3;
    asm volatile(
        "ds_read_b64_tr_b16 %0, %4\n\t"
        "ds_read_b64_tr_b16 %1, %4 offset:144\n\t"
        "ds_read_b64_tr_b16 %2, %4 offset:64\n\t"
        "ds_read_b64_tr_b16 %3, %4 offset:208\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3)
        : "v"(addr));
    const s16x4 r[4] = {r0, r1, r2, r3};
#pragma unroll
    for (int dt = 0; dt < 2; ++dt) {
      const s16x4 lo = r[2 * dt], hi = r[2 * dt + 1];
      hb[dt] = __builtin_bit_cast(half8, s16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
    }
  }
}

// Exact widening of 8 packed bf16 values (one 16-byte load) to fp16.  bf16
// values whose magnitude lies in [2^-17, 65504] are exactly representable in
// fp16; the conversion truncates toward zero so larger values saturate.
__device__ __forceinline__ half8 bf16x8_to_f16x8(u32x4 v) {
  half8 out;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float lo = __uint_as_float(v[i] << 16);
    float hi = __uint_as_float(v[i] & 0xffff0000u);
    half2v p = __builtin_bit_cast(half2v, __builtin_amdgcn_cvt_pkrtz(lo, hi));
    out[2 * i] = p[0];
    out[2 * i + 1] = p[1];
  }
  return out;
}

// Nonzero if one of 8 packed bf16 values (one 16-byte load) lies outside
// fp16's finite range: |x| > 65504, an infinity or a NaN.  With the sign
// cleared, bf16 magnitudes order like their bit patterns, and 0x477F (65280)
// is the largest bf16 value not above 65504; adding 0x3880 to a cleared half
// carries into its bit 15 exactly when the half exceeds 0x477F, and never
// into the other half (0x7FFF + 0x3880 < 0x10000).
__device__ __forceinline__ uint32_t bf16x8_range_bits(u32x4 v) {
  uint32_t bad = 0u;
#pragma unroll
  for (int i = 0; i < 4; ++i) bad |= ((v[i] & 0x7FFF7FFFu) + 0x38803880u) & 0x80008000u;
  return bad;
}

// Largest u with base[u] <= x, for a non-decreasing base[0..R] with base[0] = 0
// and x < base[R].  Users with no tiles (base[u] == base[u+1]) are skipped.
__device__ __forceinline__ int find_user(const int32_t* base, int R, int32_t x) {
  int lo = 0, hi = R;  // invariant: base[lo] <= x < base[hi]
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (base[mid] <= x) lo = mid; else hi = mid;
  }
  return lo;
}

__device__ __forceinline__ int32_t* ws_i32(void* ws, size_t off) {
  return reinterpret_cast<int32_t*>(reinterpret_cast<char*>(ws) + off);
}
__device__ __forceinline__ float* ws_f32(void* ws, size_t off) {
  return reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + off);
}
__device__ __forceinline__ _Float16* ws_f16(void* ws, size_t off) {
  return reinterpret_cast<_Float16*>(reinterpret_cast<char*>(ws) + off);
}

// The largest row norm of the fp16 queries: the maximum of the per-32-row
// maxima the preparation writes (in every lane of the calling wave).
__device__ __forceinline__ float query_norm_max(const Layout& L, void* ws) {
  const float* qp = ws_f32(ws, L.off_qpart);
  float m = 0.f;
  for (int i = threadIdx.x & 63; i < L.k / 32; i += 64) m = fmaxf(m, qp[i]);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  return m;
}

// Where a tile lives: user, first token (packed index) and valid row count.
struct TileInfo {
  int user;
  int64_t tok0;
  int count;
};

__device__ __forceinline__ TileInfo tile_info(const int32_t* tile_base, const int64_t* offsets,
                                              int R, int32_t tile) {
  TileInfo t;
  t.user = find_user(tile_base, R, tile);
  int32_t i = tile - tile_base[t.user];
  int64_t lo = offsets[t.user], hi = offsets[t.user + 1];
  t.tok0 = lo + (int64_t)i * kTile;
  int64_t rem = hi - t.tok0;
  t.count = rem < kTile ? (int)rem : kTile;
  return t;
}

}  // namespace sa
