// sa_pass1.hip — FlashSA pass 1 on gfx950 (bf16 inputs).
//
// Sketch Attention normalises each token's logits across the k prototypes
// (SequenceO1 review page, FAQ on how SA differs from standard attention;
// blog "How it works" item 1: every item spreads its mass over the
// prototypes).  Pass 1 computes, for every token t, the base-2 logsumexp
//     lse_t = log2 sum_j 2^(q_j . h_t)
// over ALL k prototypes without materialising the k x n logit matrix (blog
// "How it works" item 3: FlashSA avoids the huge intermediates), and emits
// the token in the form pass 2 consumes:
//   * the fp16 row h_t (bf16 widened exactly),
//   * -l_t = -(lse_t - 14) as two fp16 parts (hi, lo), the token's entries of
//     pass 2's extra MFMA K step, so that step subtracts l_t from every logit
//     (the 2^14 keeps fp16 allocations in the normal range).
// Masked tokens and tile padding get zero rows and -l = -60000, i.e. A = 0.
//
// Layout: one workgroup = 4 waves = 8 tiles (256 tokens).  Each wave keeps the
// fp16 history of its 2 tiles in registers as MFMA B operands (lane = token)
// and streams the prototype queries through LDS in chunks of 128 (direct
// global->LDS loads, double-buffered, rows XOR-swizzled for the 64-bank
// LDS), computing S[j, t] = Q H^T with v_mfma_f32_32x32x16_f16.  The
// accumulator layout puts one token per lane, so the reduction over
// prototypes stays in the lane.
//
// Exponent range: every logit obeys |q_j . h_t| <= qmax |h_t| (Cauchy-Schwarz,
// qmax = largest query norm).  When that bound is below 100 for every token of
// the workgroup, 2^L can neither overflow nor leave the normal range, so the
// sum is taken without a running maximum (one exp and one add per logit).
// Otherwise the workgroup runs the exact two-sweep form (maximum, then the
// shifted sum).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "sa_device.h"
#include "sa_launch.h"

namespace sa {

namespace {

constexpr int kModeFast = 0;   // sum of 2^L
constexpr int kModeMax = 1;    // running max of L
constexpr int kModeShift = 2;  // sum of 2^(L - max)
constexpr int kQC = 128;       // prototypes per LDS chunk

template <int D>
struct P1 {
  static constexpr int S = D / 16;                   // MFMA K steps over d
  static constexpr int CPR = D / 8;                  // 16-B chunks per query row
  static constexpr int ROWSH = (CPR == 16) ? 0 : 1;
  static constexpr int CHUNK_BYTES = kQC * D * 2;    // one LDS query chunk
  static constexpr int LOADS = CHUNK_BYTES / 1024;   // 1-KB direct loads per chunk
};

template <int D>
__device__ __forceinline__ int swz(int row) {
  return (row >> P1<D>::ROWSH) & (P1<D>::CPR - 1);
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Direct loads of query chunk c (rows c*128 .. +127) into LDS buffer `dst`.
template <int D>
__device__ __forceinline__ void issue_chunk(const char* q16, int c, int nrows, char* dst, int wave, int lane) {
  using C = P1<D>;
#pragma unroll
  for (int i = wave; i < C::LOADS; i += 4) {
    const int q = 64 * i + lane;
    const int row = q / C::CPR, cs = q % C::CPR;
    if (row >= nrows) break;   // uniform: a 64-prototype last chunk
    const int cl = cs ^ swz<D>(row);
    const char* src = q16 + ((int64_t)c * kQC + row) * (D * 2) + cl * 16;
    __builtin_amdgcn_global_load_lds(src, (lds_ptr_t)(dst + 1024 * i), 16, 0, 0);
  }
}

// Reduce one 32-prototype group of logits (two 32-token tiles, 16 values per
// lane each) into the per-lane running statistics.
template <int MODE>
__device__ __forceinline__ void reduce_group(const float16v (&acc)[2], float (&acc_sum)[2], float (&acc_max)[2]) {
#pragma unroll
  for (int tau = 0; tau < 2; ++tau) {
    if (MODE == kModeFast) {
      float s0 = 0.f, s1 = 0.f;
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        s0 += __builtin_amdgcn_exp2f(acc[tau][r]);
        s1 += __builtin_amdgcn_exp2f(acc[tau][r + 1]);
      }
      acc_sum[tau] += s0 + s1;
    } else if (MODE == kModeMax) {
      float m = acc_max[tau];
#pragma unroll
      for (int r = 0; r < 16; ++r) m = fmaxf(m, acc[tau][r]);
      acc_max[tau] = m;
    } else {
      float s0 = 0.f, s1 = 0.f;
      const float mx = acc_max[tau];
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        s0 += __builtin_amdgcn_exp2f(acc[tau][r] - mx);
        s1 += __builtin_amdgcn_exp2f(acc[tau][r + 1] - mx);
      }
      acc_sum[tau] += s0 + s1;
    }
  }
}

// One sweep over all k prototypes.  Software-pipelined over 32-prototype
// groups: the MFMAs of group i are issued interleaved with the reduction of
// group i-1 (independent work), so the exponentials run under the matrix
// cores.  The pending group starts at -inf, which every reduction ignores.
template <int D, int MODE>
__device__ __forceinline__ void sweep(const char* q16, int k, char* lds, const half8 (&hreg)[2][P1<D>::S],
                                      float (&acc_sum)[2], float (&acc_max)[2], int wave, int lane, int col, int g) {
  using C = P1<D>;
  const int nchunks = (k + kQC - 1) / kQC;
  float16v pend[2];
#pragma unroll
  for (int tau = 0; tau < 2; ++tau)
#pragma unroll
    for (int r = 0; r < 16; ++r) pend[tau][r] = -INFINITY;
  issue_chunk<D>(q16, 0, min(kQC, k), lds, wave, lane);
  for (int c = 0; c < nchunks; ++c) {
    char* cur = lds + (c & 1) * C::CHUNK_BYTES;
    const int npt = min(kQC, k - c * kQC) / 32;
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's loads of chunk c landed
    __syncthreads();                     // ... and everyone's; chunk c-1's buffer is free
    if (c + 1 < nchunks)
      issue_chunk<D>(q16, c + 1, min(kQC, k - (c + 1) * kQC), lds + ((c + 1) & 1) * C::CHUNK_BYTES, wave, lane);
#pragma unroll
    for (int pt = 0; pt < kQC / 32; ++pt) {
      if (pt < npt) {   // uniform; false only in a 64-prototype last chunk
        const int row = pt * 32 + col;
        half8 af[C::S];
#pragma unroll
        for (int s = 0; s < C::S; ++s) {
          const int cl = (2 * s + g) ^ swz<D>(row);
          af[s] = *reinterpret_cast<const half8*>(cur + row * (D * 2) + cl * 16);
        }
        float16v acc[2] = {float16v{}, float16v{}};
#pragma unroll
        for (int s = 0; s < C::S; ++s)
#pragma unroll
          for (int tau = 0; tau < 2; ++tau) acc[tau] = mfma32x32x16(af[s], hreg[tau][s], acc[tau]);
        reduce_group<MODE>(pend, acc_sum, acc_max);
#pragma unroll
        for (int i = 0; i < 2 * C::S; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // 1 MFMA
          __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);  // 4 VALU
        }
        pend[0] = acc[0];
        pend[1] = acc[1];
      }
    }
  }
  reduce_group<MODE>(pend, acc_sum, acc_max);
  __syncthreads();  // all waves are done with the last chunk before LDS is reused
}

}  // namespace

template <int D>
__global__ __launch_bounds__(256) void pass1_lse(const uint16_t* __restrict__ H, const int64_t* __restrict__ offsets,
                                                 const uint8_t* __restrict__ mask, Layout L, void* ws) {
  using C = P1<D>;
  __shared__ __attribute__((aligned(1024))) char lds[2 * C::CHUNK_BYTES];
  const int32_t* hdr = ws_i32(ws, L.off_hdr);
  const int32_t total_tiles = hdr[kHdrTiles];
  const int32_t tile0 = blockIdx.x * kPass1Tiles;
  if (tile0 >= total_tiles) return;  // uniform over the workgroup
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, g = lane >> 5;
  const int32_t* tile_base = ws_i32(ws, L.off_tile_base);
  const float qmax = query_norm_max(L, ws);

  half8 hreg[2][C::S];
  bool valid[2];
  int32_t tiles[2];
  bool need_exact = false;
  uint32_t range_bad = 0u;   // kept values outside fp16's finite range
#pragma unroll
  for (int tau = 0; tau < 2; ++tau) {
    const int32_t tile = tile0 + 2 * wave + tau;
    tiles[tau] = tile;
    valid[tau] = false;
#pragma unroll
    for (int s = 0; s < C::S; ++s) hreg[tau][s] = half8{};
    if (tile < total_tiles) {
      TileInfo ti = tile_info(tile_base, offsets, L.R, tile);
      if (col < ti.count) {
        const int64_t tok = ti.tok0 + col;
        valid[tau] = (mask == nullptr) || (mask[tok] != 0);
        if (valid[tau]) {
          const u32x4* src = reinterpret_cast<const u32x4*>(H + tok * D);
#pragma unroll
          for (int s = 0; s < C::S; ++s) {
            const u32x4 raw = src[2 * s + g];
            range_bad |= bf16x8_range_bits(raw);
            hreg[tau][s] = bf16x8_to_f16x8(raw);
          }
        }
      }
    }
    float n2 = 0.f;
#pragma unroll
    for (int s = 0; s < C::S; ++s)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float v = (float)hreg[tau][s][e];
        n2 = fmaf(v, v, n2);
      }
    n2 += __shfl_xor(n2, 32);
    if (valid[tau] && qmax * sqrtf(n2) >= 100.0f) need_exact = true;
  }
  need_exact = __syncthreads_or(need_exact);
  if (__ballot(range_bad != 0u) != 0ull && lane == 0) atomicOr(ws_i32(ws, L.off_hdr) + kHdrErr, kErrRange);

  const char* q16 = reinterpret_cast<const char*>(ws_f16(ws, L.off_q16));
  float sum[2] = {0.f, 0.f};
  float mx[2] = {-INFINITY, -INFINITY};
  if (!need_exact) {
    sweep<D, kModeFast>(q16, L.k, lds, hreg, sum, mx, wave, lane, col, g);
  } else {
    sweep<D, kModeMax>(q16, L.k, lds, hreg, sum, mx, wave, lane, col, g);
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) mx[tau] = fmaxf(mx[tau], __shfl_xor(mx[tau], 32));
    sweep<D, kModeShift>(q16, L.k, lds, hreg, sum, mx, wave, lane, col, g);
  }

  _Float16* h16 = ws_f16(ws, L.off_h16);
  uint32_t* nl = reinterpret_cast<uint32_t*>(ws_i32(ws, L.off_nl));
#pragma unroll
  for (int tau = 0; tau < 2; ++tau) {
    const int32_t tile = tiles[tau];
    if (tile >= total_tiles) continue;
    const float tot = sum[tau] + __shfl_xor(sum[tau], 32);
    const float lse = need_exact ? mx[tau] + log2f(tot) : log2f(tot);
    _Float16* dst = h16 + ((int64_t)tile * kTile + col) * D;
#pragma unroll
    for (int s = 0; s < C::S; ++s) *reinterpret_cast<half8*>(dst + 16 * s + 8 * g) = hreg[tau][s];
    if (g == 0) {
      // -l = 14 - lse as an fp16 pair (hi, lo) with hi + lo = -l to ~2^-16
      const float nlv = valid[tau] ? kAllocShift - lse : -60000.0f;
      const _Float16 hi = (_Float16)nlv;
      const _Float16 lo = valid[tau] ? (_Float16)(nlv - (float)hi) : (_Float16)0.0f;
      half2v pr = {hi, lo};
      nl[(int64_t)tile * kTile + col] = __builtin_bit_cast(uint32_t, pr);
    }
  }
}

hipError_t launch_pass1(const Layout& L, const void* H, const int64_t* offsets, const uint8_t* mask, void* ws,
                        hipStream_t stream) {
  const int grid = (L.tiles_max + kPass1Tiles - 1) / kPass1Tiles;
  if (grid == 0) return hipSuccess;
  if (L.d == 128)
    hipLaunchKernelGGL(pass1_lse<128>, dim3(grid), dim3(256), 0, stream, (const uint16_t*)H, offsets, mask, L, ws);
  else
    hipLaunchKernelGGL(pass1_lse<64>, dim3(grid), dim3(256), 0, stream, (const uint16_t*)H, offsets, mask, L, ws);
  return hipGetLastError();
}

}  // namespace sa
