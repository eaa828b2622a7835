// sa_target.hip — sketch-branch target attention on gfx950.
//
// After compression, each candidate item attends over its user's fixed-size
// sketch (blog "100,000 videos in your pocket", "How it works" item 2: the
// sketch branch of STCA), and one user's many candidates share one read of
// that sketch (same page, item 3: multi-request user-level batching).  The
// pages define STCA's stacking only by reference to an earlier paper, so
// this is the single-layer reading: for candidate query q_c of user u and
// the user's sketch rows s_j (keys and values at once)
//     out_c = sum_j softmax_j(q_c . s_j / sqrt(d)) s_j.
//
// Work split: the candidates of every user are cut into tiles of 32, the
// tile count rounded up to a multiple of 4 (the forward's schedule kernel
// computes these prefix sums from the candidate offsets); a workgroup of 4
// waves takes 4 consecutive tiles, all of one user, so each staged sketch
// block serves 128 candidates, and the workgroups of one user run on one
// XCD so that its L2 serves the user's sketch to all of them.  Per wave:
//   the 32 candidate queries are the B operand of C[j, c] = s_j . q_c (fp16
//   widened exactly from bf16, kept in registers); the user's sketch is
//   staged block by block (32 rows, fp32 -> fp16) in LDS;
//   per block: the logits, the block maximum (both lane halves), the
//   running maximum m and sum l per candidate (lane = candidate), P =
//   2^(logit - m) in fp16 -- the accumulator registers are exactly the A
//   operand of out = P s (candidate = lane, sketch rows in the transposing
//   read's order) -- and out += P s with B operands from the staged block
//   through ds_read_b64_tr_b16.  m moves only when a logit exceeds it by
//   more than 2^8 (then out and l are rescaled by 2^(m_old - m)), so after
//   the first blocks the rescale is rare.  The output rows sit in another
//   lane layout than the per-candidate statistics, so the rescale factors
//   (and finally 1 / l) pass through a small per-wave LDS area.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <algorithm>

#include "sa_device.h"
#include "sa_launch.h"

namespace sa {

template <int D>
__global__ __launch_bounds__(256, 2) void ta_attend(const uint16_t* __restrict__ Q,
                                                    const int64_t* __restrict__ cand_offsets,
                                                    const float* __restrict__ Sk,
                                                    const int32_t* __restrict__ sketch_rows, int64_t sketch_count,
                                                    const int32_t* __restrict__ tile_base, Layout L, void* ws,
                                                    float* __restrict__ out, float* __restrict__ lse_out) {
  constexpr int S = D / 16, DT = D / 32, PITCH = tile_pitch<D>(), BLK = kTile * PITCH;
  constexpr int F4R = D / 4;                  // float4 per sketch row
  constexpr int LPT = kTile * F4R / 256;      // float4 loads per thread per block
  static_assert(LPT * 256 == kTile * F4R, "whole loads");
  __shared__ __attribute__((aligned(16))) char lds[2][BLK];
  __shared__ __attribute__((aligned(16))) float xch[4][kTile];   // per-wave candidate factors
  const int32_t T = ws_i32(ws, L.off_hdr)[kHdrTiles];
  const int tid = threadIdx.x;
  if (T == 0) {
    // no candidate tiles (offsets broke their contract): zero outputs
    const int64_t n = L.N * D;
    for (int64_t i = (int64_t)blockIdx.x * 256 + tid; i < n; i += (int64_t)gridDim.x * 256) out[i] = 0.f;
    if (lse_out != nullptr)
      for (int64_t i = (int64_t)blockIdx.x * 256 + tid; i < L.N; i += (int64_t)gridDim.x * 256) lse_out[i] = 0.f;
    return;
  }
  // XCD-aware order: workgroup x runs on XCD x % 8; consecutive quads (the
  // workgroups of one user) go to one XCD, so its L2 serves that user's
  // sketch to all of them
  const int nq = T / 4, qx = (nq + 7) / 8;
  const int slot = blockIdx.x >> 3;
  if (slot >= qx) return;
  const int quad = (blockIdx.x & 7) * qx + slot;
  if (quad >= nq) return;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, g = lane >> 5;
  const int tile = 4 * quad + wave;
  const int u = find_user(tile_base, L.R, 4 * quad);
  const int64_t c0 = cand_offsets[u] + (int64_t)(tile - tile_base[u]) * kTile;
  const int64_t rem = cand_offsets[u + 1] - c0;
  const int count = rem < 0 ? 0 : (rem < kTile ? (int)rem : kTile);
  const bool active = __builtin_amdgcn_readfirstlane(count) > 0;   // uniform over the wave

  // the user's sketch: row u of Sk, or row sketch_rows[u] (e.g. a cache
  // slot).  An index outside [0, sketch_count) reads nothing: the user's
  // candidates get zero outputs and the device error flag is raised (the
  // test is uniform over the workgroup: its 4 tiles belong to user u).
  const int64_t srow = sketch_rows != nullptr ? (int64_t)sketch_rows[u] : (int64_t)u;
  if (srow < 0 || srow >= sketch_count) {
    for (int t = 0; t < count; ++t) out[(c0 + t) * D + lane] = 0.f;
    if constexpr (D > 64)
      for (int t = 0; t < count; ++t) out[(c0 + t) * D + 64 + lane] = 0.f;
    if (lse_out != nullptr && lane < count) lse_out[c0 + lane] = 0.f;
    if (tid == 0) atomicOr(ws_i32(ws, L.off_hdr) + kHdrErr, kErrSketchRow);
    return;
  }
  const float* Su = Sk + srow * L.k * D;

  // candidate queries and sketch values outside fp16's finite range (they
  // become fp16 MFMA operands) raise a device error bit at the end
  uint32_t range_bad = 0u;
  half8 qB[S];
  if (col < count) {
    const uint16_t* qrow = Q + (c0 + col) * D;
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const u32x4 raw = *reinterpret_cast<const u32x4*>(qrow + 16 * s + 8 * g);
      range_bad |= bf16x8_range_bits(raw);
      qB[s] = bf16x8_to_f16x8(raw);
    }
  } else {
#pragma unroll
    for (int s = 0; s < S; ++s) qB[s] = half8{};
  }
  const int NB = L.k / kTile;
  // two register sets: the global loads of block i + 2 are issued while
  // block i is computed, and block i + 1 (loaded an iteration earlier) goes
  // to LDS at the end of the iteration
  float4 pfa[LPT], pfb[LPT];
  auto gload = [&](int i, float4 (&pf)[LPT]) {
    const float* src = Su + (int64_t)i * kTile * D;
#pragma unroll
    for (int k2 = 0; k2 < LPT; ++k2) pf[k2] = reinterpret_cast<const float4*>(src)[tid + 256 * k2];
  };
  auto swrite = [&](int buf, const float4 (&pf)[LPT]) {
#pragma unroll
    for (int k2 = 0; k2 < LPT; ++k2) {
      const int idx = tid + 256 * k2, row = idx / F4R, c4 = idx % F4R;
      const float big = fmaxf(fmaxf(fabsf(pf[k2].x), fabsf(pf[k2].y)), fmaxf(fabsf(pf[k2].z), fabsf(pf[k2].w)));
      range_bad |= !(big <= 65504.0f) ? 1u : 0u;   // NaN fails the test too
      const half2v lo = __builtin_bit_cast(half2v, __builtin_amdgcn_cvt_pkrtz(pf[k2].x, pf[k2].y));
      const half2v hi = __builtin_bit_cast(half2v, __builtin_amdgcn_cvt_pkrtz(pf[k2].z, pf[k2].w));
      uint2 w;
      w.x = __builtin_bit_cast(uint32_t, lo);
      w.y = __builtin_bit_cast(uint32_t, hi);
      *reinterpret_cast<uint2*>(lds[buf] + row * PITCH + 8 * c4) = w;
    }
  };
  const int abase = tau(col) * PITCH + 16 * g;
  const int i16 = lane & 15, gh = (lane >> 4) & 1;
  const int tr_base = (4 * (i16 >> 2) + 2 * g) * PITCH + 32 * gh + 8 * (i16 & 3);
  const float sc2 = 1.4426950408889634f / sqrtf((float)D);
  float* wx = xch[wave];
  // the factor of candidate acc_row(r, g) for each output register, from
  // the per-candidate values lane col has put in wx (same wave: LDS
  // operations complete in order)
  auto row_factors = [&](float (&f)[16]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float4 v = *reinterpret_cast<const float4*>(wx + 8 * i + 4 * g);
      f[4 * i] = v.x;
      f[4 * i + 1] = v.y;
      f[4 * i + 2] = v.z;
      f[4 * i + 3] = v.w;
    }
  };

  // One sweep with a running maximum m (base 2) per candidate, shared by
  // both lane halves; l = the lane half's sum of 2^(x - m); O rescaled by
  // 2^(m_old - m_new) whenever m grows.
  float m = -INFINITY, l = 0.f;
  float16v O[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) O[dt] = float16v{};

  auto step = [&](int i, float4 (&pf_next)[LPT], float4 (&pf_free)[LPT]) {
    if (i + 2 < NB) gload(i + 2, pf_free);
    const char* sb = lds[i & 1];
    // a wave whose tile is padding (the user's tile count rounded up to 4)
    // only helps stage the blocks
    if (active) {
      float16v C = float16v{};
#pragma unroll
      for (int s0 = 0; s0 < S; s0 += 4) {
        half8 a[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) a[s] = *reinterpret_cast<const half8*>(sb + abase + 32 * (s0 + s));
#pragma unroll
        for (int s = 0; s < 4; ++s) C = mfma32x32x16(a[s], qB[s0 + s], C);
      }
      float bm = C[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) bm = fmaxf(bm, C[r]);
      bm = fmaxf(bm, __shfl_xor(bm, 32)) * sc2;
      // Lazy rescale: the running maximum m moves (and O, l are rescaled)
      // only when some candidate of the wave sees a logit more than 2^8 above
      // it; otherwise P = 2^(logit - m) <= 2^8 and 2^6 P stays in fp16 range.
      if (__any(bm > m + 8.0f)) {   // uniform over the wave
        const float mn = fmaxf(m, bm);
        const float alpha = __builtin_amdgcn_exp2f(m - mn);   // 0 on the first block
        m = mn;
        l *= alpha;
        if (i > 0) {
          if (g == 0) wx[col] = alpha;
          float f[16];
          row_factors(f);
#pragma unroll
          for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r) O[dt][r] *= f[r];
        }
      }
      half8 ap[2];
      float sum = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(C[r] * sc2 - m);
        sum += p;
        ap[r >> 3][r & 7] = (_Float16)(p * 64.0f);   // 2^6 P <= 2^14: small weights stay normal fp16
      }
      l += sum;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        half8 hb[DT];
        tile_tr_reads_kk<D>(lds_addr(sb) + tr_base + kk * 16 * PITCH, hb);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) O[dt] = mfma32x32x16(ap[kk], hb[dt], O[dt]);
      }
    }
    if (i + 1 < NB) swrite((i + 1) & 1, pf_next);
    __syncthreads();
  };
  gload(0, pfa);
  swrite(0, pfa);
  if (NB > 1) gload(1, pfb);
  __syncthreads();
  for (int i = 0; i < NB; i += 2) {
    step(i, pfb, pfa);
    if (i + 1 < NB) step(i + 1, pfa, pfb);
  }
  l += __shfl_xor(l, 32);
  if (g == 0) wx[col] = 1.0f / (64.0f * l);
  float f[16];
  row_factors(f);
  // output rows are candidates acc_row(r, g), columns 32 dt + col
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int t = acc_row(r, g);
    if (t < count) {
      float* dst = out + (c0 + t) * D + col;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) dst[32 * dt] = O[dt][r] * f[r];
    }
  }
  if (lse_out != nullptr && g == 0 && col < count) lse_out[c0 + col] = (m + __log2f(l)) * 0.69314718055994531f;
  if (__ballot(range_bad != 0u) != 0ull && lane == 0) atomicOr(ws_i32(ws, L.off_hdr) + kHdrErr, kErrRange);
}

hipError_t launch_target_attention(const Layout& L, const void* Q, const int64_t* cand_offsets, const float* S,
                                   const int32_t* sketch_rows, int64_t sketch_count, void* ws, float* out, float* lse,
                                   hipStream_t stream) {
  if (launch_schedule(L, cand_offsets, ws, stream) != hipSuccess) return hipErrorLaunchFailure;
  if (L.N == 0) return hipSuccess;
  // a multiple of 8 workgroups covering every quad of tiles (see ta_attend)
  const int64_t grid = std::max<int64_t>(8, (L.tiles_max / kUserTileAlign + 7) / 8 * 8);
  const int32_t* tb = reinterpret_cast<const int32_t*>(reinterpret_cast<const char*>(ws) + L.off_tile_base);
  if (L.d == 128)
    hipLaunchKernelGGL((ta_attend<128>), dim3((unsigned)grid), dim3(256), 0, stream, (const uint16_t*)Q, cand_offsets,
                       S, sketch_rows, sketch_count, tb, L, ws, out, lse);
  else
    hipLaunchKernelGGL((ta_attend<64>), dim3((unsigned)grid), dim3(256), 0, stream, (const uint16_t*)Q, cand_offsets,
                       S, sketch_rows, sketch_count, tb, L, ws, out, lse);
  return hipGetLastError();
}

}  // namespace sa
