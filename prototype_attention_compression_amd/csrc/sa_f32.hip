// sa_f32.hip — Sketch Attention for float32 inputs (fp32 arithmetic on the
// vector ALUs), the same two passes as the bf16 path:
//   pass 1: lse_t = log2 sum_j 2^(q_j . h_t) per token, in one sweep with a
//           running maximum (the sum rescaled whenever the maximum grows);
//   pass 2: per (chunk, 64-prototype block) A[j,t] = 2^(q_j . h_t - lse_t),
//           U[j,:] += A[j,t] h_t and m_j += A[j,t].
// The softmax runs over prototypes for each token (SequenceO1 blog "How it
// works" item 1; review FAQ on how SA differs from standard attention).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "sa_device.h"
#include "sa_launch.h"

namespace sa {

// Pass 1: eight threads per token slot (tile * 32 + row), 32 slots (one
// tile) per workgroup.  Thread (slot sl = tid / 8, part = tid % 8) takes the
// prototypes j = 8 i + part.  The queries pass through LDS 64 rows at a time,
// each row padded by 16 bytes so that the eight rows a wave reads at once sit
// in different banks (the 16 lanes of a part read the same address: a
// broadcast).  Each thread keeps a running maximum m and the sum of 2^(x - m)
// over its prototypes (one sweep: the sum is rescaled when the maximum
// grows); the eight partial pairs of a token are combined by lane shuffles.
// Every thread takes part in the staging barriers; slots past the batch's
// last tile compute on zeros and write nothing.
template <int D>
__global__ __launch_bounds__(256) void pass1_f32(const float* __restrict__ H, const int64_t* __restrict__ offsets,
                                                 const uint8_t* __restrict__ mask, Layout L, void* ws) {
  constexpr int QP = D + 4;   // padded query row (floats)
  __shared__ __attribute__((aligned(16))) float qs[64 * QP];
  const int32_t* hdr = ws_i32(ws, L.off_hdr);
  constexpr int TPT = 8;   // threads per token
  const int tid = threadIdx.x, part = tid % TPT;
  const int64_t slot = (int64_t)blockIdx.x * (256 / TPT) + tid / TPT;
  const int32_t T = hdr[kHdrTiles];
  const int32_t tile = (int32_t)(slot / kTile);
  const int row = (int)(slot % kTile);
  bool valid = false;
  int64_t tok = 0;
  if (tile < T) {
    const TileInfo ti = tile_info(ws_i32(ws, L.off_tile_base), offsets, L.R, tile);
    valid = row < ti.count;
    tok = ti.tok0 + row;
    if (valid && mask != nullptr) valid = mask[tok] != 0;
  }
  float h[D];
  if (valid) {   // one branch around the row's loads
#pragma unroll
    for (int a = 0; a < D; a += 4) {
      const float4 v = *reinterpret_cast<const float4*>(H + tok * D + a);
      h[a] = v.x;
      h[a + 1] = v.y;
      h[a + 2] = v.z;
      h[a + 3] = v.w;
    }
  } else {
#pragma unroll
    for (int a = 0; a < D; ++a) h[a] = 0.f;
  }
  const float* q = ws_f32(ws, L.off_q32);
  float m = -INFINITY, sum = 0.f;
  auto update = [&](float x) {
    const float mn = fmaxf(m, x);
    sum = sum * exp2f(m - mn) + exp2f(x - mn);
    m = mn;
  };
  constexpr int SL = 64 * (D / 4) / 256;   // 16-byte staging loads per thread and chunk
  for (int j0 = 0; j0 < L.k; j0 += 64) {
    // the chunk's loads issued together, then written (a vector type: an
    // array of the float4 struct would stay in scratch memory)
    u32x4 st[SL];
#pragma unroll
    for (int k2 = 0; k2 < SL; ++k2) {
      const int e = tid + 256 * k2, r = e / (D / 4), c = e % (D / 4);
      st[k2] = *reinterpret_cast<const u32x4*>(q + (int64_t)(j0 + r) * D + 4 * c);
    }
    __syncthreads();   // every read of the previous chunk is done
#pragma unroll
    for (int k2 = 0; k2 < SL; ++k2) {
      const int e = tid + 256 * k2, r = e / (D / 4), c = e % (D / 4);
      *reinterpret_cast<u32x4*>(qs + r * QP + 4 * c) = st[k2];
    }
    __syncthreads();
    // two prototypes at a time, each dot product in two partial sums (four
    // independent FMA chains)
    for (int i = 0; i < 64 / TPT; i += 2) {
      const float* q0 = qs + (TPT * i + part) * QP;
      const float* q1 = q0 + TPT * QP;
      float x0a = 0.f, x0b = 0.f, x1a = 0.f, x1b = 0.f;
#pragma unroll
      for (int a = 0; a < D; a += 8) {
        const float4 u0 = *reinterpret_cast<const float4*>(q0 + a), v0 = *reinterpret_cast<const float4*>(q0 + a + 4);
        const float4 u1 = *reinterpret_cast<const float4*>(q1 + a), v1 = *reinterpret_cast<const float4*>(q1 + a + 4);
        x0a = fmaf(u0.x, h[a], x0a);
        x0b = fmaf(v0.x, h[a + 4], x0b);
        x1a = fmaf(u1.x, h[a], x1a);
        x1b = fmaf(v1.x, h[a + 4], x1b);
        x0a = fmaf(u0.y, h[a + 1], x0a);
        x0b = fmaf(v0.y, h[a + 5], x0b);
        x1a = fmaf(u1.y, h[a + 1], x1a);
        x1b = fmaf(v1.y, h[a + 5], x1b);
        x0a = fmaf(u0.z, h[a + 2], x0a);
        x0b = fmaf(v0.z, h[a + 6], x0b);
        x1a = fmaf(u1.z, h[a + 2], x1a);
        x1b = fmaf(v1.z, h[a + 6], x1b);
        x0a = fmaf(u0.w, h[a + 3], x0a);
        x0b = fmaf(v0.w, h[a + 7], x0b);
        x1a = fmaf(u1.w, h[a + 3], x1a);
        x1b = fmaf(v1.w, h[a + 7], x1b);
      }
      update(x0a + x0b);
      update(x1a + x1b);
    }
  }
  // the parts of a token are lanes TPT sl .. TPT sl + TPT - 1 of one wave
#pragma unroll
  for (int off = 1; off < TPT; off <<= 1) {
    const float mo = __shfl_xor(m, off), so = __shfl_xor(sum, off);
    const float mn = fmaxf(m, mo);
    sum = sum * exp2f(m - mn) + so * exp2f(mo - mn);
    m = mn;
  }
  if (part == 0 && tile < T) ws_f32(ws, L.off_lse32)[slot] = valid ? m + log2f(sum) : INFINITY;
}

// Workgroup = (chunk, block of 16 prototypes), 256 threads.  Per tile: thread
// (j = tid % 16, grp = tid / 16) computes the allocations of prototype j for
// tokens 2*grp and 2*grp+1, then accumulates U[j, grp*D/16 .. +D/16).  Small
// blocks give small batches (one user of a few thousand tokens) enough
// workgroups: the per-thread chains are short, and latency, not arithmetic,
// sets their time.
template <int D>
__global__ __launch_bounds__(256) void pass2_f32(const float* __restrict__ H, const int64_t* __restrict__ offsets,
                                                 const uint8_t* __restrict__ mask, Layout L, void* ws) {
  constexpr int PB = 16, NG = 256 / PB, TPG = kTile / NG;   // prototypes, groups, tokens per group
  constexpr int DQ = D / NG;
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  __shared__ __attribute__((aligned(16))) float hs[kTile][D + 4];   // rows 16-byte aligned: vector reads
  __shared__ float as[PB][kTile + 1];
  __shared__ float ls[kTile];
  const int32_t* hdr = ws_i32(ws, L.off_hdr);
  const int nblk = L.k / PB;
  const int chunk = blockIdx.x / nblk, pb = blockIdx.x % nblk;
  if (chunk >= hdr[kHdrChunks]) return;
  const int32_t* tile_base = ws_i32(ws, L.off_tile_base);
  const int32_t* chunk_base = ws_i32(ws, L.off_chunk_base);
  const int u = find_user(chunk_base, L.R, chunk);
  const int ci = chunk - chunk_base[u];
  const int CT = L.tiles_per_chunk;
  const int tiles_u = tile_base[u + 1] - tile_base[u];
  const int32_t t0 = tile_base[u] + ci * CT;
  const int nt = min(CT, tiles_u - ci * CT);
  const int tid = threadIdx.x, j = tid % PB, grp = tid / PB;
  const int p = pb * PB + j;
  const float* q32 = ws_f32(ws, L.off_q32);
  const float* lse = ws_f32(ws, L.off_lse32);
  float qv[D];
#pragma unroll
  for (int a = 0; a < D; ++a) qv[a] = q32[(int64_t)p * D + a];
  float U[DQ];
#pragma unroll
  for (int c = 0; c < DQ; ++c) U[c] = 0.f;
  float m = 0.f;
  const int64_t u_lo = offsets[u], u_hi = offsets[u + 1];
  // A tile's rows as 16-byte pieces, NV per thread, loaded together from
  // addresses clamped to the user's rows (a user with tiles has a token) and
  // zeroed past its end or where masked; the next tile's loads are issued
  // before the current tile's arithmetic.
  constexpr int NV = kTile * D / 4 / 256;
  static_assert(NV * 256 * 4 == kTile * D, "whole pieces");
  u32x4 rv[NV];
  uint8_t mk[NV];      // the mask bytes of the pieces' tokens (1 without a mask)
  uint32_t inb = 0;    // bit k2: piece k2's token lies inside the user's rows
  float lv = 0.f;
  auto load_tile = [&](int it) {
    const int64_t tok0 = u_lo + (int64_t)(ci * CT + it) * kTile;
    inb = 0;
#pragma unroll
    for (int k2 = 0; k2 < NV; ++k2) {
      const int e = tid + 256 * k2, r = e / (D / 4), c4 = e % (D / 4);
      const int64_t tok = tok0 + r, tc = tok < u_hi ? tok : u_hi - 1;
      rv[k2] = *reinterpret_cast<const u32x4*>(H + tc * D + 4 * c4);
      mk[k2] = mask != nullptr ? mask[tc] : (uint8_t)1;
      inb |= (tok < u_hi ? 1u : 0u) << k2;
    }
    if (tid < kTile) lv = lse[(int64_t)(t0 + it) * kTile + tid];
  };
  if (nt > 0) load_tile(0);
  for (int it = 0; it < nt; ++it) {
#pragma unroll
    for (int k2 = 0; k2 < NV; ++k2) {
      const int e = tid + 256 * k2, r = e / (D / 4), c4 = e % (D / 4);
      const bool ok = ((inb >> k2) & 1u) != 0 && mk[k2] != 0;
      *reinterpret_cast<u32x4*>(&hs[r][4 * c4]) = ok ? rv[k2] : u32x4{0u, 0u, 0u, 0u};
    }
    if (tid < kTile) ls[tid] = lv;
    __syncthreads();
    if (it + 1 < nt) load_tile(it + 1);
    // the logits of prototype j for tokens TPG grp ..: TPG chains of two
    // partial sums each, rows read 16 bytes at a time (a wave's four groups
    // read four rows, in distinct banks)
    float sx[TPG][2];
#pragma unroll
    for (int r = 0; r < TPG; ++r) sx[r][0] = sx[r][1] = 0.f;
#pragma unroll
    for (int a = 0; a < D; a += 8) {
#pragma unroll
      for (int r = 0; r < TPG; ++r) {
        const f32x4 h4 = *reinterpret_cast<const f32x4*>(&hs[grp * TPG + r][a]);
        const f32x4 g4 = *reinterpret_cast<const f32x4*>(&hs[grp * TPG + r][a + 4]);
        sx[r][0] = fmaf(qv[a], h4.x, sx[r][0]);
        sx[r][1] = fmaf(qv[a + 4], g4.x, sx[r][1]);
        sx[r][0] = fmaf(qv[a + 1], h4.y, sx[r][0]);
        sx[r][1] = fmaf(qv[a + 5], g4.y, sx[r][1]);
        sx[r][0] = fmaf(qv[a + 2], h4.z, sx[r][0]);
        sx[r][1] = fmaf(qv[a + 6], g4.z, sx[r][1]);
        sx[r][0] = fmaf(qv[a + 3], h4.w, sx[r][0]);
        sx[r][1] = fmaf(qv[a + 7], g4.w, sx[r][1]);
      }
    }
#pragma unroll
    for (int r = 0; r < TPG; ++r)
      as[j][grp * TPG + r] = exp2f(sx[r][0] + sx[r][1] - ls[grp * TPG + r]);
    __syncthreads();
    for (int r = 0; r < kTile; ++r) {
      const float a = as[j][r];
      m += a;
#pragma unroll
      for (int c = 0; c < DQ; c += 4) {
        const f32x4 h4 = *reinterpret_cast<const f32x4*>(&hs[r][grp * DQ + c]);
        U[c] = fmaf(a, h4.x, U[c]);
        U[c + 1] = fmaf(a, h4.y, U[c + 1]);
        U[c + 2] = fmaf(a, h4.z, U[c + 2]);
        U[c + 3] = fmaf(a, h4.w, U[c + 3]);
      }
    }
    __syncthreads();
  }
  float* part_u = ws_f32(ws, L.off_part_u) + ((int64_t)chunk * L.k + p) * D;
#pragma unroll
  for (int c = 0; c < DQ; ++c) part_u[grp * DQ + c] = U[c];
  if (grp == 0) ws_f32(ws, L.off_part_m)[(int64_t)chunk * L.k + p] = m;
}

hipError_t launch_f32(const Layout& L, const void* H, const int64_t* offsets, const uint8_t* mask, void* ws,
                      hipStream_t stream) {
  const int64_t g1 = ((int64_t)L.tiles_max * kTile + 31) / 32;
  if (g1 == 0) return hipSuccess;
  if (L.d == 128)
    hipLaunchKernelGGL(pass1_f32<128>, dim3((unsigned)g1), dim3(256), 0, stream, (const float*)H, offsets, mask, L, ws);
  else
    hipLaunchKernelGGL(pass1_f32<64>, dim3((unsigned)g1), dim3(256), 0, stream, (const float*)H, offsets, mask, L, ws);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t g2 = (int64_t)L.chunks_max * (L.k / 16);
  if (g2 == 0) return hipSuccess;
  if (L.d == 128)
    hipLaunchKernelGGL(pass2_f32<128>, dim3((unsigned)g2), dim3(256), 0, stream, (const float*)H, offsets, mask, L, ws);
  else
    hipLaunchKernelGGL(pass2_f32<64>, dim3((unsigned)g2), dim3(256), 0, stream, (const float*)H, offsets, mask, L, ws);
  return hipGetLastError();
}

}  // namespace sa
