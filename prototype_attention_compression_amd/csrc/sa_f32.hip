// sa_f32.hip — Sketch Attention for float32 inputs (fp32 arithmetic on the
// vector ALUs), the same two passes as the bf16 path:
//   pass 1: lse_t = log2 sum_j 2^(q_j . h_t) per token, exact two-sweep form
//           (maximum, then the shifted sum);
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

// One thread per token slot (tile * 32 + row).
template <int D>
__global__ __launch_bounds__(256) void pass1_f32(const float* __restrict__ H, const int64_t* __restrict__ offsets,
                                                 const uint8_t* __restrict__ mask, Layout L, void* ws) {
  const int32_t* hdr = ws_i32(ws, L.off_hdr);
  const int64_t slot = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int32_t tile = (int32_t)(slot / kTile);
  const int row = (int)(slot % kTile);
  if (tile >= hdr[kHdrTiles]) return;
  const TileInfo ti = tile_info(ws_i32(ws, L.off_tile_base), offsets, L.R, tile);
  float* lse = ws_f32(ws, L.off_lse32);
  bool valid = row < ti.count;
  const int64_t tok = ti.tok0 + row;
  if (valid && mask != nullptr) valid = mask[tok] != 0;
  if (!valid) {
    lse[slot] = INFINITY;
    return;
  }
  float h[D];
#pragma unroll
  for (int a = 0; a < D; ++a) h[a] = H[tok * D + a];
  const float* q = ws_f32(ws, L.off_q32);
  float mx = -INFINITY;
  for (int j = 0; j < L.k; ++j) {
    float s = 0.f;
#pragma unroll
    for (int a = 0; a < D; ++a) s = fmaf(q[(int64_t)j * D + a], h[a], s);
    mx = fmaxf(mx, s);
  }
  float sum = 0.f;
  for (int j = 0; j < L.k; ++j) {
    float s = 0.f;
#pragma unroll
    for (int a = 0; a < D; ++a) s = fmaf(q[(int64_t)j * D + a], h[a], s);
    sum += exp2f(s - mx);
  }
  lse[slot] = mx + log2f(sum);
}

// Workgroup = (chunk, block of 64 prototypes), 256 threads.  Per tile: thread
// (j = tid % 64, grp = tid / 64) computes the allocations of prototype j for
// tokens 8*grp .. 8*grp+7, then accumulates U[j, grp*D/4 .. +D/4).
template <int D>
__global__ __launch_bounds__(256) void pass2_f32(const float* __restrict__ H, const int64_t* __restrict__ offsets,
                                                 const uint8_t* __restrict__ mask, Layout L, void* ws) {
  constexpr int DQ = D / 4;
  __shared__ float hs[kTile][D + 1];
  __shared__ float as[64][kTile + 1];
  __shared__ float ls[kTile];
  const int32_t* hdr = ws_i32(ws, L.off_hdr);
  const int nblk = L.k / 64;
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
  const int tid = threadIdx.x, j = tid & 63, grp = tid >> 6;
  const int p = pb * 64 + j;
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
  for (int it = 0; it < nt; ++it) {
    const int32_t tile = t0 + it;
    const int64_t tok0 = u_lo + (int64_t)(ci * CT + it) * kTile;
    for (int e = tid; e < kTile * D; e += 256) {
      const int r = e / D, a = e % D;
      const int64_t tok = tok0 + r;
      bool ok = tok < u_hi;
      if (ok && mask != nullptr) ok = mask[tok] != 0;
      hs[r][a] = ok ? H[tok * D + a] : 0.f;
    }
    if (tid < kTile) ls[tid] = lse[(int64_t)tile * kTile + tid];
    __syncthreads();
#pragma unroll
    for (int r8 = 0; r8 < 8; ++r8) {
      const int r = grp * 8 + r8;
      float s = 0.f;
#pragma unroll
      for (int a = 0; a < D; ++a) s = fmaf(qv[a], hs[r][a], s);
      as[j][r] = exp2f(s - ls[r]);
    }
    __syncthreads();
    for (int r = 0; r < kTile; ++r) {
      const float a = as[j][r];
      m += a;
#pragma unroll
      for (int c = 0; c < DQ; ++c) U[c] = fmaf(a, hs[r][grp * DQ + c], U[c]);
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
  const int64_t g1 = ((int64_t)L.tiles_max * kTile + 255) / 256;
  if (g1 == 0) return hipSuccess;
  if (L.d == 128)
    hipLaunchKernelGGL(pass1_f32<128>, dim3((unsigned)g1), dim3(256), 0, stream, (const float*)H, offsets, mask, L, ws);
  else
    hipLaunchKernelGGL(pass1_f32<64>, dim3((unsigned)g1), dim3(256), 0, stream, (const float*)H, offsets, mask, L, ws);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t g2 = (int64_t)L.chunks_max * (L.k / 64);
  if (g2 == 0) return hipSuccess;
  if (L.d == 128)
    hipLaunchKernelGGL(pass2_f32<128>, dim3((unsigned)g2), dim3(256), 0, stream, (const float*)H, offsets, mask, L, ws);
  else
    hipLaunchKernelGGL(pass2_f32<64>, dim3((unsigned)g2), dim3(256), 0, stream, (const float*)H, offsets, mask, L, ws);
  return hipGetLastError();
}

}  // namespace sa
