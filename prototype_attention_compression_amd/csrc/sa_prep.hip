// sa_prep.hip — per-launch preparation for Sketch Attention:
//   * prototype queries Q = P Wk^T * (log2(e) / sqrt(d)) (the logit
//     L[j,t] = p_j . (h_t Wk) / sqrt(d) equals q_j . h_t after this
//     reassociation; the log2(e) factor lets the kernels use exp2);
//   * the ragged schedule: per-user tile and chunk prefix sums read from the
//     device `offsets`, plus the offsets contract check.
// The logit definition follows the SequenceO1 arXiv abstract (learnable
// prototypes) with keys projected from the history and a 1/sqrt(d) scale.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "sa_device.h"
#include "sa_launch.h"

namespace sa {

template <typename T>
__device__ __forceinline__ float load_in(const T* p, int64_t i);
template <>
__device__ __forceinline__ float load_in<uint16_t>(const uint16_t* p, int64_t i) {
  return __uint_as_float(((uint32_t)p[i]) << 16);
}
template <>
__device__ __forceinline__ float load_in<float>(const float* p, int64_t i) {
  return p[i];
}

// One workgroup of 256 threads computes 256 / D query rows.  Thread (j, c)
// forms q[j][c] = sum_a P[j][a] * Wk[c][a], scaled.  The bf16 path stores the
// rows in fp16 (the MFMA operand type) with their norms; the fp32 path stores
// fp32 rows.
template <int D, typename T>
__global__ __launch_bounds__(256) void prep_queries(const T* __restrict__ P, const T* __restrict__ Wk,
                                                    Layout L, void* ws) {
  constexpr int PR = 256 / D;
  // Wk staged in LDS with all of its 16-byte loads in flight together (a
  // row-per-thread walk through global memory waited on each load); the
  // padded pitch keeps the row-per-thread LDS reads on distinct banks
  constexpr int EPC = 16 / (int)sizeof(T);                 // elements per 16-byte chunk
  constexpr int WCH = D * D / EPC / 256;                   // chunks per thread
  constexpr int WP = D + (sizeof(T) == 2 ? 2 : 1);
  static_assert(WCH * 256 * EPC == D * D, "whole chunks");
  __shared__ float prow[PR][D];
  __shared__ float red[256];
  __shared__ T wk[D * WP];
  const int tid = threadIdx.x;
  {
    u32x4 w[WCH];
#pragma unroll
    for (int i = 0; i < WCH; ++i) w[i] = reinterpret_cast<const u32x4*>(Wk)[tid + 256 * i];
#pragma unroll
    for (int i = 0; i < WCH; ++i) {
      const int q = tid + 256 * i, row = q / (D / EPC), e0 = EPC * (q % (D / EPC));
      const T* v = reinterpret_cast<const T*>(&w[i]);
#pragma unroll
      for (int e = 0; e < EPC; ++e) wk[row * WP + e0 + e] = v[e];
    }
  }
  const int jl = tid / D, c = tid % D;
  const int j = blockIdx.x * PR + jl;
  prow[jl][c] = load_in<T>(P, (int64_t)j * D + c);
  __syncthreads();
  float acc = 0.f;
#pragma unroll 8
  for (int a = 0; a < D; ++a) acc = fmaf(prow[jl][a], load_in<T>(wk, c * WP + a), acc);
  const float scale = 1.4426950408889634f / sqrtf((float)D);
  const float q = acc * scale;
  if (L.dtype == 1) {
    ws_f32(ws, L.off_q32)[(int64_t)j * D + c] = q;
    return;
  }
  _Float16* q16 = ws_f16(ws, L.off_q16) + (int64_t)j * D;
  const _Float16 qh = (_Float16)q;
  q16[c] = qh;
  const float qf = (float)qh;
  red[tid] = qf * qf;
  __syncthreads();
  if (c == 0) {
    float s = 0.f;
    for (int a = 0; a < D; ++a) s += red[jl * D + a];
    ws_f32(ws, L.off_qnorm)[j] = sqrtf(s);
  }
}

// Single workgroup.  Checks 0 = offsets[0] <= ... <= offsets[R] = N; on a
// violation every user is treated as empty and the error flag is raised.
// Writes tile_base / chunk_base (exclusive prefix sums of tiles_u = ceil(n_u /
// 32) rounded up to a multiple of kUserTileAlign, and ceil(tiles_u /
// tiles_per_chunk)), the totals, and the largest query norm.
__global__ __launch_bounds__(1024) void prep_schedule(const int64_t* __restrict__ offsets, Layout L,
                                                      void* ws) {
  __shared__ int32_t sc_t[1024];
  __shared__ int32_t sc_c[1024];
  __shared__ float sq[1024];
  const int tid = threadIdx.x;
  const int R = L.R;
  int bad = 0;
  for (int u = tid; u < R; u += 1024)
    if (offsets[u + 1] < offsets[u]) bad = 1;
  if (tid == 0 && (offsets[0] != 0 || offsets[R] != L.N)) bad = 1;
  bad = __syncthreads_or(bad);

  const int seg = (R + 1023) / 1024;
  const int u0 = min(R, tid * seg), u1 = min(R, u0 + seg);
  const int CT = L.tiles_per_chunk;
  int32_t nt = 0, nc = 0;
  for (int u = u0; u < u1; ++u) {
    int64_t n = bad ? 0 : offsets[u + 1] - offsets[u];
    int32_t t = (int32_t)((n + kTile * kUserTileAlign - 1) / (kTile * kUserTileAlign)) * kUserTileAlign;
    nt += t;
    nc += (t + CT - 1) / CT;
  }
  sc_t[tid] = nt;
  sc_c[tid] = nc;
  __syncthreads();
  // inclusive Hillis-Steele scan over the 1024 per-thread totals
  for (int off = 1; off < 1024; off <<= 1) {
    int32_t a = tid >= off ? sc_t[tid - off] : 0;
    int32_t b = tid >= off ? sc_c[tid - off] : 0;
    __syncthreads();
    sc_t[tid] += a;
    sc_c[tid] += b;
    __syncthreads();
  }
  int32_t bt = sc_t[tid] - nt, bc = sc_c[tid] - nc;
  int32_t* tile_base = ws_i32(ws, L.off_tile_base);
  int32_t* chunk_base = ws_i32(ws, L.off_chunk_base);
  for (int u = u0; u < u1; ++u) {
    tile_base[u] = bt;
    chunk_base[u] = bc;
    int64_t n = bad ? 0 : offsets[u + 1] - offsets[u];
    int32_t t = (int32_t)((n + kTile * kUserTileAlign - 1) / (kTile * kUserTileAlign)) * kUserTileAlign;
    bt += t;
    bc += (t + CT - 1) / CT;
  }
  int32_t* hdr = ws_i32(ws, L.off_hdr);
  if (tid == 1023) {
    tile_base[R] = sc_t[1023];
    chunk_base[R] = sc_c[1023];
    hdr[kHdrErr] = bad ? kErrBadOffsets : 0;
    hdr[kHdrTiles] = sc_t[1023];
    hdr[kHdrChunks] = sc_c[1023];
    hdr[kHdrHmax] = 0;
  }
  if (L.dtype == 0) {
    float m = 0.f;
    const float* qn = ws_f32(ws, L.off_qnorm);
    for (int j = tid; j < L.k; j += 1024) m = fmaxf(m, qn[j]);
    sq[tid] = m;
    __syncthreads();
    for (int off = 512; off > 0; off >>= 1) {
      if (tid < off) sq[tid] = fmaxf(sq[tid], sq[tid + off]);
      __syncthreads();
    }
    if (tid == 0) hdr[kHdrQmax] = __float_as_int(sq[0]);
  } else if (tid == 0) {
    hdr[kHdrQmax] = 0;
  }
}

// Zero fill of the one-pass exchange ring (its tags must not match a tile of
// this call).  A kernel rather than a memset so that the sequence can be
// captured in a graph.
__global__ __launch_bounds__(256) void clear_words(uint64_t* __restrict__ p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = 0ull;
}

// dst[0] = the workspace's device error word (a kernel rather than a copy,
// so that the sequence can be captured in a graph)
__global__ __launch_bounds__(64) void copy_error_word(const int32_t* __restrict__ hdr, int32_t* __restrict__ dst) {
  if (threadIdx.x == 0) dst[0] = hdr[kHdrErr];
}

hipError_t launch_copy_error(const Layout& L, const void* ws, int32_t* dst, hipStream_t stream) {
  const int32_t* hdr = reinterpret_cast<const int32_t*>(static_cast<const char*>(ws) + L.off_hdr);
  hipLaunchKernelGGL(copy_error_word, dim3(1), dim3(64), 0, stream, hdr, dst);
  return hipGetLastError();
}

hipError_t launch_schedule(const Layout& L, const int64_t* offsets, void* ws, hipStream_t stream) {
  hipLaunchKernelGGL(prep_schedule, dim3(1), dim3(1024), 0, stream, offsets, L, ws);
  return hipGetLastError();
}

hipError_t launch_prep(const Layout& L, const void* P, const void* Wk, const int64_t* offsets, void* ws,
                       hipStream_t stream) {
  const int PR = 256 / L.d;
  dim3 gq(L.k / PR), bq(256);
  if (L.dtype == 0) {
    if (L.d == 128)
      hipLaunchKernelGGL((prep_queries<128, uint16_t>), gq, bq, 0, stream, (const uint16_t*)P,
                         (const uint16_t*)Wk, L, ws);
    else
      hipLaunchKernelGGL((prep_queries<64, uint16_t>), gq, bq, 0, stream, (const uint16_t*)P,
                         (const uint16_t*)Wk, L, ws);
  } else {
    if (L.d == 128)
      hipLaunchKernelGGL((prep_queries<128, float>), gq, bq, 0, stream, (const float*)P, (const float*)Wk, L, ws);
    else
      hipLaunchKernelGGL((prep_queries<64, float>), gq, bq, 0, stream, (const float*)P, (const float*)Wk, L, ws);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(prep_schedule, dim3(1), dim3(1024), 0, stream, offsets, L, ws);
  e = hipGetLastError();
  if (e != hipSuccess || !L.fused) return e;
  const int64_t words = (int64_t)L.groups * kXSlots * kTile * (L.k / kFusedProtos);
  hipLaunchKernelGGL(clear_words, dim3(64), dim3(256), 0, stream,
                     reinterpret_cast<uint64_t*>(reinterpret_cast<char*>(ws) + L.off_xbuf), words);
  return hipGetLastError();
}

}  // namespace sa
