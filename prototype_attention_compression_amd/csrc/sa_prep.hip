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

#include <type_traits>

#include "sa_device.h"
#include "sa_launch.h"

namespace sa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// Queries from bf16 inputs on bf16 MFMAs: P and Wk are exact in bf16, so the
// products are exact in fp32 and the sums are fp32, the same arithmetic as an
// fp32 dot product in another order.  The workgroup (4 waves) computes rows
// r0 .. r0 + 32 RB - 1; wave w the 32 x 32 output block (row block w / CB,
// column block w % CB).  Operands come straight from global memory: lane
// (col, g) reads 8 consecutive elements of row col of P and of Wk (the
// A operand's row m = col, the B operand's column n = col, K elements 8 g ..
// 8 g + 7 of the step).  The rows go to fp16 (the MFMA operand type of the
// passes); qpart receives each 32-row block's largest row norm of the fp16
// values, which bounds every logit of a token by |h_t| times its maximum.
template <int D>
__device__ __forceinline__ void queries_bf16(const uint16_t* __restrict__ P, const uint16_t* __restrict__ Wk,
                                             const Layout& L, void* ws, int blk) {
  constexpr int CB = D / 32;      // 32-column blocks
  constexpr int RB = 4 / CB;      // 32-row blocks per workgroup
  constexpr int ROWS = 32 * RB;
  constexpr int TPR = 256 / ROWS; // threads per row in the norm sums
  __shared__ float sq[ROWS][D + 1];
  __shared__ float rn[ROWS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, g = lane >> 5;
  const int rb = wave / CB, cb = wave % CB;
  const int r0 = blk * ROWS + 32 * rb, c0 = 32 * cb;
  const bf16x8* pa = reinterpret_cast<const bf16x8*>(P + (int64_t)(r0 + col) * D + 8 * g);
  const bf16x8* wb = reinterpret_cast<const bf16x8*>(Wk + (int64_t)(c0 + col) * D + 8 * g);
  bf16x8 a[D / 16], b[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    a[s] = pa[2 * s];
    b[s] = wb[2 * s];
  }
  float16v acc = float16v{};
#pragma unroll
  for (int s = 0; s < D / 16; ++s) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[s], b[s], acc, 0, 0, 0);
  const float scale = 1.4426950408889634f / sqrtf((float)D);
  _Float16* q16 = ws_f16(ws, L.off_q16);
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int m = acc_row(r, g);
    const _Float16 qh = (_Float16)(acc[r] * scale);
    q16[(int64_t)(r0 + m) * D + c0 + col] = qh;
    const float qf = (float)qh;
    sq[32 * rb + m][c0 + col] = qf * qf;
  }
  __syncthreads();
  {
    const int row = tid / TPR, part = tid % TPR;
    float s = 0.f;
    for (int c = part; c < D; c += TPR) s += sq[row][c];
#pragma unroll
    for (int o = 1; o < TPR; o <<= 1) s += __shfl_xor(s, o);
    if (part == 0) rn[row] = s;
  }
  __syncthreads();
  if (tid < RB) {
    float m = 0.f;
    for (int r = 0; r < 32; ++r) m = fmaxf(m, rn[32 * tid + r]);
    ws_f32(ws, L.off_qpart)[blk * RB + tid] = sqrtf(m);
  }
}

// Queries from fp32 inputs: one workgroup of 256 threads computes 256 / D
// rows; thread (j, c) forms q[j][c] = sum_a P[j][a] Wk[c][a], scaled, in
// fp32 (the fp32 path's passes bound nothing by the query norms).
template <int D>
__device__ __forceinline__ void queries_f32(const float* __restrict__ P, const float* __restrict__ Wk,
                                            const Layout& L, void* ws, int blk) {
  constexpr int PR = 256 / D;
  // Wk staged in LDS with all of its 16-byte loads in flight together (a
  // row-per-thread walk through global memory waited on each load); the
  // padded pitch keeps the row-per-thread LDS reads on distinct banks
  constexpr int WCH = D * D / 4 / 256;                     // 16-byte chunks per thread
  constexpr int WP = D + 1;
  static_assert(WCH * 256 * 4 == D * D, "whole chunks");
  __shared__ float prow[PR][D];
  __shared__ float wk[D * WP];
  const int tid = threadIdx.x;
  {
    u32x4 w[WCH];
#pragma unroll
    for (int i = 0; i < WCH; ++i) w[i] = reinterpret_cast<const u32x4*>(Wk)[tid + 256 * i];
#pragma unroll
    for (int i = 0; i < WCH; ++i) {
      const int q = tid + 256 * i, row = q / (D / 4), e0 = 4 * (q % (D / 4));
#pragma unroll
      for (int e = 0; e < 4; ++e) wk[row * WP + e0 + e] = __uint_as_float(w[i][e]);
    }
  }
  const int jl = tid / D, c = tid % D;
  const int j = blk * PR + jl;
  prow[jl][c] = P[(int64_t)j * D + c];
  __syncthreads();
  float acc = 0.f;
#pragma unroll 8
  for (int a = 0; a < D; ++a) acc = fmaf(prow[jl][a], wk[c * WP + a], acc);
  ws_f32(ws, L.off_q32)[(int64_t)j * D + c] = acc * (1.4426950408889634f / sqrtf((float)D));
}

// The ragged schedule (one workgroup of 256 threads).  Checks 0 = offsets[0]
// <= ... <= offsets[R] = N; on a violation every user is treated as empty and
// the error flag is raised.  Writes tile_base / chunk_base (exclusive prefix
// sums of tiles_u = ceil(n_u / 32) rounded up to a multiple of
// kUserTileAlign, and of ceil(tiles_u / tiles_per_chunk)) and the totals.
// Users go 2048 at a time, 8 consecutive ones per thread (their offsets are
// loaded together): per-thread sums, a scan within each wave (lane shuffles),
// the four wave totals through LDS, and a running carry.
__device__ __forceinline__ void schedule(const int64_t* __restrict__ offsets, const Layout& L, void* ws) {
  constexpr int UPT = 8;             // users per thread
  constexpr int CHUNK = 256 * UPT;   // users per pass
  __shared__ int32_t wt[2][4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int R = L.R;
  const int CT = L.tiles_per_chunk;
  int32_t* tile_base = ws_i32(ws, L.off_tile_base);
  // the zero row that pass 1 reads for tile slots holding no token
  if (L.dtype == 0 && tid < 64) ws_i32(ws, L.off_zrow)[tid] = 0;
  int32_t* chunk_base = ws_i32(ws, L.off_chunk_base);
  int bad = 0;
  int32_t carry_t = 0, carry_c = 0;
  for (int u0 = 0; u0 < R; u0 += CHUNK) {
    const int ub = u0 + UPT * tid;   // this thread's users ub .. ub + UPT - 1
    int64_t o[UPT + 1];
#pragma unroll
    for (int i = 0; i <= UPT; ++i) o[i] = ub + i <= R ? offsets[ub + i] : 0;
    int32_t t[UPT], c[UPT];
    int32_t st = 0, sc = 0;
#pragma unroll
    for (int i = 0; i < UPT; ++i) {
      t[i] = 0;
      if (ub + i < R) {
        const int64_t n = o[i + 1] - o[i];
        if (n < 0) bad = 1;
        else t[i] = (int32_t)((n + kTile * kUserTileAlign - 1) / (kTile * kUserTileAlign)) * kUserTileAlign;
      }
      c[i] = (t[i] + CT - 1) / CT;
      st += t[i];
      sc += c[i];
    }
    const int32_t own_t = st, own_c = sc;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {   // inclusive scans over the wave
      const int32_t xt = __shfl_up(st, off), xc = __shfl_up(sc, off);
      if (lane >= off) {
        st += xt;
        sc += xc;
      }
    }
    if (lane == 63) {
      wt[0][wave] = st;
      wt[1][wave] = sc;
    }
    __syncthreads();
    int32_t bt = carry_t + st - own_t, bc = carry_c + sc - own_c;
    for (int w = 0; w < wave; ++w) {
      bt += wt[0][w];
      bc += wt[1][w];
    }
    carry_t += wt[0][0] + wt[0][1] + wt[0][2] + wt[0][3];
    carry_c += wt[1][0] + wt[1][1] + wt[1][2] + wt[1][3];
    __syncthreads();   // every read of wt is done before the next users' totals
#pragma unroll
    for (int i = 0; i < UPT; ++i) {
      if (ub + i < R) {
        tile_base[ub + i] = bt;
        chunk_base[ub + i] = bc;
      }
      bt += t[i];
      bc += c[i];
    }
  }
  if (tid == 0 && (offsets[0] != 0 || offsets[R] != L.N)) bad = 1;
  bad = __syncthreads_or(bad);   // also orders the stores above before those below
  if (bad) {
    for (int u = tid; u < R; u += 256) {
      tile_base[u] = 0;
      chunk_base[u] = 0;
    }
    carry_t = 0;
    carry_c = 0;
  }
  if (tid == 0) {
    int32_t* hdr = ws_i32(ws, L.off_hdr);
    if (L.dtype == 0) {
      // zero pairs after the last tile: pass 2 reads each token's -l pair
      // together with the next three tokens' (multiplied by zeros there)
      uint32_t* nl = reinterpret_cast<uint32_t*>(ws_i32(ws, L.off_nl)) + (int64_t)carry_t * kTile;
      nl[0] = 0u;
      nl[1] = 0u;
      nl[2] = 0u;
      nl[3] = 0u;
    }
    tile_base[R] = carry_t;
    chunk_base[R] = carry_c;
    hdr[kHdrErr] = bad ? kErrBadOffsets : 0;
    hdr[kHdrTiles] = carry_t;
    hdr[kHdrChunks] = carry_c;
    hdr[kHdrHmax] = 0;
  }
}

// Per-launch preparation in one launch: workgroups 0 .. nq - 1 compute the
// queries, workgroup nq the schedule (the two are independent).
template <int D, typename T>
__global__ __launch_bounds__(256) void prep(const T* __restrict__ P, const T* __restrict__ Wk,
                                            const int64_t* __restrict__ offsets, Layout L, void* ws, int nq) {
  const int blk = blockIdx.x;
  if (blk == nq) {
    schedule(offsets, L, ws);
    return;
  }
  if constexpr (std::is_same<T, uint16_t>::value) queries_bf16<D>(P, Wk, L, ws, blk);
  else queries_f32<D>(P, Wk, L, ws, blk);
}

// The schedule alone (target attention's candidate tiles).
__global__ __launch_bounds__(256) void prep_schedule(const int64_t* __restrict__ offsets, Layout L, void* ws) {
  schedule(offsets, L, ws);
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
  hipLaunchKernelGGL(prep_schedule, dim3(1), dim3(256), 0, stream, offsets, L, ws);
  return hipGetLastError();
}

hipError_t launch_prep(const Layout& L, const void* P, const void* Wk, const int64_t* offsets, void* ws,
                       hipStream_t stream) {
  // query workgroups: 32 (d = 128) or 64 (d = 64) rows each on MFMAs, 256 / d
  // rows each in fp32; one more workgroup for the schedule
  const int nq = L.dtype == 0 ? L.k / (L.d == 128 ? 32 : 64) : L.k / (256 / L.d);
  const dim3 grid((unsigned)(nq + 1)), block(256);
  if (L.dtype == 0) {
    if (L.d == 128)
      hipLaunchKernelGGL((prep<128, uint16_t>), grid, block, 0, stream, (const uint16_t*)P, (const uint16_t*)Wk,
                         offsets, L, ws, nq);
    else
      hipLaunchKernelGGL((prep<64, uint16_t>), grid, block, 0, stream, (const uint16_t*)P, (const uint16_t*)Wk,
                         offsets, L, ws, nq);
  } else {
    if (L.d == 128)
      hipLaunchKernelGGL((prep<128, float>), grid, block, 0, stream, (const float*)P, (const float*)Wk, offsets, L,
                         ws, nq);
    else
      hipLaunchKernelGGL((prep<64, float>), grid, block, 0, stream, (const float*)P, (const float*)Wk, offsets, L,
                         ws, nq);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !L.fused) return e;
  const int64_t words = (int64_t)L.groups * kXSlots * kTile * (L.k / kFusedProtos);
  hipLaunchKernelGGL(clear_words, dim3(64), dim3(256), 0, stream,
                     reinterpret_cast<uint64_t*>(reinterpret_cast<char*>(ws) + L.off_xbuf), words);
  return hipGetLastError();
}

}  // namespace sa
