// sa_pass2.hip — FlashSA pass 2 on gfx950 (bf16 inputs).
//
// With the per-token logsumexp from pass 1, each token's allocation over the
// prototypes is A[j,t] = 2^(q_j . h_t - lse_t) (softmax over prototypes:
// SequenceO1 blog "How it works" item 1, review FAQ on SA).  Pass 2 recomputes
// the logits tile by tile and accumulates, for its block of prototypes and its
// chunk of one user's tokens,
//     U[j, :] = sum_t A[j,t] h_t      m_j = sum_t A[j,t]
// in registers; the finalize kernel sums chunks, divides by the mass
// (prototype-wise normalisation) and applies Wv.  Nothing of size k x n is
// ever stored (blog "How it works" item 3).
//
// Per 32-token tile, each wave (64 prototypes = 2 blocks of 32) runs
//   GEMM1  C[t, j] = [h_t | features] . [q_j | 1, 1, 0..]  = L - l   (fp16 MFMA)
//   A'     = 2^C  (= 2^14 A, fits fp16), converted pairwise to fp16,
//          mass += A' pairs (v_dot2 on the rounded values)
//   GEMM2  U[j, c] += sum_t A'[j,t] h_t[c]                           (fp16 MFMA)
// The accumulator of GEMM1 holds prototype (lane % 32) and 16 tokens per lane;
// those registers are exactly the A operand of GEMM2 once the transposed tile
// stores tokens in the accumulator's row order (done by pass 1), so no data
// moves between lanes.  The 2^14 scale cancels in U / m.
//
// Work item = (chunk of <= tiles_per_chunk tiles of one user, prototype block
// of waves*64).  Workgroups are numbered so that the prototype blocks of one
// chunk land on the same XCD back to back (dispatch goes round-robin over the
// 8 XCDs), letting them share the chunk's tiles through that XCD's L2.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sa_device.h"
#include "sa_launch.h"

namespace sa {

template <int D, int WAVES>
__global__ __launch_bounds__(WAVES * 64) void pass2_accum(Layout L, void* ws) {
  constexpr int NT = WAVES * 64;
  constexpr int S = D / 16;        // history K steps
  constexpr int SF = S + 1;        // + the feature step
  constexpr int ROW = D + kFeat;
  constexpr int HS = ROW + 8;      // LDS row stride of token rows (fp16)
  constexpr int TS = kTile + 8;    // LDS row stride of the transposed tile (fp16)
  constexpr int DT = D / 32;       // 32-column blocks of the output
  constexpr int P_ROWS = kTile * ROW / 8;   // 16-B pieces per tile, token rows
  constexpr int P_TR = D * kTile / 8;       // 16-B pieces per tile, transposed
  constexpr int PIECES = P_ROWS + P_TR;
  constexpr int PPT = (PIECES + NT - 1) / NT;
  __shared__ __attribute__((aligned(16))) _Float16 hrow[2][kTile * HS];
  __shared__ __attribute__((aligned(16))) _Float16 htr[2][D * TS];

  const int32_t* hdr = ws_i32(ws, L.off_hdr);
  const int x = blockIdx.x, xcd = x & 7, slot = x >> 3;
  const int chunk = (slot / L.n_pblocks) * 8 + xcd;
  const int pb = slot % L.n_pblocks;
  if (chunk >= hdr[kHdrChunks]) return;  // uniform over the workgroup

  const int32_t* tile_base = ws_i32(ws, L.off_tile_base);
  const int32_t* chunk_base = ws_i32(ws, L.off_chunk_base);
  const int u = find_user(chunk_base, L.R, chunk);
  const int ci = chunk - chunk_base[u];
  const int CT = L.tiles_per_chunk;
  const int tiles_u = tile_base[u + 1] - tile_base[u];
  const int32_t t0 = tile_base[u] + ci * CT;
  const int nt = min(CT, tiles_u - ci * CT);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, g = lane >> 5;
  const int p0 = pb * (WAVES * kProtoPerWave) + wave * kProtoPerWave;

  const _Float16* q16 = ws_f16(ws, L.off_q16);
  half8 qf[2][SF];
#pragma unroll
  for (int pt = 0; pt < 2; ++pt)
#pragma unroll
    for (int s = 0; s < SF; ++s)
      qf[pt][s] = *reinterpret_cast<const half8*>(q16 + (int64_t)(p0 + 32 * pt + col) * ROW + 16 * s + 8 * g);

  const _Float16* h16 = ws_f16(ws, L.off_h16);
  const _Float16* h16t = ws_f16(ws, L.off_h16t);
  auto load_tile = [&](int32_t tile, u32x4 (&pre)[PPT]) {
    const _Float16* rows = h16 + (int64_t)tile * kTile * ROW;
    const _Float16* tr = h16t + (int64_t)tile * D * kTile;
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
      const int p = tid + NT * i;
      if (p < P_ROWS) {
        pre[i] = *reinterpret_cast<const u32x4*>(rows + p * 8);
      } else if (p < PIECES) {
        pre[i] = *reinterpret_cast<const u32x4*>(tr + (p - P_ROWS) * 8);
      }
    }
  };
  auto store_tile = [&](int buf, const u32x4 (&pre)[PPT]) {
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
      const int p = tid + NT * i;
      if (p < P_ROWS) {
        const int r = p / (ROW / 8), c = p % (ROW / 8);
        *reinterpret_cast<u32x4*>(&hrow[buf][r * HS + c * 8]) = pre[i];
      } else if (p < PIECES) {
        const int q = p - P_ROWS, r = q / (kTile / 8), c = q % (kTile / 8);
        *reinterpret_cast<u32x4*>(&htr[buf][r * TS + c * 8]) = pre[i];
      }
    }
  };

  float16v U[2][DT];
#pragma unroll
  for (int pt = 0; pt < 2; ++pt)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) U[pt][dt] = float16v{};
  float msum[2] = {0.f, 0.f};
  const half2v ones = {(_Float16)1.0f, (_Float16)1.0f};

  {
    u32x4 pre[PPT];
    load_tile(t0, pre);
    store_tile(0, pre);
  }
  __syncthreads();

  for (int i = 0; i < nt; ++i) {
    const int buf = i & 1;
    u32x4 pre[PPT];
    if (i + 1 < nt) load_tile(t0 + i + 1, pre);

    // GEMM1: C[t, j] = L[j, t] - l_t for the wave's 2 x 32 prototypes
    float16v Cm[2] = {float16v{}, float16v{}};
#pragma unroll
    for (int s = 0; s < SF; ++s) {
      const half8 ha = *reinterpret_cast<const half8*>(&hrow[buf][col * HS + 16 * s + 8 * g]);
#pragma unroll
      for (int pt = 0; pt < 2; ++pt) Cm[pt] = mfma32x32x16(ha, qf[pt][s], Cm[pt]);
    }
    // allocations (scaled by 2^14) in fp16, and the masses of the rounded values
    half8 ap[2][2];
#pragma unroll
    for (int pt = 0; pt < 2; ++pt)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          float2v v = {__builtin_amdgcn_exp2f(Cm[pt][8 * kk + e]), __builtin_amdgcn_exp2f(Cm[pt][8 * kk + e + 1])};
          half2v h = __builtin_convertvector(v, half2v);
          msum[pt] = __builtin_amdgcn_fdot2(h, ones, msum[pt], false);
          ap[pt][kk][e] = h[0];
          ap[pt][kk][e + 1] = h[1];
        }
    // GEMM2: U[j, c] += sum_t A'[j, t] h_t[c]
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const half8 hb = *reinterpret_cast<const half8*>(&htr[buf][(32 * dt + col) * TS + 16 * kk + 8 * g]);
#pragma unroll
        for (int pt = 0; pt < 2; ++pt) U[pt][dt] = mfma32x32x16(ap[pt][kk], hb, U[pt][dt]);
      }
    if (i + 1 < nt) store_tile(buf ^ 1, pre);
    __syncthreads();
  }

  float* part_u = ws_f32(ws, L.off_part_u) + (int64_t)chunk * L.k * D;
  float* part_m = ws_f32(ws, L.off_part_m) + (int64_t)chunk * L.k;
#pragma unroll
  for (int pt = 0; pt < 2; ++pt) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        part_u[(int64_t)(p0 + 32 * pt + acc_row(r, g)) * D + 32 * dt + col] = U[pt][dt][r];
    const float m = msum[pt] + __shfl_xor(msum[pt], 32);
    if (g == 0) part_m[p0 + 32 * pt + col] = m;
  }
}

hipError_t launch_pass2(const Layout& L, void* ws, hipStream_t stream) {
  const int64_t padded = ((int64_t)L.chunks_max + 7) / 8 * 8;
  const int64_t grid = padded * L.n_pblocks;
  if (grid == 0) return hipSuccess;
#define SA_P2(DD, WW) \
  hipLaunchKernelGGL((pass2_accum<DD, WW>), dim3((unsigned)grid), dim3(WW * 64), 0, stream, L, ws)
  if (L.d == 128) {
    switch (L.waves) {
      case 4: SA_P2(128, 4); break;
      case 3: SA_P2(128, 3); break;
      case 2: SA_P2(128, 2); break;
      default: SA_P2(128, 1); break;
    }
  } else {
    switch (L.waves) {
      case 4: SA_P2(64, 4); break;
      case 3: SA_P2(64, 3); break;
      case 2: SA_P2(64, 2); break;
      default: SA_P2(64, 1); break;
    }
  }
#undef SA_P2
  return hipGetLastError();
}

}  // namespace sa
