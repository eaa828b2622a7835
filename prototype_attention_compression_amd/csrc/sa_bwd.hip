// sa_bwd.hip — the backward pass of Sketch Attention compression on gfx950
// (bf16 inputs): given dS = dLoss/dS for every user's sketch, the gradients
// dLoss/dH (per token) and dLoss/dP, dLoss/dWk, dLoss/dWv (summed over the
// users).  SequenceO1 trains the compressor end to end through the ranking
// loss (blog "100,000 videos in your pocket", "How it works" item 1: the
// compression is differentiable and its gradients reach the prototypes and
// projections; same page, "Takeaways": the compressor is trained on the real
// loss).  The pages give no backward formulas; these follow from the chain
// rule on the forward definition (softmax over prototypes per token, each
// sketch row the mass-weighted mean of v_t = h_t Wv).
//
// With A[j,t] the allocations, m_j the masses, Sbar_j = (sum_t A[j,t] h_t) / m_j
// (so S_j = Sbar_j Wv) and G = dS:
//   Gm_j  = G_j / m_j,   Z_j = Gm_j Wv^T,   c_j = Z_j . Sbar_j        (per user)
//   dA[j,t] = Z_j . h_t - c_j                  (through both U and the mass)
//   delta_t = sum_j A[j,t] dA[j,t]
//   dL[j,t] = A[j,t] (dA[j,t] - delta_t)       (softmax Jacobian per token)
//   dh_t    = sum_j A[j,t] Z_j + dL[j,t] q'_j, q' = P Wk^T / sqrt(d)
//   E_j     = sum_t dL[j,t] h_t  (over every token of the batch)
//   dP = E Wk / sqrt(d),  dWk = E^T P / sqrt(d),  dWv = sum_u Sbar_u^T G_u
// Every per-token product is a contraction with the token row h_t, so the
// kernels reuse the fp16 token rows and logsumexps of forward passes 1 and 2
// and never form a k x n array:
//   bwd_user   per (user, 32 prototypes): sums pass 2's partial slots into
//              U and m, writes Sbar, Z (fp32) and the block's largest |Z|;
//   bwd_zpack  per user scale zs (a power of two putting max |Z| in
//              [2^13, 2^14)): Z zs in fp16 (MFMA operand) and c zs from
//              that rounded row;
//   bwd_dh     token-major: a wave owns a 32-token tile with its rows as the
//              B operand in registers and walks every prototype block twice
//              (queries and Z rows staged in LDS): sweep 1 sums delta_t and
//              the bound b_t = max_j |Y - c|; sweep 2 forms A and dL in fp16
//              with a per-token power-of-two scale and accumulates dh_t
//              with MFMAs whose B operands are the staged rows read with the
//              transposing LDS read;
//   bwd_e      prototype-major (like pass 2): E += dL h over token tiles,
//              queries and Z rows resident, per-user scale, partial E per
//              (group, user) segment;
//   bwd_ereduce, bwd_outer, bwd_sum: E, dP, dWk, dWv.
// Both token kernels run two waves per SIMD and stage their operand blocks
// two steps ahead through registers of a native vector type (an array of
// the struct-typed uint4 stayed in scratch memory, with a wait right after
// every prefetch).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <type_traits>

#include "sa_device.h"
#include "sa_launch.h"
#include "sa_slots.h"

namespace sa {

namespace {

constexpr int kRows = 32;                         // prototypes per bwd_user workgroup
constexpr float kLn2 = 0.69314718055994531f;
constexpr float kScaleMax = 16384.0f;             // 2^14
constexpr int kSlotBatch = 4;                     // partial slots whose loads are in flight together
constexpr int kERows = 8;                         // prototypes per E-reduction workgroup
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 half4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16f(uint16_t v) { return __uint_as_float(((uint32_t)v) << 16); }

// 2^e with 2^e x in [2^(t-1), 2^t) for finite x > 0 (e clamped to +-100);
// 1 otherwise.
__device__ __forceinline__ float pow2_scale(float x, int t) {
  if (!(x > 0.f) || !(x < INFINITY)) return 1.f;
  int ex = 0;
  (void)frexpf(x, &ex);   // x = f 2^ex, f in [0.5, 1)
  const int e = max(-100, min(100, t - ex));
  return ldexpf(1.f, e);
}

// Scale for fp16 operands derived from a bound b on |Y - c|: |dL| <= 2 b, so
// with s b < 2^14 the scaled dL stays below 2^15; the scaled allocations
// (<= s <= 2^14) also fit fp16.
__device__ __forceinline__ float operand_scale(float b) {
  return b > 0.f ? fminf(kScaleMax, pow2_scale(b, 14)) : kScaleMax;
}

// log2 of such a scale (a normal power of two, 2^-100 .. 2^14), as an fp16
// value (exact): a feature step that adds it to the logits makes the
// exponentials come out already scaled
__device__ __forceinline__ _Float16 scale_log2(float s) {
  return (_Float16)(float)((int)((__float_as_uint(s) >> 23) & 0xFFu) - 127);
}

// Position of token i of a tile among the 16 accumulator registers of lane
// half g (GEMM rows read from LDS row tau(m)): i = tau(acc_row(r, g)).
__device__ __forceinline__ int acc_pos(int i) {
  const int kk = i >> 4, g = (i >> 1) & 1, q = ((i & 1) << 2) | ((i >> 2) & 3);
  return 16 * g + 8 * kk + q;
}

__device__ __forceinline__ float negl_of(uint32_t w) {
  const half2v p = __builtin_bit_cast(half2v, w);
  return (float)p[0] + (float)p[1] - kAllocShift;
}

}  // namespace

// ---------------------------------------------------------------- per user
// Sbar_in / mass_in (optional): the forward's mass-normalised rows and
// masses of these inputs, given instead of pass 2's partial sums.
template <int D>
__global__ __launch_bounds__(256) void bwd_user(const uint16_t* __restrict__ Wv, const float* __restrict__ dS,
                                                const float* __restrict__ Sbar_in, const float* __restrict__ mass_in,
                                                Layout L, void* ws, int presummed) {
  constexpr int PER = kRows * D / 256;
  __shared__ float gz[kRows][D + 1];   // dS / m
  __shared__ float ms[kRows];
  __shared__ float red[256];
  const int nrb = L.k / kRows;
  const int u = blockIdx.x / nrb, rb = blockIdx.x % nrb;
  const int j0 = rb * kRows;
  const int tid = threadIdx.x;
  const int64_t row0 = (int64_t)u * L.k + j0;
  float acc[PER];
  if (Sbar_in == nullptr) {
    // the user's partial slots, or the heads of their pre-summed sub-ranges,
    // added in slot order exactly as the forward's finalize adds them (the
    // same values to the bit)
    int c0, c1;
    user_slots(L, ws, u, c0, c1);
    const int n = c1 - c0;
    const bool pre = presummed && n > kPreMin;
    const float* part_u = ws_f32(ws, L.off_part_u);
    const float* part_m = ws_f32(ws, L.off_part_m);
#pragma unroll
    for (int i = 0; i < PER; ++i) acc[i] = 0.f;
    if (pre) {
      float v[kPreSplit][PER];
#pragma unroll
      for (int q = 0; q < kPreSplit; ++q) {
        const float* base = part_u + ((int64_t)sub_head(c0, n, q) * L.k + j0) * D;
#pragma unroll
        for (int i = 0; i < PER; ++i) v[q][i] = base[tid + 256 * i];
      }
#pragma unroll
      for (int q = 0; q < kPreSplit; ++q)
#pragma unroll
        for (int i = 0; i < PER; ++i) acc[i] += v[q][i];
    } else {
      int c = c0;
      for (; c + kSlotBatch <= c1; c += kSlotBatch) {
        float v[kSlotBatch][PER];
#pragma unroll
        for (int q = 0; q < kSlotBatch; ++q) {
          const float* base = part_u + ((int64_t)(c + q) * L.k + j0) * D;
#pragma unroll
          for (int i = 0; i < PER; ++i) v[q][i] = base[tid + 256 * i];
        }
#pragma unroll
        for (int q = 0; q < kSlotBatch; ++q)
#pragma unroll
          for (int i = 0; i < PER; ++i) acc[i] += v[q][i];
      }
      for (; c < c1; ++c) {
        const float* base = part_u + ((int64_t)c * L.k + j0) * D;
#pragma unroll
        for (int i = 0; i < PER; ++i) acc[i] += base[tid + 256 * i];
      }
    }
    if (tid < kRows) {
      float m = 0.f;
      if (pre) {
        for (int q = 0; q < kPreSplit; ++q) m += part_m[(int64_t)sub_head(c0, n, q) * L.k + j0 + tid];
      } else {
        for (int cc = c0; cc < c1; ++cc) m += part_m[(int64_t)cc * L.k + j0 + tid];
      }
      ms[tid] = m;   // 2^14 m (the allocations of pass 2 carry 2^14)
    }
  } else {
#pragma unroll
    for (int i = 0; i < PER; ++i) acc[i] = Sbar_in[row0 * D + tid + 256 * i];
    if (tid < kRows) ms[tid] = mass_in[row0 + tid] * kScaleMax;   // 2^14 m, as above
  }
  __syncthreads();
  float* sbar = ws_f32(ws, L.off_bsbar) + row0 * D;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = tid + 256 * i, j = e / D, a = e % D;
    const float m = ms[j];
    const float v = m > 0.f ? (Sbar_in == nullptr ? acc[i] / m : acc[i]) : 0.f;
    sbar[e] = v;
    gz[j][a] = m > 0.f ? dS[row0 * D + e] * (kScaleMax / m) : 0.f;
  }
  __syncthreads();
  // Z[j][a] = sum_b Gm[j][b] Wv[a][b] on bf16 MFMAs: wave w takes columns
  // a = 32 w .. 32 w + 31 (D = 64: waves 0 and 1).  The B operand
  // (8 consecutive b of row a of Wv) is a plain 16-byte load; Wv is exact in
  // bf16 and each fp32 Gm value is split exactly into three bf16 terms, so
  // the products keep fp32 accuracy with fp32 sums.
  const int lane = tid & 63, wave = tid >> 6, col = lane & 31, g = lane >> 5;
  float16v zacc = float16v{};
  const bool zw = 32 * wave < D;   // uniform over the wave
  if (zw) {
    const bf16x8* wrow = reinterpret_cast<const bf16x8*>(Wv + (int64_t)(32 * wave + col) * D);
    bf16x8 wb[D / 16];
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) wb[ks] = wrow[2 * ks + g];
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      const int k0 = 16 * ks + 8 * g;
      bf16x8 hi, mid, lo;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = gz[col][k0 + e];
        const __bf16 h = (__bf16)x;
        const float r1 = x - (float)h;
        const __bf16 m1 = (__bf16)r1;
        hi[e] = h;
        mid[e] = m1;
        lo[e] = (__bf16)(r1 - (float)m1);
      }
      zacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(hi, wb[ks], zacc, 0, 0, 0);
      zacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(mid, wb[ks], zacc, 0, 0, 0);
      zacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lo, wb[ks], zacc, 0, 0, 0);
    }
  }
  float zm = 0.f;
  float* z32 = ws_f32(ws, L.off_bz32) + row0 * D;
  if (zw) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int j = acc_row(r, g), a = 32 * wave + col;
      z32[(int64_t)j * D + a] = zacc[r];
      zm = fmaxf(zm, fabsf(zacc[r]));
    }
  }
  red[tid] = zm;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if (tid < off) red[tid] = fmaxf(red[tid], red[tid + off]);
    __syncthreads();
  }
  if (tid == 0) ws_f32(ws, L.off_bzmax)[(int64_t)u * nrb + rb] = red[0];
}

template <int D>
__global__ __launch_bounds__(256) void bwd_zpack(Layout L, void* ws) {
  __shared__ float red[256];
  const int nrb = L.k / kRows;
  const int u = blockIdx.x / nrb, rb = blockIdx.x % nrb;
  const int tid = threadIdx.x;
  const float* bm = ws_f32(ws, L.off_bzmax) + (int64_t)u * nrb;
  float m = 0.f;
  for (int i = tid; i < nrb; i += 256) m = fmaxf(m, bm[i]);
  red[tid] = m;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if (tid < off) red[tid] = fmaxf(red[tid], red[tid + off]);
    __syncthreads();
  }
  const float zs = pow2_scale(red[0], 14);
  const int64_t row0 = (int64_t)u * L.k + rb * kRows;
  // 8 threads per row, each with 16-byte pieces part + 8 m of it: Z zs in
  // fp16, and c_j zs = Zs_j . Sbar_j from that rounded row itself, so that
  // Y - c zs = Zs_j . (h_t - Sbar_j) keeps its accuracy where h_t is close to
  // Sbar_j (a user of one token: exactly zero), rather than the fp16 rounding
  // of Zs_j . h_t
  const int j = tid >> 3, part = tid & 7;
  const f32x4* zr = reinterpret_cast<const f32x4*>(ws_f32(ws, L.off_bz32) + (row0 + j) * D);
  const f32x4* sr = reinterpret_cast<const f32x4*>(ws_f32(ws, L.off_bsbar) + (row0 + j) * D);
  half4v* zo = reinterpret_cast<half4v*>(ws_f16(ws, L.off_bz16) + (row0 + j) * D);
  f32x4 zv[D / 32], sv[D / 32];
#pragma unroll
  for (int m = 0; m < D / 32; ++m) {
    zv[m] = zr[part + 8 * m];
    sv[m] = sr[part + 8 * m];
  }
  float s = 0.f;
#pragma unroll
  for (int m = 0; m < D / 32; ++m) {
    half4v h;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      h[c] = (_Float16)(zv[m][c] * zs);
      s = fmaf((float)h[c], sv[m][c], s);
    }
    zo[part + 8 * m] = h;
  }
  s += __shfl_xor(s, 1);
  s += __shfl_xor(s, 2);
  s += __shfl_xor(s, 4);
  if (part == 0) ws_f32(ws, L.off_bcz)[row0 + j] = s;
  if (rb == 0 && tid == 0) {
    ws_f32(ws, L.off_bzs)[u] = zs;
    ws_i32(ws, L.off_bbmax)[u] = 0;
  }
}

// ---------------------------------------------------------------- dH
// One workgroup = 4 waves = 4 consecutive tiles (one user: every user's tile
// count is a multiple of 4).  Each wave keeps its tile's rows as the B
// operand (token = lane % 32) of C[j, t] = q_j . h_t and Y[j, t] = Zs_j . h_t,
// whose A operands (32 prototypes, row tau(m) of the staged block) come from
// LDS.  The accumulators hold prototype tau(acc_row(r, g)) and token lane % 32,
// which is exactly the A operand (row = token, contraction = prototypes) of
// dh = sum_j (sA[j, t] Zs_j + sdL[j, t] ln2 q_j); its B operands are the
// staged rows through the transposing read.
template <int D>
__global__ __launch_bounds__(256, 2) void bwd_dh(const int64_t* __restrict__ offsets,
                                              const int32_t* __restrict__ tile_base, Layout L, void* ws,
                                              float* __restrict__ dH) {
  constexpr int S = D / 16, DT = D / 32, PITCH = tile_pitch<D>(), BLK = kTile * PITCH, CPR = D / 8;
  constexpr int LPT = kTile * CPR / 256;            // 16-B loads per thread per staged block
  static_assert(LPT * 256 == kTile * CPR, "whole loads");
  constexpr int STAGE = 2 * BLK + 2 * kTile * 4;
  __shared__ __attribute__((aligned(16))) char lds[2][STAGE];
  __shared__ float sinv[4][kTile];
  const int32_t T = ws_i32(ws, L.off_hdr)[kHdrTiles];
  const int tid = threadIdx.x;
  if (T == 0) {
    // offsets broke their contract: every user counts as empty, dh = 0
    const int64_t n = L.N * D;
    for (int64_t i = (int64_t)blockIdx.x * 256 + tid; i < n; i += (int64_t)gridDim.x * 256) dH[i] = 0.f;
    return;
  }
  const int quad = blockIdx.x;
  if (4 * quad >= T) return;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, g = lane >> 5;
  const int tile = 4 * quad + wave;
  const int u = find_user(tile_base, L.R, 4 * quad);
  const int64_t tok0 = offsets[u] + (int64_t)(tile - tile_base[u]) * kTile;
  const int64_t rem = offsets[u + 1] - tok0;
  const int count = rem < 0 ? 0 : (rem < kTile ? (int)rem : kTile);

  const _Float16* q16 = ws_f16(ws, L.off_q16);
  const _Float16* z16 = ws_f16(ws, L.off_bz16) + (int64_t)u * L.k * D;
  const float* czu = ws_f32(ws, L.off_bcz) + (int64_t)u * L.k;
  const float zs = ws_f32(ws, L.off_bzs)[u];

  const _Float16* hrow = ws_f16(ws, L.off_h16) + ((int64_t)tile * kTile + col) * D;
  half8 hB[S];
#pragma unroll
  for (int s = 0; s < S; ++s) hB[s] = *reinterpret_cast<const half8*>(hrow + 16 * s + 8 * g);
  const uint32_t nlw = reinterpret_cast<const uint32_t*>(ws_i32(ws, L.off_nl))[(int64_t)tile * kTile + col];
  const bool keep = negl_of(nlw) > -30000.f;
  // Feature step of the logits: the token supplies (-l_hi, -l_lo, -14, e)
  // (the lower lane half's K positions), the prototype (1, 1, 1, 1), so the
  // logit accumulators start at e - lse_t and the allocations are
  // 2^accumulator = 2^e A; e = 0 in sweep 1, log2 of the token's operand
  // scale in sweep 2
  const half2v nlp = __builtin_bit_cast(half2v, nlw);
  const _Float16 z0 = (_Float16)0.0f;
  const half8 hfeat = g == 0 ? half8{nlp[0], nlp[1], (_Float16)(-kAllocShift), z0, z0, z0, z0, z0}
                             : half8{z0, z0, z0, z0, z0, z0, z0, z0};
  const half8 qones = {(_Float16)1.0f, (_Float16)1.0f, (_Float16)1.0f, (_Float16)1.0f, z0, z0, z0, z0};

  const int NB = L.k / kTile;
  // Staging of the 2 NB block steps (block i % NB of sweep i / NB): two
  // register sets, so the global loads of step i + 2 are issued while step i
  // is computed and step i + 1 (loaded an iteration earlier) goes to LDS at
  // the end of the iteration.
  u32x4 qa[LPT], za[LPT], qb2[LPT], zb2[LPT];
  float ca = 0.f, cb = 0.f;
  auto gload = [&](int i, u32x4 (&q)[LPT], u32x4 (&z)[LPT], float& c) {
    const int jb = i % NB;
#pragma unroll
    for (int k2 = 0; k2 < LPT; ++k2) {
      const int idx = tid + 256 * k2, row = idx / CPR, ch = idx % CPR;
      q[k2] = *reinterpret_cast<const u32x4*>(q16 + (int64_t)(jb * kTile + row) * D + 8 * ch);
      z[k2] = *reinterpret_cast<const u32x4*>(z16 + (int64_t)(jb * kTile + row) * D + 8 * ch);
    }
    if (tid < kTile) c = czu[jb * kTile + tid];
  };
  auto swrite = [&](int buf, const u32x4 (&q)[LPT], const u32x4 (&z)[LPT], float c) {
    char* base = lds[buf];
#pragma unroll
    for (int k2 = 0; k2 < LPT; ++k2) {
      const int idx = tid + 256 * k2, row = idx / CPR, ch = idx % CPR;
      *reinterpret_cast<u32x4*>(base + row * PITCH + 16 * ch) = q[k2];
      *reinterpret_cast<u32x4*>(base + BLK + row * PITCH + 16 * ch) = z[k2];
    }
    if (tid < kTile) reinterpret_cast<float*>(base + 2 * BLK)[acc_pos(tid)] = c;
  };
  // step i (even: set b holds step i + 1, set a is free; odd: the reverse)
  auto run = [&](int i, auto odd, auto&& body) {
    if constexpr (!decltype(odd)::value) {
      if (i + 2 < 2 * NB) gload(i + 2, qa, za, ca);
    } else {
      if (i + 2 < 2 * NB) gload(i + 2, qb2, zb2, cb);
    }
    body(static_cast<const char*>(lds[i & 1]));
    if constexpr (!decltype(odd)::value) {
      if (i + 1 < 2 * NB) swrite((i + 1) & 1, qb2, zb2, cb);
    } else {
      if (i + 1 < 2 * NB) swrite((i + 1) & 1, qa, za, ca);
    }
    __syncthreads();
  };
  using Even = std::false_type;
  using Odd = std::true_type;

  const int abase = tau(col) * PITCH + 16 * g;
  const int i16 = lane & 15, gh = (lane >> 4) & 1;
  const int tr_base = (4 * (i16 >> 2) + 2 * g) * PITCH + 32 * gh + 8 * (i16 & 3);

  float dsum = 0.f, bmx = 0.f;
  float16v dHc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) dHc[dt] = float16v{};

  // C = q . h and Y = Zs . h of the staged block (A operands read in halves)
  auto gemms = [&](const char* qb, float16v& Lc, float16v& Yc, const half8& feat) {
    Lc = mfma32x32x16(qones, feat, float16v{});
    Yc = float16v{};
#pragma unroll
    for (int s0 = 0; s0 < S; s0 += 4) {
      half8 a[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) a[s] = *reinterpret_cast<const half8*>(qb + abase + 32 * (s0 + s));
#pragma unroll
      for (int s = 0; s < 4; ++s) Lc = mfma32x32x16(a[s], hB[s0 + s], Lc);
    }
#pragma unroll
    for (int s0 = 0; s0 < S; s0 += 4) {
      half8 a[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) a[s] = *reinterpret_cast<const half8*>(qb + BLK + abase + 32 * (s0 + s));
#pragma unroll
      for (int s = 0; s < 4; ++s) Yc = mfma32x32x16(a[s], hB[s0 + s], Yc);
    }
  };

  // sweep 1: delta_t and the bound b_t
  auto sweep1 = [&](const char* qb) {
    float16v Lc, Yc;
    gemms(qb, Lc, Yc, hfeat);
    const float4* cp = reinterpret_cast<const float4*>(qb + 2 * BLK) + 4 * g;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const float4 c4 = cp[v];
      const float cv[4] = {c4.x, c4.y, c4.z, c4.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float A = __builtin_amdgcn_exp2f(Lc[4 * v + e]);
        const float yc = Yc[4 * v + e] - cv[e];
        dsum = fmaf(A, yc, dsum);
        bmx = fmaxf(bmx, fabsf(yc));
      }
    }
  };
  gload(0, qa, za, ca);
  swrite(0, qa, za, ca);
  gload(1, qb2, zb2, cb);
  __syncthreads();
  for (int i = 0; i < NB; i += 2) {   // NB = k / 32 is even
    run(i, Even{}, sweep1);
    run(i + 1, Odd{}, sweep1);
  }
  dsum += __shfl_xor(dsum, 32);
  bmx = fmaxf(bmx, __shfl_xor(bmx, 32));
  if (!keep) bmx = 0.f;
  const float delta = dsum;
  const float sg = operand_scale(bmx);
  // sweep 2's feature operand: the allocations come out as sg A
  half8 hfeat2 = hfeat;
  if (g == 0) hfeat2[3] = scale_log2(sg);
  if (g == 0) {
    sinv[wave][col] = 1.0f / (sg * zs);
    ws_f32(ws, L.off_bdelta)[(int64_t)tile * kTile + col] = delta;
  }
  {
    float wm = bmx;
#pragma unroll
    for (int o = 16; o > 0; o >>= 1) wm = fmaxf(wm, __shfl_xor(wm, o));
    if (lane == 0 && wm > 0.f)
      atomicMax(reinterpret_cast<unsigned int*>(ws_i32(ws, L.off_bbmax)) + u, __float_as_uint(wm));
  }
  // sweep 2: dh += (sg ln2 dL)^T q + (sg A)^T Zs
  auto sweep2 = [&](const char* qb) {
    float16v Lc, Yc;
    gemms(qb, Lc, Yc, hfeat2);
    const float4* cp = reinterpret_cast<const float4*>(qb + 2 * BLK) + 4 * g;
    half8 al[2], ad[2];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const float4 c4 = cp[v];
      const float cv[4] = {c4.x, c4.y, c4.z, c4.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * v + e;
        const float A = __builtin_amdgcn_exp2f(Lc[r]);   // sg A
        const float dl = A * (Yc[r] - cv[e] - delta);
        al[r >> 3][r & 7] = (_Float16)(dl * kLn2);
        ad[r >> 3][r & 7] = (_Float16)A;
      }
    }
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      half8 hb[DT];
      tile_tr_reads_kk<D>(lds_addr(qb) + tr_base + kk * 16 * PITCH, hb);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) dHc[dt] = mfma32x32x16(al[kk], hb[dt], dHc[dt]);
    }
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      half8 hb[DT];
      tile_tr_reads_kk<D>(lds_addr(qb + BLK) + tr_base + kk * 16 * PITCH, hb);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) dHc[dt] = mfma32x32x16(ad[kk], hb[dt], dHc[dt]);
    }
  };
  for (int i = NB; i < 2 * NB; i += 2) {
    run(i, Even{}, sweep2);
    run(i + 1, Odd{}, sweep2);
  }
  // accumulator rows are tokens acc_row(r, g), columns 32 dt + col
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int t = acc_row(r, g);
    if (t < count) {
      const float sc = sinv[wave][t];
      float* dst = dH + (tok0 + t) * D + col;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) dst[32 * dt] = dHc[dt][r] * sc;
    }
  }
}

// ---------------------------------------------------------------- E
// Prototype-major like pass 2: W waves of 32 prototypes; groups of
// e_pblocks workgroups walk equal tile ranges cut at user boundaries; per
// tile
//   C[t, j] = h_t . q_j, Y[t, j] = h_t . Zs_j (token rows from LDS as the A
//   operand, queries and Z rows resident as B operands),
//   sdL = s_u A (Y - cs_j - delta_t) in fp16, E += sdL h (transposing reads).
// A segment's E, rescaled to true units, goes to partial slot group + user
// (unique among the groups whose ranges meet that user, as in pass 2).
template <int D, int W>
__global__ __launch_bounds__(W * 64, W == 8 ? 1 : 2) void bwd_e(const int32_t* __restrict__ tile_base, Layout L, void* ws) {
  constexpr int S = D / 16, DT = D / 32, PITCH = tile_pitch<D>(), TB = kTile * PITCH, CPR = D / 8;
  constexpr int NT = W * 64;
  constexpr int LPT = kTile * CPR / NT;
  static_assert(LPT * NT == kTile * CPR, "whole loads");
  // the tile's rows, then per token the logits' feature piece
  // {-l_hi, -l_lo, -14, 1, 0 ...} (16 bytes), then delta_t zs (floats)
  constexpr int FEAT = TB, DLT = TB + kTile * 16;
  constexpr int STAGE = DLT + kTile * 4;
  __shared__ __attribute__((aligned(16))) char lds[2][STAGE];
  const int P = L.e_pblocks, G = L.e_groups;
  const int x = blockIdx.x, xcd = x & 7, slotw = x >> 3;
  const int group = xcd + 8 * (slotw / P);
  const int pb = slotw % P;
  if (group >= G) return;
  const int32_t T = ws_i32(ws, L.off_hdr)[kHdrTiles];
  const int32_t Tg = (T + 4 * G - 1) / (4 * G) * 4;
  const int32_t s0 = group * Tg, s1 = min(T, s0 + Tg);
  if (s0 >= s1) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, g = lane >> 5;
  const int p0 = pb * (W * kTile) + wave * kTile;

  const _Float16* q16 = ws_f16(ws, L.off_q16);
  half8 qf[S], zf[S];
#pragma unroll
  for (int s = 0; s < S; ++s) qf[s] = *reinterpret_cast<const half8*>(q16 + (int64_t)(p0 + col) * D + 16 * s + 8 * g);
  const _Float16* h16 = ws_f16(ws, L.off_h16);
  const uint32_t* nlw = reinterpret_cast<const uint32_t*>(ws_i32(ws, L.off_nl));
  const float* dlt = ws_f32(ws, L.off_bdelta);
  u32x4 pr[LPT];
  uint32_t pn = 0;
  float pd = 0.f;
  auto gload = [&](int32_t t) {
    const _Float16* src = h16 + (int64_t)t * kTile * D;
#pragma unroll
    for (int k2 = 0; k2 < LPT; ++k2) {
      const int idx = tid + NT * k2, row = idx / CPR, ch = idx % CPR;
      pr[k2] = *reinterpret_cast<const u32x4*>(src + row * D + 8 * ch);
    }
    if (tid < kTile) {
      pn = nlw[(int64_t)t * kTile + tid];
      pd = dlt[(int64_t)t * kTile + tid];
    }
  };
  auto swrite = [&](int buf) {
    char* base = lds[buf];
#pragma unroll
    for (int k2 = 0; k2 < LPT; ++k2) {
      const int idx = tid + NT * k2, row = idx / CPR, ch = idx % CPR;
      *reinterpret_cast<u32x4*>(base + row * PITCH + 16 * ch) = pr[k2];
    }
    if (tid < kTile) {
      // -14 and 1 in fp16 are 0xCB00 and 0x3C00
      reinterpret_cast<u32x4*>(base + FEAT)[tid] = u32x4{pn, 0x3C00CB00u, 0u, 0u};
      reinterpret_cast<float*>(base + DLT)[acc_pos(tid)] = pd;
    }
  };
  const int abase = tau(col) * PITCH + 16 * g;
  const int i16 = lane & 15, gh = (lane >> 4) & 1;
  const int tr_base = (4 * (i16 >> 2) + 2 * g) * PITCH + 32 * gh + 8 * (i16 & 3);
  // feature step of the logits: the token's piece (A operand, lane's token
  // tau(col)) against (1, 1, 1, log2 su) at the lower lane half's K
  // positions, so the logit accumulators start at log2 su - lse_t and the
  // exponentials come out as su A (the upper half meets zeros)
  const int fbase = FEAT + tau(col) * 16;
  const _Float16 f1 = g == 0 ? (_Float16)1.0f : (_Float16)0.0f, f0 = (_Float16)0.0f;
  half8 qones = {f1, f1, f1, f0, f0, f0, f0, f0};

  int u = find_user(tile_base, L.R, s0);
  int32_t ub = tile_base[u + 1];
  float cz = 0.f, su = kScaleMax, back = 1.f;
  auto load_user = [&]() {
    const _Float16* z16 = ws_f16(ws, L.off_bz16) + ((int64_t)u * L.k + p0 + col) * D;
#pragma unroll
    for (int s = 0; s < S; ++s) zf[s] = *reinterpret_cast<const half8*>(z16 + 16 * s + 8 * g);
    cz = ws_f32(ws, L.off_bcz)[(int64_t)u * L.k + p0 + col];
    const float bm = __uint_as_float(reinterpret_cast<const uint32_t*>(ws_i32(ws, L.off_bbmax))[u]);
    su = operand_scale(bm);
    qones[3] = g == 0 ? scale_log2(su) : f0;
    back = 1.0f / (su * ws_f32(ws, L.off_bzs)[u]);
  };
  float16v Ea[DT];
  auto flush = [&]() {   // the segment of user u: true units to slot group + u
    float* dst = ws_f32(ws, L.off_bepart) + ((int64_t)(group + u) * L.k + p0) * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) dst[(int64_t)acc_row(r, g) * D + 32 * dt + col] = Ea[dt][r] * back;
  };
  load_user();
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) Ea[dt] = float16v{};

  gload(s0);
  swrite(0);
  __syncthreads();
  for (int32_t t = s0; t < s1; ++t) {
    const int buf = (t - s0) & 1;
    if (t + 1 < s1) gload(t + 1);
    if (t == ub) {   // uniform: the next user's tiles start here
      flush();
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) Ea[dt] = float16v{};
      while (tile_base[u + 1] <= t) ++u;
      ub = tile_base[u + 1];
      load_user();
    }
    const char* hb_ = lds[buf];
    float16v Lc = mfma32x32x16(*reinterpret_cast<const half8*>(hb_ + fbase), qones, float16v{});
    float16v Yc = float16v{};
#pragma unroll
    for (int s0h = 0; s0h < S; s0h += 4) {
      half8 ha[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) ha[s] = *reinterpret_cast<const half8*>(hb_ + abase + 32 * (s0h + s));
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        Lc = mfma32x32x16(ha[s], qf[s0h + s], Lc);
        Yc = mfma32x32x16(ha[s], zf[s0h + s], Yc);
      }
    }
    const float4* pv = reinterpret_cast<const float4*>(hb_ + DLT);
    half8 al[2];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const float4 d4 = pv[4 * g + v];
      const float dd[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * v + e;
        const float A = __builtin_amdgcn_exp2f(Lc[r]);   // su A
        al[r >> 3][r & 7] = (_Float16)(A * (Yc[r] - cz - dd[e]));
      }
    }
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      half8 hbv[DT];
      tile_tr_reads_kk<D>(lds_addr(hb_) + tr_base + kk * 16 * PITCH, hbv);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) Ea[dt] = mfma32x32x16(al[kk], hbv[dt], Ea[dt]);
    }
    if (t + 1 < s1) swrite(buf ^ 1);
    __syncthreads();
  }
  flush();
}

// ---------------------------------------------------------------- reductions
// E = sum over the (group, user) partial slots (users, then groups, in
// order: bitwise repeatable), and dP = E Wk / sqrt(d)
template <int D>
__global__ __launch_bounds__(256) void bwd_ereduce(const uint16_t* __restrict__ Wk,
                                                   const int32_t* __restrict__ tile_base, Layout L, void* ws,
                                                   float* __restrict__ dP) {
  constexpr int PER = kERows * D / 256;
  constexpr int RPI = 256 / D;
  constexpr int WCH = D * D / 8 / 256;   // 16-byte chunks of Wk per thread
  constexpr int SB = 16;                 // slots whose loads are in flight together
  __shared__ float es[kERows][D + 1];
  __shared__ __attribute__((aligned(16))) uint16_t wk[D * D];
  const int j0 = blockIdx.x * kERows, tid = threadIdx.x;
  {
    // Wk staged in LDS, all of its loads in flight together
    u32x4 w[WCH];
#pragma unroll
    for (int i = 0; i < WCH; ++i) w[i] = reinterpret_cast<const u32x4*>(Wk)[tid + 256 * i];
#pragma unroll
    for (int i = 0; i < WCH; ++i) reinterpret_cast<u32x4*>(wk)[tid + 256 * i] = w[i];
  }
  const float* ep = ws_f32(ws, L.off_bepart);
  float* et = ws_f32(ws, L.off_betot) + (int64_t)j0 * D;
  float acc[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) acc[i] = 0.f;
  // the slots bwd_e wrote: group + u for every group whose tile range meets
  // user u's tiles, walked users in order, then groups in order, with the
  // loads of SB consecutive slots of that walk in flight together
  const int32_t T = ws_i32(ws, L.off_hdr)[kHdrTiles];
  const int G = L.e_groups;
  const int32_t Tg = (T + 4 * G - 1) / (4 * G) * 4;
  int u = 0, c = 0, cend = 0;   // next user to open; the open user's remaining slots [c, cend)
  auto seek = [&]() {
    while (c >= cend) {
      if (u >= L.R) return false;
      const int32_t t0 = tile_base[u], t1 = tile_base[u + 1];
      if (t1 > t0) {
        c = t0 / Tg + u;
        cend = (t1 - 1) / Tg + 1 + u;
      }
      ++u;
    }
    return true;
  };
  for (;;) {
    int sl[SB];
    int n = 0;
#pragma unroll
    for (int q = 0; q < SB; ++q) {
      sl[q] = 0;
      if (n == q && seek()) {
        sl[q] = c++;
        ++n;
      }
    }
    if (n == 0) break;
    float v[SB][PER];
#pragma unroll
    for (int q = 0; q < SB; ++q) {
      if (q < n) {
        const float* base = ep + ((int64_t)sl[q] * L.k + j0) * D;
#pragma unroll
        for (int i = 0; i < PER; ++i) v[q][i] = base[tid + 256 * i];
      }
    }
#pragma unroll
    for (int q = 0; q < SB; ++q)
      if (q < n)
#pragma unroll
        for (int i = 0; i < PER; ++i) acc[i] += v[q][i];
  }
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = tid + 256 * i;
    et[e] = acc[i];
    es[e / D][e % D] = acc[i];
  }
  __syncthreads();
  const int b = tid % D, jr = tid / D;
  float out[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) out[i] = 0.f;
#pragma unroll 4
  for (int a = 0; a < D; ++a) {
    const float w = bf16f(wk[a * D + b]);
#pragma unroll
    for (int i = 0; i < PER; ++i) out[i] = fmaf(es[jr + RPI * i][a], w, out[i]);
  }
  const float rs = 1.0f / sqrtf((float)D);
#pragma unroll
  for (int i = 0; i < PER; ++i) dP[(int64_t)(j0 + jr + RPI * i) * D + b] = out[i] * rs;
}

template <typename T>
__device__ __forceinline__ float ld_any(const T* p, int64_t i);
template <>
__device__ __forceinline__ float ld_any<float>(const float* p, int64_t i) { return p[i]; }
template <>
__device__ __forceinline__ float ld_any<uint16_t>(const uint16_t* p, int64_t i) { return bf16f(p[i]); }

// part[c][a][b] = sum over rows i of chunk c of X[i][a] Y[i][b]
template <int D, typename TY>
__global__ __launch_bounds__(256) void bwd_outer(const float* __restrict__ X, const TY* __restrict__ Y, int64_t rows,
                                                 int chunk_rows, float* __restrict__ part) {
  constexpr int TA = D / 16;           // outputs per thread: TA x TA
  constexpr int RB = 32;               // rows staged per round
  constexpr int SL = RB * D / 256;     // staged elements per thread and operand
  __shared__ float xs[RB][D];
  __shared__ float ys[RB][D];
  const int tid = threadIdx.x;
  const int a0 = (tid >> 4) * TA, b0 = (tid & 15) * TA;
  const int64_t r0 = (int64_t)blockIdx.x * chunk_rows;
  const int64_t r1 = min(rows, r0 + chunk_rows);
  float acc[TA][TA];
#pragma unroll
  for (int i = 0; i < TA; ++i)
#pragma unroll
    for (int j = 0; j < TA; ++j) acc[i][j] = 0.f;
  for (int64_t rb = r0; rb < r1; rb += RB) {
    // every load of the round in flight before the LDS stores
    float xv_[SL], yv_[SL];
#pragma unroll
    for (int q = 0; q < SL; ++q) {
      const int e = tid + 256 * q, rr = e / D, cc = e % D;
      const int64_t row = rb + rr;
      const bool ok = row < r1;
      xv_[q] = ok ? X[row * D + cc] : 0.f;
      yv_[q] = ok ? ld_any<TY>(Y, row * D + cc) : 0.f;
    }
#pragma unroll
    for (int q = 0; q < SL; ++q) {
      const int e = tid + 256 * q, rr = e / D, cc = e % D;
      xs[rr][cc] = xv_[q];
      ys[rr][cc] = yv_[q];
    }
    __syncthreads();
    for (int rr = 0; rr < RB; ++rr) {
      float xv[TA], yv[TA];
#pragma unroll
      for (int i = 0; i < TA; ++i) {
        xv[i] = xs[rr][a0 + i];
        yv[i] = ys[rr][b0 + i];
      }
#pragma unroll
      for (int i = 0; i < TA; ++i)
#pragma unroll
        for (int j = 0; j < TA; ++j) acc[i][j] = fmaf(xv[i], yv[j], acc[i][j]);
    }
    __syncthreads();
  }
  float* dst = part + (int64_t)blockIdx.x * D * D;
#pragma unroll
  for (int i = 0; i < TA; ++i)
#pragma unroll
    for (int j = 0; j < TA; ++j) dst[(a0 + i) * D + b0 + j] = acc[i][j];
}

// out[e] = scale * sum_c part[c][e] (fixed order); n_chunks = 0 writes zeros
__global__ __launch_bounds__(256) void bwd_sum(const float* __restrict__ part, int n_chunks, int64_t n, float scale,
                                               float* __restrict__ out) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= n) return;
  // chunk order, with eight chunks' loads in flight at a time
  float s = 0.f;
  int c = 0;
  for (; c + 8 <= n_chunks; c += 8) {
    float v[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) v[q] = part[(int64_t)(c + q) * n + e];
#pragma unroll
    for (int q = 0; q < 8; ++q) s += v[q];
  }
  for (; c < n_chunks; ++c) s += part[(int64_t)c * n + e];
  out[e] = s * scale;
}

__global__ __launch_bounds__(256) void fill_zero(float* __restrict__ p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = 0.f;
}

// ---------------------------------------------------------------- launchers
template <typename T>
static T* hptr(void* ws, size_t off) {
  return reinterpret_cast<T*>(reinterpret_cast<char*>(ws) + off);
}

hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  const int64_t grid = std::min<int64_t>(1024, (n + 255) / 256);
  hipLaunchKernelGGL(fill_zero, dim3((unsigned)grid), dim3(256), 0, stream, p, n);
  return hipGetLastError();
}

hipError_t launch_bwd_user(const Layout& L, const void* Wv, const float* dS, const float* Sbar_in,
                           const float* mass_in, void* ws, hipStream_t stream) {
  const int64_t grid = (int64_t)L.R * (L.k / kRows);
  if (grid == 0) return hipSuccess;
  // the partial slots are reduced as the forward's finalize reduces them
  const int pre = (Sbar_in == nullptr && presum_launch(L)) ? 1 : 0;
  if (pre && launch_presum(L, ws, stream) != hipSuccess) return hipErrorLaunchFailure;
  if (L.d == 128) {
    hipLaunchKernelGGL((bwd_user<128>), dim3((unsigned)grid), dim3(256), 0, stream, (const uint16_t*)Wv, dS, Sbar_in,
                       mass_in, L, ws, pre);
    if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
    hipLaunchKernelGGL((bwd_zpack<128>), dim3((unsigned)grid), dim3(256), 0, stream, L, ws);
  } else {
    hipLaunchKernelGGL((bwd_user<64>), dim3((unsigned)grid), dim3(256), 0, stream, (const uint16_t*)Wv, dS, Sbar_in,
                       mass_in, L, ws, pre);
    if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
    hipLaunchKernelGGL((bwd_zpack<64>), dim3((unsigned)grid), dim3(256), 0, stream, L, ws);
  }
  return hipGetLastError();
}

hipError_t launch_bwd_dh(const Layout& L, const int64_t* offsets, void* ws, float* dH, hipStream_t stream) {
  if (L.N == 0) return hipSuccess;
  const int64_t grid = std::max<int64_t>(1, L.tiles_max / kUserTileAlign);
  const int32_t* tb = hptr<int32_t>(ws, L.off_tile_base);
  if (L.d == 128)
    hipLaunchKernelGGL((bwd_dh<128>), dim3((unsigned)grid), dim3(256), 0, stream, offsets, tb, L, ws, dH);
  else
    hipLaunchKernelGGL((bwd_dh<64>), dim3((unsigned)grid), dim3(256), 0, stream, offsets, tb, L, ws, dH);
  return hipGetLastError();
}

hipError_t launch_bwd_e(const Layout& L, void* ws, hipStream_t stream) {
  const int64_t grid = (int64_t)8 * L.e_pblocks * ((L.e_groups + 7) / 8);
  const int32_t* tb = hptr<int32_t>(ws, L.off_tile_base);
  const dim3 g((unsigned)grid);
  if (L.d == 128) {
    if (L.e_waves == 8)
      hipLaunchKernelGGL((bwd_e<128, 8>), g, dim3(512), 0, stream, tb, L, ws);
    else if (L.e_waves == 4)
      hipLaunchKernelGGL((bwd_e<128, 4>), g, dim3(256), 0, stream, tb, L, ws);
    else
      hipLaunchKernelGGL((bwd_e<128, 2>), g, dim3(128), 0, stream, tb, L, ws);
  } else {
    if (L.e_waves == 4)
      hipLaunchKernelGGL((bwd_e<64, 4>), g, dim3(256), 0, stream, tb, L, ws);
    else
      hipLaunchKernelGGL((bwd_e<64, 2>), g, dim3(128), 0, stream, tb, L, ws);
  }
  return hipGetLastError();
}

hipError_t launch_bwd_params(const Layout& L, const void* P, const void* Wk, const float* dS, void* ws, float* dP,
                             float* dWk, float* dWv, hipStream_t stream) {
  const int D = L.d;
  const int64_t dd = (int64_t)D * D;
  const dim3 gsum((unsigned)((dd + 255) / 256));
  float* et = hptr<float>(ws, L.off_betot);
  float* op = hptr<float>(ws, L.off_bopart);
  const float* sbar = hptr<float>(ws, L.off_bsbar);
  const int32_t* tb = hptr<const int32_t>(ws, L.off_tile_base);
  // E and dP
  if (D == 128)
    hipLaunchKernelGGL((bwd_ereduce<128>), dim3(L.k / kERows), dim3(256), 0, stream, (const uint16_t*)Wk, tb, L, ws,
                       dP);
  else
    hipLaunchKernelGGL((bwd_ereduce<64>), dim3(L.k / kERows), dim3(256), 0, stream, (const uint16_t*)Wk, tb, L, ws,
                       dP);
  if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  // dWk = E^T P / sqrt(d): k rows in as many chunks of a multiple of 32 rows
  // as the partial buffer holds (o_chunks >= k / 256)
  const int64_t per = (L.k + L.o_chunks - 1) / L.o_chunks;
  const int rk = (int)std::max<int64_t>(32, (per + 31) / 32 * 32);
  const int ck = (L.k + rk - 1) / rk;
  if (D == 128)
    hipLaunchKernelGGL((bwd_outer<128, uint16_t>), dim3(ck), dim3(256), 0, stream, (const float*)et,
                       (const uint16_t*)P, (int64_t)L.k, rk, op);
  else
    hipLaunchKernelGGL((bwd_outer<64, uint16_t>), dim3(ck), dim3(256), 0, stream, (const float*)et,
                       (const uint16_t*)P, (int64_t)L.k, rk, op);
  if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  hipLaunchKernelGGL(bwd_sum, gsum, dim3(256), 0, stream, (const float*)op, ck, dd, 1.0f / sqrtf((float)D), dWk);
  if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  // dWv = sum_u Sbar_u^T dS_u
  const int64_t rows = (int64_t)L.R * L.k;
  const int cv = (int)((rows + kOuterRows - 1) / kOuterRows);
  if (cv > 0) {
    if (D == 128)
      hipLaunchKernelGGL((bwd_outer<128, float>), dim3(cv), dim3(256), 0, stream, sbar, dS, rows, (int)kOuterRows,
                         op);
    else
      hipLaunchKernelGGL((bwd_outer<64, float>), dim3(cv), dim3(256), 0, stream, sbar, dS, rows, (int)kOuterRows, op);
    if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  }
  hipLaunchKernelGGL(bwd_sum, gsum, dim3(256), 0, stream, (const float*)op, cv, dd, 1.0f, dWv);
  return hipGetLastError();
}

}  // namespace sa
