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
// Per 32-token tile, each wave (32 prototypes) runs
//   GEMM1  C[t, j] = h_t . q_j - l_t with fp16 MFMAs: 8 K steps over d plus
//          one "feature" step in which the token supplies (-l_hi, -l_lo) and
//          the prototype (1, 1), l_t = lse_t - 14 split into two fp16 parts;
//   A'     = 2^C (= 2^14 A, inside fp16 range), converted pairwise to fp16;
//          mass += A' pairs (v_dot2 on the rounded values);
//   GEMM2  U[j, c] += sum_t A'[j,t] h_t[c]                           (fp16 MFMA)
// The accumulator of GEMM1 holds prototype (lane % 32) and 16 tokens per lane;
// those registers are exactly the A operand of GEMM2 because the transposed
// tile stores tokens in the accumulator's row order (pass 1 writes it so), so
// no data moves between lanes.  The 2^14 scale cancels in U / m.
//
// Data movement: tiles reach LDS with direct global->LDS loads (16 B per
// lane), 4 tiles (128 tokens) per stage, two stages in flight.  LDS rows are
// XOR-swizzled by 16-byte chunk so each group of 16 lanes of a ds_read_b128
// hits 16 different 16-byte bank slots (gfx950 LDS: 64 banks of 4 bytes).
// Every user's tile count is a multiple of 4 (pass 1 fills the padding tiles
// with zero rows and A = 0), so every stage is full and the stage body is one
// straight-line block.  A workgroup has up to 8 waves of 32 prototypes (two
// waves per SIMD, every MFMA operand and result in VGPRs), so one wave's
// exponentials and LDS reads run while the other wave's MFMAs execute.  LDS
// read traffic is about 1 KB per MFMA, close to what the LDS sustains; the
// feature step keeps the per-token -l down to 4 bytes per lane.
//
// Work item = (chunk of <= tiles_per_chunk tiles of one user, prototype block
// of waves*32).  Workgroups are numbered so that the prototype blocks of one
// chunk land on the same XCD back to back (dispatch goes round-robin over the
// 8 XCDs), letting them share the chunk's tiles through that XCD's L2.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sa_device.h"
#include "sa_launch.h"

namespace sa {

namespace {

constexpr int kStageTiles = 4;

template <int D>
struct P2 {
  static constexpr int S = D / 16;                   // MFMA K steps over d
  static constexpr int DT = D / 32;                  // 32-column output blocks
  static constexpr int CPR = D / 8;                  // 16-B chunks per token row
  static constexpr int ROWSH = (CPR == 16) ? 0 : 1;  // rows sharing a 256-B bank line: 2^ROWSH
  static constexpr int TILE_BYTES = kTile * D * 2;   // one tile, rows or transposed
  static constexpr int ROWS_BYTES = kStageTiles * TILE_BYTES;
  static constexpr int NL_OFF = 2 * ROWS_BYTES;      // (-l_hi, -l_lo) pairs of the stage
  static constexpr int STAGE_BYTES = NL_OFF + kStageTiles * kTile * 4;
  static constexpr int LOADS_ROWS = ROWS_BYTES / 1024;   // 1-KB direct loads per stage, rows
  static constexpr int LOADS_TR = ROWS_BYTES / 1024;     // and transposed tiles
};

// chunk swizzle of a token row (row index within the stage) and of a
// transposed-tile row (feature column)
template <int D>
__device__ __forceinline__ int swz_row(int tok) {
  return (tok >> P2<D>::ROWSH) & (P2<D>::CPR - 1);
}
__device__ __forceinline__ int swz_tr(int dcol) { return (dcol >> 2) & 3; }

typedef __attribute__((address_space(3))) void* lds_ptr_t;

}  // namespace

template <int D, int WAVES>
__global__ __launch_bounds__(WAVES * 64) void pass2_accum(Layout L, void* ws) {
  using C = P2<D>;
  __shared__ __attribute__((aligned(1024))) char lds[2 * C::STAGE_BYTES];

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

  // B operands of GEMM1: the wave's 32 query rows (kept in registers), and the
  // feature step's (1, 1, 0, ...) column pair
  const _Float16* q16 = ws_f16(ws, L.off_q16);
  half8 qf[C::S];
#pragma unroll
  for (int s = 0; s < C::S; ++s)
    qf[s] = *reinterpret_cast<const half8*>(q16 + (int64_t)(p0 + col) * D + 16 * s + 8 * g);
  const half8 qfeat = {(_Float16)1.0f, (_Float16)1.0f, (_Float16)0.0f, (_Float16)0.0f,
                       (_Float16)0.0f, (_Float16)0.0f, (_Float16)0.0f, (_Float16)0.0f};

  const char* h16 = reinterpret_cast<const char*>(ws_f16(ws, L.off_h16));
  const char* h16t = reinterpret_cast<const char*>(ws_f16(ws, L.off_h16t));
  const char* nlg = reinterpret_cast<const char*>(ws_i32(ws, L.off_nl));

  // Direct loads of stage `ts` (tiles 4 ts .. 4 ts + 3 of the chunk) into
  // buffer b.  Load i of the rows part fills LDS bytes [1024 i, 1024 i + 1024)
  // of the stage: lane l writes chunk slot 64 i + l = (token, swizzled chunk).
  auto issue = [&](int ts, int b) {
    char* base = lds + b * C::STAGE_BYTES;
    const int64_t tile0 = (int64_t)t0 + (int64_t)ts * kStageTiles;
#pragma unroll
    for (int i = wave; i < C::LOADS_ROWS; i += WAVES) {
      const int q = 64 * i + lane;
      const int tok = q / C::CPR, cs = q % C::CPR;
      const int c = cs ^ swz_row<D>(tok);
      const char* src = h16 + (tile0 * kTile + tok) * (D * 2) + c * 16;
      __builtin_amdgcn_global_load_lds(src, (lds_ptr_t)(base + 1024 * i), 16, 0, 0);
    }
#pragma unroll
    for (int i = wave; i < C::LOADS_TR; i += WAVES) {
      const int q = 64 * i + lane;
      const int tt = q / (C::TILE_BYTES / 16), qq = q % (C::TILE_BYTES / 16);
      const int dcol = qq >> 2, c = (qq & 3) ^ swz_tr(dcol);
      const char* src = h16t + (tile0 + tt) * C::TILE_BYTES + dcol * 64 + c * 16;
      __builtin_amdgcn_global_load_lds(src, (lds_ptr_t)(base + C::ROWS_BYTES + 1024 * i), 16, 0, 0);
    }
    if (wave == WAVES - 1 && lane < 8 * kStageTiles) {
      const char* src = nlg + tile0 * (kTile * 4) + lane * 16;
      __builtin_amdgcn_global_load_lds(src, (lds_ptr_t)(base + C::NL_OFF), 16, 0, 0);
    }
  };

  float16v U[C::DT];
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt) U[dt] = float16v{};
  float msum = 0.f;
  const half2v ones = {(_Float16)1.0f, (_Float16)1.0f};

  const int nstages = nt / kStageTiles;
  issue(0, 0);
  for (int st = 0; st < nstages; ++st) {
    const int b = st & 1;
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's loads of stage st landed
    __syncthreads();                     // ... every wave's; and stage st-1's buffer is free
    if (st + 1 < nstages) issue(st + 1, b ^ 1);
    const char* base = lds + b * C::STAGE_BYTES;
#pragma unroll
    for (int t = 0; t < kStageTiles; ++t) {
      const char* rows = base + t * C::TILE_BYTES;
      const char* tr = base + C::ROWS_BYTES + t * C::TILE_BYTES;
      // GEMM1: C[tok, proto] = h_tok . q_proto - l_tok
      const uint32_t nlp = reinterpret_cast<const uint32_t*>(base + C::NL_OFF)[t * kTile + col];
      const u32x4 fv = {g == 0 ? nlp : 0u, 0u, 0u, 0u};
      float16v Cm = mfma32x32x16(__builtin_bit_cast(half8, fv), qfeat, float16v{});
      const int tok = t * kTile + col;   // row within the stage
#pragma unroll
      for (int s = 0; s < C::S; ++s) {
        const int c = (2 * s + g) ^ swz_row<D>(tok);
        const half8 ha = *reinterpret_cast<const half8*>(rows + col * (D * 2) + c * 16);
        Cm = mfma32x32x16(ha, qf[s], Cm);
      }
      // allocations 2^C (= 2^14 A) in fp16, masses of the rounded values
      half8 ap[2];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          float2v v = {__builtin_amdgcn_exp2f(Cm[8 * kk + e]), __builtin_amdgcn_exp2f(Cm[8 * kk + e + 1])};
          half2v h = __builtin_convertvector(v, half2v);
          msum = __builtin_amdgcn_fdot2(h, ones, msum, false);
          ap[kk][e] = h[0];
          ap[kk][e + 1] = h[1];
        }
      // GEMM2: U[proto, c] += sum_tok A'[proto, tok] h_tok[c]
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt) {
          const int dcol = 32 * dt + col;
          const int c = (2 * kk + g) ^ swz_tr(dcol);
          const half8 hb = *reinterpret_cast<const half8*>(tr + dcol * 64 + c * 16);
          U[dt] = mfma32x32x16(ap[kk], hb, U[dt]);
        }
    }
  }

  float* part_u = ws_f32(ws, L.off_part_u) + (int64_t)chunk * L.k * D;
  float* part_m = ws_f32(ws, L.off_part_m) + (int64_t)chunk * L.k;
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r)
      part_u[(int64_t)(p0 + acc_row(r, g)) * D + 32 * dt + col] = U[dt][r];
  const float m = msum + __shfl_xor(msum, 32);
  if (g == 0) part_m[p0 + col] = m;
}

hipError_t launch_pass2(const Layout& L, void* ws, hipStream_t stream) {
  const int64_t padded = ((int64_t)L.chunks_max + 7) / 8 * 8;
  const int64_t grid = padded * L.n_pblocks;
  if (grid == 0) return hipSuccess;
#define SA_P2(DD, WW) \
  hipLaunchKernelGGL((pass2_accum<DD, WW>), dim3((unsigned)grid), dim3(WW * 64), 0, stream, L, ws)
  if (L.d == 128) {
    switch (L.waves) {
      case 8: SA_P2(128, 8); break;
      case 4: SA_P2(128, 4); break;
      default: SA_P2(128, 2); break;
    }
  } else {
    switch (L.waves) {
      case 8: SA_P2(64, 8); break;
      case 4: SA_P2(64, 4); break;
      default: SA_P2(64, 2); break;
    }
  }
#undef SA_P2
  return hipGetLastError();
}

}  // namespace sa
