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
// those registers are exactly the A operand of GEMM2, so no data moves
// between lanes.  GEMM2's B operand (lane = feature column, 8 tokens in the
// accumulator's row order) comes from the same token rows in LDS through the
// gfx950 transposing read ds_read_b64_tr_b16: within each group of 16 lanes,
// destination lane i receives element i % 4 of the 4-element vectors that
// source lanes i/4, i/4 + 4, i/4 + 8, i/4 + 12 address, so source lane s
// addresses token (s / 4) of the group's 4 tokens at columns 4 (s % 4) ...
// The 2^14 scale cancels in U / m.
//
// Data movement: token rows reach LDS with direct global->LDS loads (16 B per
// lane), 4 tiles (128 tokens) per stage, four stage buffers (loads run three
// stages ahead: the loads are latency-bound, so the bytes in flight per CU
// set their rate).  A row occupies 2d + 16 bytes (one 16-byte chunk of
// padding, filled by the same loads); GEMM1's operand row m holds token
// tau(m), which puts the 4 tokens of one transposing read 4 rows apart.  Then
// the 16-byte GEMM1 reads and the transposing 8-byte reads both touch 64
// distinct banks per pass (gfx950 LDS: 64 banks of 4 bytes), and every read
// is one per-lane base register plus an immediate.
// Every user's tile count is a multiple of 4 (pass 1 fills the padding tiles
// with zero rows and A = 0), so every stage is full and the stage body is one
// straight-line block.  A workgroup has up to 8 waves of 32 prototypes (two
// waves per SIMD, every MFMA operand and result in VGPRs), so one wave's
// exponentials and LDS reads run while the other wave's MFMAs execute.  LDS
// read traffic is about 1 KB per MFMA; the feature step keeps the per-token -l
// down to 4 bytes per lane.
//
// Work item = (chunk of <= tiles_per_chunk tiles of one user, prototype block
// of waves*32).  Workgroups are numbered so that the prototype blocks of one
// chunk land on the same XCD back to back (dispatch goes round-robin over the
// 8 XCDs), letting them share the chunk's tiles through that XCD's L2.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "sa_device.h"
#include "sa_launch.h"

namespace sa {

namespace {

constexpr int kStageTiles = 4;
constexpr int kBufs = 4;           // stage buffers: loads run three stages ahead

template <int D>
struct P2 {
  static constexpr int S = D / 16;                   // MFMA K steps over d
  static constexpr int DT = D / 32;                  // 32-column output blocks
  static constexpr int CPR = D / 8;                  // 16-B chunks per token row
  static constexpr int SLOTS = CPR + 1;              // ... plus one chunk of padding
  static constexpr int PITCH = SLOTS * 16;           // LDS bytes per token row
  static constexpr int TILE_BYTES = kTile * PITCH;   // one tile of token rows
  static constexpr int ROWS_BYTES = kStageTiles * TILE_BYTES;
  static constexpr int NL_OFF = ROWS_BYTES;          // (-l_hi, -l_lo) pairs of the stage
  static constexpr int STAGE_BYTES = NL_OFF + kStageTiles * kTile * 4;
  static constexpr int LOADS_ROWS = kStageTiles * kTile * SLOTS / 64;   // 1-KB direct loads per stage
  static_assert(LOADS_ROWS * 64 == kStageTiles * kTile * SLOTS, "whole loads per stage");
};

// Token held by GEMM1 operand row m (m = 16 kk + 8 h + 4 g + e in bits):
// 16 kk + 4 e + 2 g + h.  GEMM1's accumulator rows are GEMM2's K order, so
// the 4 tokens of one transposing read (e = 0..3) lie 4 rows apart; with the
// padded row pitch (2d + 16 bytes) such a read (32 lanes: 4 tokens x 64
// bytes) meets all 64 banks once, and so do the 16-byte GEMM1 reads (16
// consecutive operand rows, one chunk).
__device__ __forceinline__ int tau(int m) {
  return (m & 16) | ((m & 3) << 2) | (((m >> 2) & 1) << 1) | ((m >> 3) & 1);
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// s_waitcnt immediate that waits until at most n vector-memory operations of
// this wave are outstanding (gfx9 encoding: vmcnt in bits 3:0 and 15:14,
// expcnt and lgkmcnt left at their no-wait maxima)
constexpr int waitcnt_vm(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }

}  // namespace

template <int D, int WAVES, int NB>
__global__ __launch_bounds__(WAVES * 64) void pass2_accum(Layout L, void* ws) {
  using C = P2<D>;
  __shared__ __attribute__((aligned(1024))) char lds[kBufs * C::STAGE_BYTES];

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
  // the wave owns NB blocks of 32 prototypes: p0 + 32 b + (0 .. 31)
  const int p0 = pb * (WAVES * NB * kProtoPerWave) + wave * (NB * kProtoPerWave);

  // B operands of GEMM1: the wave's query rows (kept in registers), and the
  // feature step's (1, 1, 0, ...) column pair
  const _Float16* q16 = ws_f16(ws, L.off_q16);
  half8 qf[NB][C::S];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int s = 0; s < C::S; ++s)
      qf[b][s] = *reinterpret_cast<const half8*>(q16 + (int64_t)(p0 + 32 * b + col) * D + 16 * s + 8 * g);
  const half8 qfeat = {(_Float16)1.0f, (_Float16)1.0f, (_Float16)0.0f, (_Float16)0.0f,
                       (_Float16)0.0f, (_Float16)0.0f, (_Float16)0.0f, (_Float16)0.0f};

  const char* h16 = reinterpret_cast<const char*>(ws_f16(ws, L.off_h16));
  const char* nlg = reinterpret_cast<const char*>(ws_i32(ws, L.off_nl));

  // Direct loads of stage `ts` (tiles 4 ts .. 4 ts + 3 of the chunk) into
  // buffer b.  Load i fills LDS bytes [1024 i, 1024 i + 1024) of the stage:
  // lane l writes 16-byte slot 64 i + l = (row q / SLOTS, chunk q % SLOTS);
  // the padding chunk re-reads chunk 0 of its row.  Row loads go round-robin
  // over the waves, and every wave adds one slice of the -l pairs; a wave's
  // vmcnt waits count its own loads (LMAX or LMIN per stage).
  constexpr int LMAX = (C::LOADS_ROWS + WAVES - 1) / WAVES + 1;
  constexpr int LMIN = C::LOADS_ROWS / WAVES + 1;
  static_assert(2 * LMAX < 64, "vmcnt range");
  const bool big = (C::LOADS_ROWS % WAVES == 0) || (wave < C::LOADS_ROWS % WAVES);
  auto issue = [&](int ts, int b) {
    char* base = lds + b * C::STAGE_BYTES;
    const int64_t tile0 = (int64_t)t0 + (int64_t)ts * kStageTiles;
#pragma unroll 1
    for (int i = wave; i < C::LOADS_ROWS; i += WAVES) {
      const int q = 64 * i + lane;
      const int row = q / C::SLOTS;
      int c = q - row * C::SLOTS;
      c = c == C::CPR ? 0 : c;
      const char* src = h16 + (tile0 * kTile + row) * (D * 2) + c * 16;
      __builtin_amdgcn_global_load_lds(src, (lds_ptr_t)(base + 1024 * i), 16, 0, 0);
    }
    constexpr int NL_LANES = kStageTiles * kTile * 4 / 16 / WAVES;   // 16-B pieces per wave
    if (lane < NL_LANES) {
      const char* src = nlg + tile0 * (kTile * 4) + (wave * NL_LANES + lane) * 16;
      __builtin_amdgcn_global_load_lds(src, (lds_ptr_t)(base + C::NL_OFF + wave * NL_LANES * 16), 16, 0, 0);
    }
  };
  // wait until only this wave's loads of the `later` stages after the
  // current one are still in flight
  auto wait_stage = [&](int later) {
    if (later >= 2) {
      if (big) __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * LMAX));
      else __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * LMIN));
    } else if (later == 1) {
      if (big) __builtin_amdgcn_s_waitcnt(waitcnt_vm(LMAX));
      else __builtin_amdgcn_s_waitcnt(waitcnt_vm(LMIN));
    } else {
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    }
  };
  static_assert(kBufs == 4, "the stage loop below is unrolled over 4 buffers");

  // per-lane byte offsets of the transposing reads (GEMM2 B operands):
  // source lane i16 of 16-lane group gh reads the row of token 4 (i16 / 4) +
  // 2 g (+ 16 kk + h) at columns 16 gh + 4 (i16 % 4) (+ 32 dt) .. + 3, which
  // is K element 4 h + i16 / 4 of lane half g in GEMM1's row order (tau)
  const int i16 = lane & 15, gh = (lane >> 4) & 1;
  const int tr_base = (4 * (i16 >> 2) + 2 * g) * C::PITCH + 32 * gh + 8 * (i16 & 3);

  float16v U[NB][C::DT];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) U[b][dt] = float16v{};
  float msum[NB] = {};
  const half2v ones = {(_Float16)1.0f, (_Float16)1.0f};

  // per-lane byte offset of the GEMM1 operand reads: row of token tau(col),
  // chunk 2 s + g at + 32 s
  const int tcol = tau(col);
  const int ha_base = tcol * C::PITCH + 16 * g;

  // One stage held in buffer B (a compile-time constant, so every LDS read is
  // a per-lane offset register plus an immediate).
  const int nstages = nt / kStageTiles;
  auto stage = [&](int st, auto Bc) {
    constexpr int B = decltype(Bc)::value;
    // this wave's loads of stage st have landed (those of st+1, st+2 may still fly)
    wait_stage(min(2, nstages - 1 - st));
    __syncthreads();                             // ... every wave's; stage st-1's buffer is free
    if (st + 3 < nstages) issue(st + 3, (B + 3) % kBufs);
    const char* base = lds + B * C::STAGE_BYTES;
    typedef __attribute__((address_space(3))) s16x4* tr_ptr;
    // GEMM1 of tile t: C[tok, proto] = h_tok . q_proto - l_tok
    auto gemm1 = [&](int t, float16v (&Cm)[NB]) {
      const char* rows = base + t * C::TILE_BYTES;
      const uint32_t nlp = reinterpret_cast<const uint32_t*>(base + C::NL_OFF)[t * kTile + tcol];
      half8 ha[C::S];
#pragma unroll
      for (int s = 0; s < C::S; ++s) ha[s] = *reinterpret_cast<const half8*>(rows + ha_base + 32 * s);
      const u32x4 fv = {g == 0 ? nlp : 0u, 0u, 0u, 0u};
#pragma unroll
      for (int b = 0; b < NB; ++b) Cm[b] = mfma32x32x16(__builtin_bit_cast(half8, fv), qfeat, float16v{});
#pragma unroll
      for (int s = 0; s < C::S; ++s)
#pragma unroll
        for (int b = 0; b < NB; ++b) Cm[b] = mfma32x32x16(ha[s], qf[b][s], Cm[b]);
    };
    // allocations 2^C (= 2^14 A) in fp16, masses of the rounded values
    auto expo = [&](const float16v (&Cm)[NB], half8 (&ap)[NB][2]) {
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
          for (int e = 0; e < 8; e += 2) {
            float2v v = {__builtin_amdgcn_exp2f(Cm[b][8 * kk + e]), __builtin_amdgcn_exp2f(Cm[b][8 * kk + e + 1])};
            half2v h = __builtin_convertvector(v, half2v);
            msum[b] = __builtin_amdgcn_fdot2(h, ones, msum[b], false);
            ap[b][kk][e] = h[0];
            ap[b][kk][e + 1] = h[1];
          }
    };
    // GEMM2 of tile t: U[proto, c] += sum_tok A'[proto, tok] h_tok[c]
    auto gemm2 = [&](int t, const half8 (&ap)[NB][2]) {
      const char* rows = base + t * C::TILE_BYTES + tr_base;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt) {
          const char* pr0 = rows + 16 * kk * C::PITCH + 64 * dt;
          const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((tr_ptr)(pr0));
          const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((tr_ptr)(pr0 + C::PITCH));
          const s16x8 hb = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
          for (int b = 0; b < NB; ++b) U[b][dt] = mfma32x32x16(ap[b][kk], __builtin_bit_cast(half8, hb), U[b][dt]);
        }
    };
    // Pipeline within the stage: GEMM1 of tile t+1 is issued interleaved
    // with the exponentials of tile t (independent work), then GEMM2 of t.
    float16v Ca[NB], Cb[NB];
    half8 ap[NB][2];
    __builtin_amdgcn_sched_barrier(0);
    gemm1(0, Ca);
#pragma unroll
    for (int t = 0; t < kStageTiles; ++t) {
      float16v (&Cx)[NB] = (t & 1) ? Cb : Ca;
      float16v (&Cy)[NB] = (t & 1) ? Ca : Cb;
      __builtin_amdgcn_sched_barrier(0);
      if (t + 1 < kStageTiles) {
        gemm1(t + 1, Cy);
        expo(Cx, ap);
        __builtin_amdgcn_sched_group_barrier(0x100, C::S + 1, 0);   // GEMM1 LDS reads
#pragma unroll
        for (int i = 0; i < NB * (C::S + 1); ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);        // 1 MFMA
          __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);        // 4 VALU
        }
      } else {
        expo(Cx, ap);
      }
      __builtin_amdgcn_sched_barrier(0);
      gemm2(t, ap);
    }
  };
  issue(0, 0);
  if (nstages > 1) issue(1, 1);
  if (nstages > 2) issue(2, 2);
  for (int st = 0; st < nstages; st += kBufs) {
    stage(st, std::integral_constant<int, 0>{});
    if (st + 1 < nstages) stage(st + 1, std::integral_constant<int, 1>{});
    if (st + 2 < nstages) stage(st + 2, std::integral_constant<int, 2>{});
    if (st + 3 < nstages) stage(st + 3, std::integral_constant<int, 3>{});
  }

  float* part_u = ws_f32(ws, L.off_part_u) + (int64_t)chunk * L.k * D;
  float* part_m = ws_f32(ws, L.off_part_m) + (int64_t)chunk * L.k;
#pragma unroll
  for (int b = 0; b < NB; ++b) {
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        part_u[(int64_t)(p0 + 32 * b + acc_row(r, g)) * D + 32 * dt + col] = U[b][dt][r];
    const float m = msum[b] + __shfl_xor(msum[b], 32);
    if (g == 0) part_m[p0 + 32 * b + col] = m;
  }
}

hipError_t launch_pass2(const Layout& L, void* ws, hipStream_t stream) {
  const int64_t padded = ((int64_t)L.chunks_max + 7) / 8 * 8;
  const int64_t grid = padded * L.n_pblocks;
  if (grid == 0) return hipSuccess;
#define SA_P2(DD, WW) \
  hipLaunchKernelGGL((pass2_accum<DD, WW, 1>), dim3((unsigned)grid), dim3(WW * 64), 0, stream, L, ws)
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
