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
// lane), 4 tiles (128 tokens) per stage, four stage buffers, loads two stages
// ahead; the -l pairs arrive as a 16-byte piece per token (its pair first), so
// the feature step's operand is one LDS read.  A row occupies 2d + 16 bytes (the last 16 are never read and never
// loaded); GEMM1's operand row m holds token tau(m), which puts the 4 tokens
// of one transposing read 4 rows apart.  Then the 16-byte GEMM1 reads and the
// transposing 8-byte reads both touch 64 distinct banks per pass (gfx950
// LDS: 64 banks of 4 bytes), and every read is one per-lane base register
// plus an immediate.  Every user's tile count is a multiple of 4 (pass 1
// fills the padding tiles with zero rows and A = 0), so every stage is full.
// A workgroup has up to 8 waves of 32 prototypes (two waves per SIMD, every
// MFMA operand and result in VGPRs).  The feature step keeps the per-token -l
// down to 4 bytes per lane.
//
// Measured on MI355X, random fp16 operands hold the matrix cores near 1.7
// PFLOP/s (power-limited clock) rather than the 2.5 nominal, and any other
// work shares that power: moving fewer bytes counts more than issuing fewer
// instructions.  Hence one copy of the rows (transposing reads for GEMM2)
// rather than a second, transposed copy.
//
// Work split: a persistent grid of about 256 workgroups (one per CU), in
// groups of P = k / (waves*32) workgroups, one per prototype block.  Group g
// walks an equal contiguous range of the batch's tiles, cut at user
// boundaries into segments whose sums go to partial slot g + user; every
// workgroup does the same work, so no partially filled last round of
// workgroups idles the chip, and the partial sums are (groups + users) x k x d
// rather than one per chunk.  The P workgroups of a group sit on one XCD
// (dispatch goes round-robin over the 8 XCDs) and share the tiles through
// its L2.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "sa_device.h"
#include "sa_launch.h"

namespace sa {

namespace {

constexpr int kStageTiles = 4;
constexpr int kBufs = 4;           // stage buffers: loads run two stages ahead

template <int D>
struct P2 {
  static constexpr int S = D / 16;                   // MFMA K steps over d
  static constexpr int DT = D / 32;                  // 32-column output blocks
  static constexpr int CPR = D / 8;                  // 16-B chunks per token row
  static constexpr int SLOTS = CPR + 1;              // ... plus one chunk of padding
  static constexpr int PITCH = tile_pitch<D>();      // LDS bytes per token row
  static_assert(PITCH == SLOTS * 16, "padded row");
  static constexpr int TILE_BYTES = kTile * PITCH;   // one tile of token rows
  // a 16-byte piece per token of the stage: its (-l_hi, -l_lo) pair, then the
  // next three tokens' pairs (multiplied by zeros in the feature step)
  static constexpr int NL_OFF = kStageTiles * TILE_BYTES;
  static constexpr int STAGE_BYTES = NL_OFF + kStageTiles * kTile * 16;
  static constexpr int LOADS = kStageTiles * kTile * SLOTS / 64;   // 1-KB direct loads per stage
  static_assert(LOADS * 64 == kStageTiles * kTile * SLOTS, "whole loads per stage");
  static_assert(STAGE_BYTES % 256 == 0, "load alignment");
};

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

  // Workgroup x sits on XCD x % 8 (dispatch is round-robin over the XCDs);
  // the P workgroups of a group (one per prototype block) are consecutive
  // slots x / 8 of one XCD, so they share the group's tiles through its L2.
  // Group g walks tiles [g Tg, (g + 1) Tg), Tg = the total over the G
  // groups rounded up to a multiple of 4: every workgroup does the same
  // amount of work.
  const int32_t* hdr = ws_i32(ws, L.off_hdr);
  const int P = L.n_pblocks, G = L.p2_groups;
  const int x = blockIdx.x, xcd = x & 7, slotw = x >> 3;
  const int group = xcd + 8 * (slotw / P);
  const int pb = slotw % P;
  if (group >= G) return;  // uniform over the workgroup
  const int32_t T = hdr[kHdrTiles];
  const int32_t Tg = (T + 4 * G - 1) / (4 * G) * 4;
  const int32_t s0 = group * Tg, s1 = min(T, s0 + Tg);
  if (s0 >= s1) return;
  const int32_t* tile_base = ws_i32(ws, L.off_tile_base);
  int32_t t0 = 0;   // the current segment: tiles t0 .. t0 + nt - 1 of one user
  int nt = 0;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar branches on it
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
  // (1, 1) at the pair's K positions of the lower lane half, zeros elsewhere
  // (the upper half's K positions meet the same piece again)
  const _Float16 one = g == 0 ? (_Float16)1.0f : (_Float16)0.0f;
  const half8 qfeat = {one, one, (_Float16)0.0f, (_Float16)0.0f, (_Float16)0.0f, (_Float16)0.0f, (_Float16)0.0f,
                       (_Float16)0.0f};

  const char* h16 = reinterpret_cast<const char*>(ws_f16(ws, L.off_h16));
  const char* nlg = reinterpret_cast<const char*>(ws_i32(ws, L.off_nl));

  // Direct loads of stage `ts` (tiles 4 ts .. 4 ts + 3 of the chunk) into
  // buffer b.  Load i fills LDS bytes [1024 i, 1024 i + 1024) of the stage:
  // lane l writes 16-byte slot 64 i + l = (row q / SLOTS, chunk q % SLOTS),
  // except the padding chunk, which no lane loads.  Loads go round-robin over
  // the waves (load i to wave i % WAVES), and every wave adds one slice of
  // the -l pairs; a wave's vmcnt waits count its own loads (LMAX or LMIN per
  // stage).  A lane's source offsets inside the stage's tiles are the same
  // for every stage, so they are computed once (~0 marks a padding slot).
  constexpr int KMAX = (C::LOADS + WAVES - 1) / WAVES;
  // -l pieces: 4-byte direct loads of 16 tokens' pieces each, NLL per wave
  constexpr int NLL = kStageTiles * kTile * 4 / 64 / WAVES;
  static_assert(NLL * 64 * WAVES == kStageTiles * kTile * 4, "whole -l loads");
  constexpr int LMAX = KMAX + NLL;
  constexpr int LMIN = C::LOADS / WAVES + NLL;
  const bool big = (C::LOADS % WAVES == 0) || (wave < C::LOADS % WAVES);
  uint32_t src_off[KMAX];
#pragma unroll
  for (int kq = 0; kq < KMAX; ++kq) {
    const int q = 64 * (wave + kq * WAVES) + lane;
    const int row = q / C::SLOTS;
    const int c = q - row * C::SLOTS;
    src_off[kq] = c == C::CPR ? ~0u : (uint32_t)(row * (D * 2) + c * 16);
  }
  auto issue = [&](int ts, int b) {
    char* base = lds + b * C::STAGE_BYTES;
    const int64_t tile0 = (int64_t)t0 + (int64_t)ts * kStageTiles;
    const char* rows_src = h16 + tile0 * (kTile * D * 2);
#pragma unroll
    for (int kq = 0; kq < KMAX; ++kq) {
      const int i = wave + kq * WAVES;
      if (i < C::LOADS && src_off[kq] != ~0u) {   // i uniform; the padding slot per lane
        // (a named pointer: given the sum directly, the host compilation pass
        // silently drops this kernel's instantiation)
        const char* src = rows_src + src_off[kq];
        __builtin_amdgcn_global_load_lds(src, (lds_ptr_t)(base + 1024 * i), 16, 0, 0);
      }
    }
    // the -l pieces: 4-byte direct loads; lane l of load i fills word l % 4
    // of token 16 i' + l / 4's piece (i' = NLL wave + i) with the pair of
    // token 16 i' + l / 4 + l % 4 (past the batch's last tile the pairs are
    // zeros the preparation wrote)
#pragma unroll
    for (int i = 0; i < NLL; ++i) {
      const int tk = 16 * (NLL * wave + i);
      const char* src = nlg + (tile0 * kTile + tk + (lane >> 2) + (lane & 3)) * 4;
      __builtin_amdgcn_global_load_lds(src, (lds_ptr_t)(base + C::NL_OFF + tk * 16), 4, 0, 0);
    }
  };
  // wait until only this wave's loads of the `later` stages after the
  // current one are still in flight (later <= kBufs - 2)
  auto wait_stage = [&](int later) {
    if constexpr (kBufs > 3) {
      if (later >= 2) {
        if (big) __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * LMAX));
        else __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * LMIN));
        return;
      }
    }
    if constexpr (kBufs > 2) {
      if (later == 1) {
        if (big) __builtin_amdgcn_s_waitcnt(waitcnt_vm(LMAX));
        else __builtin_amdgcn_s_waitcnt(waitcnt_vm(LMIN));
        return;
      }
    }
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  };
  static_assert(kBufs >= 3 && kBufs <= 4, "loads one or two stages ahead");
  static_assert((kBufs - 1) * LMAX < 64, "vmcnt range");

  // per-lane byte offset of the transposing reads (GEMM2 B operands):
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

  // Per-tile software pipeline; period t (one tile) of a wave:
  //   1. if tile t+1 opens stage s: wait for this wave's loads of stage s,
  //      barrier, issue the loads of stage s + kAhead;
  //   2. LDS reads of GEMM1's operands for tile t+1 (and its -l pair);
  //   3. GEMM2 of tile t-1 (its operands in registers since period t-1),
  //      interleaved with the exponentials of tile t (whose GEMM1 ran in
  //      period t-1): these MFMAs cover step 2's latency and the VALU work;
  //   4. LDS reads of GEMM2's operands for tile t;
  //   5. GEMM1 of tile t+1, covering step 4's latency.
  // Loads run kAhead = kBufs - 2 stages ahead, so the buffer of the stage
  // before the current one still holds tile t when step 4 reads it.
  constexpr int kAhead = kBufs - 2;
  static_assert(kAhead >= 1, "at least one stage of loads in flight");
  int nstages = 0;
  auto tile_lds = [&](int t) { return lds + ((t / kStageTiles) % kBufs) * C::STAGE_BYTES; };
  auto boundary = [&](int t1) {   // before the first read of tile t1
    if (t1 % kStageTiles == 0) {  // uniform
      const int st = t1 / kStageTiles;
      wait_stage(min(kAhead - 1, nstages - 1 - st));
      lds_barrier();              // stage st in LDS; every read of stage st - 2 is done
      if (st + kAhead < nstages) issue(st + kAhead, (st + kAhead) % kBufs);
    }
  };
  // GEMM1 operands of tile t: row of token tau(col), chunk 2 s + g; -l pair
  auto read_a = [&](int t, half8 (&ha)[C::S], half8& nlp) {
    const char* base = tile_lds(t);
    const char* rows = base + (t % kStageTiles) * C::TILE_BYTES + ha_base;
#pragma unroll
    for (int s = 0; s < C::S; ++s) ha[s] = *reinterpret_cast<const half8*>(rows + 32 * s);
    nlp = *reinterpret_cast<const half8*>(base + C::NL_OFF + ((t % kStageTiles) * kTile + tcol) * 16);
  };
  // GEMM1: C[tok, proto] = h_tok . q_proto - l_tok (the feature step adds
  // -l), split after its first K step
  auto gemm1_head = [&](const half8 (&ha)[C::S], const half8& nlp, float16v (&Cm)[NB]) {
#pragma unroll
    for (int b = 0; b < NB; ++b) Cm[b] = mfma32x32x16(nlp, qfeat, float16v{});
#pragma unroll
    for (int b = 0; b < NB; ++b) Cm[b] = mfma32x32x16(ha[0], qf[b][0], Cm[b]);
  };
  auto gemm1_tail = [&](const half8 (&ha)[C::S], float16v (&Cm)[NB]) {
#pragma unroll
    for (int s = 1; s < C::S; ++s)
#pragma unroll
      for (int b = 0; b < NB; ++b) Cm[b] = mfma32x32x16(ha[s], qf[b][s], Cm[b]);
  };
  // GEMM2 operands of tile t (transposing reads, waited for inside)
  auto read_b = [&](int t, half8 (&hb)[2][C::DT]) {
    tile_tr_reads<D>(lds_addr(tile_lds(t) + (t % kStageTiles) * C::TILE_BYTES) + tr_base, hb);
  };
  // allocations 2^C (= 2^14 A) in fp16 for accumulator elements 2 i, 2 i + 1
  // (i = 0..7)
  auto expo2 = [&](const float16v (&Cm)[NB], half8 (&ap)[NB][2], int i) {
    const int kk = i >> 2, e = 2 * (i & 3);
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      float2v v = {__builtin_amdgcn_exp2f(Cm[b][8 * kk + e]), __builtin_amdgcn_exp2f(Cm[b][8 * kk + e + 1])};
      half2v h = __builtin_convertvector(v, half2v);
      // keep the conversion (and its exponentials) here, between this
      // period's MFMAs, instead of next to the MFMA that consumes it
      asm volatile("" ::"v"(h));
      ap[b][kk][e] = h[0];
      ap[b][kk][e + 1] = h[1];
    }
  };
  // the masses of one tile's rounded allocations, pair i in the conversion's
  // order.  They are summed as one block at the start of the next period,
  // ahead of its MFMAs: one dot2 per GEMM2 step beside the exponentials made
  // pass 2 4.5% slower, and the block 1.5-2% faster than the compiler's own
  // placement (the same sums in the same order).
  auto mass_pair = [&](const half8 (&ap)[NB][2], int i) {
    const int kk = i >> 2, e = 2 * (i & 3);
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const half2v h = {ap[b][kk][e], ap[b][kk][e + 1]};
      msum[b] = __builtin_amdgcn_fdot2(h, ones, msum[b], false);
    }
  };
  // GEMM2 step m (m = 0 .. 2 DT - 1): U[proto, c] += sum_tok A'[proto, tok] h_tok[c]
  constexpr int M2 = 2 * C::DT;
  constexpr int EPM = 8 / M2;     // exponential pairs per GEMM2 step
  auto mma2 = [&](const half8 (&hb)[2][C::DT], const half8 (&ap)[NB][2], int m) {
    const int kk = m / C::DT, dt = m % C::DT;
#pragma unroll
    for (int b = 0; b < NB; ++b) U[b][dt] = mfma32x32x16(ap[b][kk], hb[kk][dt], U[b][dt]);
  };

  float16v C0[NB], C1[NB];
  half8 ap0[NB][2], ap1[NB][2];
  half8 ha[C::S], hb[2][C::DT];
  half8 nlp;
  // Period t sums the masses of tile t-2, runs GEMM2 of tile t-2 interleaved
  // with the exponentials of tile t-1, then GEMM1 of tile t+1, so every MFMA result is consumed a
  // whole period after its chain was issued (issue is in order per wave,
  // and both waves of a SIMD would otherwise stall on the same chain).
  // Registers: C(t-1) and C(t+1) share a set (GEMM1 of t+1 starts after the
  // exponentials of t-1 have read it), C(t) the other; A'(t-2) and A'(t-1)
  // one set each.  Flags (compile-time): G2 GEMM2 of t-2, EX exponentials
  // of t-1, MORE a tile t+1 follows, RB GEMM2's reads of tile t-1.
  // While direct-to-LDS loads are in flight the compiler can only wait for
  // all outstanding LDS reads of the wave, so each batch of reads is issued
  // one MFMA after the wait for the previous batch and consumed several MFMAs
  // later: GEMM1's reads of tile t+1 after the first GEMM2 step, GEMM2's
  // reads of tile t-1 after GEMM1's first step.
  auto period = [&](int t, float16v (&Cx)[NB], half8 (&apc)[NB][2], half8 (&app)[NB][2], auto g2c, auto exc,
                    auto morec, auto rbc) {
    constexpr bool G2 = decltype(g2c)::value, EX = decltype(exc)::value;
    constexpr bool MORE = decltype(morec)::value, RB = decltype(rbc)::value;
    if constexpr (MORE) boundary(t + 1);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (G2) {   // masses of tile t-2 (its allocations came in period t-1)
#pragma unroll
      for (int i = 0; i < 8; ++i) mass_pair(app, i);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int m = 0; m < M2; ++m) {
      if constexpr (G2) mma2(hb, app, m);
      if constexpr (EX) {
#pragma unroll
        for (int x = 0; x < EPM; ++x) expo2(Cx, apc, m * EPM + x);
      }
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (MORE) {
        if (m == 0) {
          read_a(t + 1, ha, nlp);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    if constexpr (MORE) {
      gemm1_head(ha, nlp, Cx);
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (RB) {
      read_b(t - 1, hb);
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (MORE) {
      gemm1_tail(ha, Cx);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  using T_ = std::true_type;
  using F_ = std::false_type;

  // The group's range is cut at user boundaries into segments (each a
  // multiple of 4 tiles); a segment's sums go to partial slot group + user,
  // unique among the groups whose ranges meet that user.
  float* part_u_all = ws_f32(ws, L.off_part_u);
  float* part_m_all = ws_f32(ws, L.off_part_m);
  int u = find_user(tile_base, L.R, s0);
  for (;;) {
    const int32_t ua = tile_base[u], ub = tile_base[u + 1];
    t0 = max(s0, ua);
    const int32_t te = min(s1, ub);
    if (te > t0) {
      nt = te - t0;
      nstages = nt / kStageTiles;
#pragma unroll
      for (int b = 0; b < NB; ++b) {
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt) U[b][dt] = float16v{};
        msum[b] = 0.f;
      }
#pragma unroll
      for (int st = 0; st < kAhead; ++st)
        if (st < nstages) issue(st, st);
      boundary(0);
      read_a(0, ha, nlp);
      gemm1_head(ha, nlp, C0);
      gemm1_tail(ha, C0);
      // nt is a positive multiple of 4 (a segment holds whole stages of one
      // user's tiles).  Parity p = t % 2: C(t-1), C(t+1) in set p ^ 1, A'(t-1) in set
      // p ^ 1, A'(t-2) in set p.
      period(0, C1, ap1, ap0, F_{}, F_{}, T_{}, F_{});
      period(1, C0, ap0, ap1, F_{}, T_{}, T_{}, T_{});
      int t = 2;
      for (; t < nt - 2; t += 2) {
        period(t, C1, ap1, ap0, T_{}, T_{}, T_{}, T_{});
        period(t + 1, C0, ap0, ap1, T_{}, T_{}, T_{}, T_{});
      }
      period(nt - 2, C1, ap1, ap0, T_{}, T_{}, T_{}, T_{});
      period(nt - 1, C0, ap0, ap1, T_{}, T_{}, F_{}, T_{});
      period(nt, C1, ap1, ap0, T_{}, T_{}, F_{}, T_{});
      period(nt + 1, C0, ap0, ap1, T_{}, F_{}, F_{}, F_{});

      float* part_u = part_u_all + (int64_t)(group + u) * L.k * D;
      float* part_m = part_m_all + (int64_t)(group + u) * L.k;
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
      lds_barrier();   // every wave is done with the stage buffers the next segment refills
    }
    if (ub >= s1) break;
    ++u;
  }
}

hipError_t launch_pass2(const Layout& L, void* ws, hipStream_t stream) {
  const int64_t grid = (int64_t)8 * L.n_pblocks * ((L.p2_groups + 7) / 8);
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
