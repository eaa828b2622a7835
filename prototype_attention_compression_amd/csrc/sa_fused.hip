// sa_fused.hip — one-pass FlashSA on gfx950 (bf16 inputs, k = 256 * P).
//
// What it computes (as the two-pass path): for each user and prototype j
//     U[j, :] = sum_t A[j,t] h_t,   m_j = sum_t A[j,t],
//     A[j,t]  = 2^(q_j . h_t) / Z_t,   Z_t = sum_j' 2^(q_j' . h_t)
// (per-token softmax over the prototypes: SequenceO1 blog "How it works"
// item 1, review FAQ on SA; q_j = P_j Wk^T log2(e) / sqrt(d)); the finalize
// kernel divides by the mass and applies Wv.  Nothing of size k x n is
// stored (blog "How it works" item 3).
//
// Why one pass.  A softmax over the k prototypes needs, for every token, the
// denominator Z_t over ALL k before any allocation is final, while the
// accumulators U of all k prototypes (k x d fp32 = 512 KB at k = 1024,
// d = 128) are the whole register file of a CU.  The two-pass path therefore
// computes every logit twice (pass 1 for Z_t, pass 2 again for A).  Here the
// P = k / 256 workgroups that own the prototype blocks of the same tokens run
// side by side (a cooperative launch guarantees they are co-resident) and
// exchange their per-token partial denominators through device-coherent
// memory: every logit is computed once.
//
// A workgroup has 4 waves (one per SIMD, up to 512 registers each); each
// wave owns 64 prototypes as two 32-prototype blocks, so every operand
// fragment read from LDS feeds two MFMAs.  Per 32-token tile a wave runs
//   GEMM1  C[j, t] = q_j . h_t                  (2 x 8 fp16 MFMAs, K = d)
//   E      = 2^C,  p = sum of a lane's 16 values of a block,  e = E / p in
//          fp16 (kept in registers while the denominator is exchanged)
//   partial denominator of the wave, then of the workgroup (LDS), published
//          to the group's exchange ring as a (tag, value) word
// and, three tiles later, when Z_t of that tile is known,
//   A'     = e * (p 2^14 / Z_t)  (= 2^14 A, packed fp16), staged through LDS
//          and read back transposed (ds_read_b64_tr_b16: lane = prototype)
//   mass  += A' (v_dot2 of the rounded values),  U += A' H  (2 x 8 fp16 MFMAs)
// The 2^14 scale keeps fp16 allocations in the normal range; it cancels in
// U / m.  If some token could overflow 2^C (largest |q| x largest |h| >= 100)
// the exact variant keeps per-lane maxima and exchanges partial
// log-sum-exps instead of sums.
//
// Exchange.  Wave 3 of every workgroup is the exchange wave: it publishes the
// workgroup partial of tile i at the start of iteration i + 1, polls the P
// words of tile i at the end of iteration i + 1, and at the end of iteration
// i + 2 writes 2^14 / Z_t to an LDS ring from which all waves read it in
// iteration i + 3.  It issues none of the token-row loads, so its waits on
// the polls never wait on row prefetches (vector-memory counters complete in
// order).  Every wait is bounded: on expiry the kernel raises a device error
// flag and finishes.  Measured round trip of such a word between two
// workgroups: about 0.9 us, a little over one tile of work.
//
// Data movement: token rows reach LDS with direct global->LDS loads (16 B per
// lane), 4 tiles per stage, four stage buffers (loads two stages ahead; the
// consuming GEMM2 lags three tiles behind GEMM1).  A row occupies 2d + 16
// bytes (one 16-byte chunk of padding, filled by the same direct loads).
// With that pitch the 16-byte GEMM1 reads (16 consecutive tokens, one chunk,
// per pass) meet 16 different bank groups, and so do the transposing 8-byte
// reads of GEMM2 (32 lanes: 4 tokens x 64 bytes) because the 4 tokens of one
// read are chosen 4 apart (token = 16 kk + 4 e + 2 g + h for K step kk,
// element e of read h in lane half g).  Every read is then a single per-lane
// base register plus an immediate offset.
//
// The allocation staging buffers (per wave and block, 32 tokens x 32
// prototypes fp16)
// stores token t in row 8 (t % 4) + t / 4 with its 16-byte chunks XOR'ed by
// t % 4: conflict-free for the 16-byte writes (lane = token) and for the
// transposing reads (lane = prototype, tokens as above).
//
// Work split: group g (its P workgroups on one XCD: dispatch goes round-robin
// over the 8 XCDs) walks tiles [g Tg, (g + 1) Tg) of the batch, Tg = the
// total rounded up to a multiple of 4 groups; the range is cut into segments
// at user boundaries and each segment's sums go to partial slot g + user.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "sa_device.h"
#include "sa_launch.h"

namespace sa {

namespace {

constexpr int kWaves = 4;
constexpr int kXWave = kWaves - 1;
constexpr int kNB = 2;            // 32-prototype blocks per wave
constexpr int kStageTiles = 4;
constexpr int kBufs = 4;
constexpr int kPSlots = 4;        // LDS slots of per-wave partials
constexpr int kSpinMax = 1 << 18; // bound on every wait on LDS (about 20 ms)
constexpr int kPollMax = 1 << 16; // bound on every wait on another workgroup (about 0.1 s)
constexpr float kShift = 16384.0f;  // 2^14

template <int D>
struct F {
  static constexpr int S = D / 16;                   // MFMA K steps over d
  static constexpr int DT = D / 32;                  // 32-column output blocks
  static constexpr int CPR = D / 8;                  // 16-B chunks per token row
  static constexpr int SLOTS = CPR + 1;              // ... plus one chunk of padding
  static constexpr int PITCH = SLOTS * 16;           // LDS bytes per token row
  static constexpr int TILE_BYTES = kTile * PITCH;
  static constexpr int ROWS_BYTES = kStageTiles * TILE_BYTES;
  static constexpr int VAL_OFF = ROWS_BYTES;         // per-token keep words of the stage
  static constexpr int STAGE_BYTES = VAL_OFF + kStageTiles * kTile * 4;
  static constexpr int LOADS_ROWS = kStageTiles * kTile * SLOTS / 64;   // 1-KB direct loads
  static constexpr int LOADS = LOADS_ROWS + 1;       // + one 512-B load of keep words
  // LDS map: the stage buffers (targets of the direct loads) ...
  static constexpr int ROWS_LDS = kBufs * STAGE_BYTES;
  // ... and, in a separate array (so that accesses to it provably do not
  // alias the direct loads in flight), the per-wave staging buffers and the
  // exchange state
  static constexpr int EBUF_OFF = 0;                                 // [waves][blocks][32 tok][32 proto] fp16
  static constexpr int PART_OFF = EBUF_OFF + kWaves * kNB * 2048;    // [kPSlots][32 tok][waves] float
  static constexpr int CNT_OFF = PART_OFF + kPSlots * kTile * kWaves * 4;   // [kPSlots][waves] uint32 progress
  static constexpr int ABORT_OFF = CNT_OFF + kPSlots * kWaves * 4;   // uint32
  static constexpr int ZR_OFF = CNT_OFF + 256;                       // [kXSlots][32] float
  static constexpr int ZTAG_OFF = ZR_OFF + kXSlots * kTile * 4;      // [kXSlots] uint32
  static constexpr int CTL_LDS = ZTAG_OFF + 64;
  static constexpr int LDS_BYTES = ROWS_LDS + CTL_LDS;
  static_assert(LOADS_ROWS * 64 == kStageTiles * kTile * SLOTS, "whole loads per stage");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
};

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef __attribute__((address_space(3))) s16x4* tr_ptr;

constexpr int waitcnt_vm(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }

// v_permlane32_swap with x as both operands: every lane l receives the value
// of lane l % 32 (first result) and of lane l % 32 + 32 (second result), so
// both lane halves combine the pair in the same order.
struct HalfPair {
  float lo, hi;
};
__device__ __forceinline__ HalfPair lane_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return {__uint_as_float(r[0]), __uint_as_float(r[1])};
}

__device__ __forceinline__ float log_add_exp2(float a, float b) {
  const float m = fmaxf(a, b);
  if (m == -INFINITY) return -INFINITY;
  return m + log2f(__builtin_amdgcn_exp2f(a - m) + __builtin_amdgcn_exp2f(b - m));
}

// Ordering between the waves of a workgroup through LDS.  LDS operations of
// one wave are performed in issue order, so a handshake needs only that the
// compiler keeps the order (memory clobber) and, before a flag is set, that
// this wave's earlier LDS operations are complete (lgkmcnt).  The flags are
// plain loads and stores: the compiler makes atomic LDS operations and
// language-level fences wait for every outstanding direct global->LDS load
// (vmcnt(0)), i.e. for the row prefetches two stages ahead.
__device__ __forceinline__ void cbar() { asm volatile("" ::: "memory"); }
__device__ __forceinline__ uint32_t lds_flag_load(const uint32_t* p) {
  cbar();
  const uint32_t v = *p;
  cbar();
  return v;
}
__device__ __forceinline__ void lds_flag_store(uint32_t* p, uint32_t v) {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  *p = v;
  cbar();
}
}  // namespace

template <int D, int P, bool EXACT>
__device__ __forceinline__ void fused_body(const Layout& L, void* ws, char* lds, char* ctl, int group, int pb,
                                           int32_t ga, int32_t gb) {
  using C = F<D>;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, g = lane >> 5;
  const bool xw = (wave == kXWave);
  const int p0 = pb * kFusedProtos + wave * (kNB * kProtoPerWave);   // the wave's first prototype

  // zero the progress words, abort word and ring tags (used across
  // segments; the first stage barrier orders these stores before any use)
  if (tid < 64) reinterpret_cast<uint32_t*>(ctl + C::CNT_OFF)[tid] = 0u;
  if (tid < 16) reinterpret_cast<uint32_t*>(ctl + C::ZTAG_OFF)[tid] = 0u;
  // Every wait loop gives up after a bound and then sets the workgroup's
  // abort word: from then on no wait of this workgroup blocks (it still
  // publishes, so the other workgroups of its group keep going) and the
  // device error flag is raised at the end.  A wait can thus cost its bound
  // at most once per workgroup.
  uint32_t* abort_word = reinterpret_cast<uint32_t*>(ctl + C::ABORT_OFF);
  auto aborted = [&]() { return lds_flag_load(abort_word) != 0u; };
  auto give_up = [&]() { lds_flag_store(abort_word, 1u); };
  uint32_t* prog_words = reinterpret_cast<uint32_t*>(ctl + C::CNT_OFF);
  uint32_t* ztag = reinterpret_cast<uint32_t*>(ctl + C::ZTAG_OFF);
  float* zring = reinterpret_cast<float*>(ctl + C::ZR_OFF);
  float* part = reinterpret_cast<float*>(ctl + C::PART_OFF);

  // A operands of GEMM1: per block b the 32 query rows, row m holding
  // prototype p0 + 32 b + pi(m) with pi(8 (r/4) + 4 h + r % 4) = 16 h + r, so
  // that accumulator register r of lane half h is prototype p0 + 32 b + 16 h
  // + r (16 contiguous prototypes per lane and block)
  const _Float16* q16 = ws_f16(ws, L.off_q16);
  half8 qf[kNB][C::S];
  {
    const int pm = 16 * ((col >> 2) & 1) + 4 * (col >> 3) + (col & 3);
#pragma unroll
    for (int b = 0; b < kNB; ++b)
#pragma unroll
      for (int s = 0; s < C::S; ++s)
        qf[b][s] = *reinterpret_cast<const half8*>(q16 + (int64_t)(p0 + 32 * b + pm) * D + 16 * s + 8 * g);
  }

  const char* h16 = reinterpret_cast<const char*>(ws_f16(ws, L.off_h16));
  const char* valg = reinterpret_cast<const char*>(ws_i32(ws, L.off_nl));
  uint64_t* xbuf = reinterpret_cast<uint64_t*>(reinterpret_cast<char*>(ws) + L.off_xbuf) +
                   (int64_t)group * kXSlots * kTile * P;

  // row loads: load i of a stage (i < LOADS_ROWS: 1 KB of rows; i ==
  // LOADS_ROWS: the stage's keep words) is issued by wave i % 7
  constexpr int NLW = kWaves - 1;
  const int my_loads = xw ? 0 : (C::LOADS - wave + NLW - 1) / NLW;
  constexpr int LMAX = (C::LOADS + NLW - 1) / NLW;
  constexpr int LMIN = C::LOADS / NLW;
  static_assert(LMAX < 64, "vmcnt range");

  // per-lane LDS byte offsets (per K step, output block, tile and stage
  // buffer only immediates or one scalar are added)
  const int i16 = lane & 15, gh = (lane >> 4) & 1;
  // GEMM1 B operand: token row `col`, chunk 2 s + g
  const int ha_base = col * C::PITCH + 16 * g;
  // GEMM2 B operand, transposing reads: source lane i16 of 16-lane group gh
  // reads token 4 (i16 / 4) + 2 g (+ 16 kk + h) at columns 16 gh + 4 (i16 % 4)
  // (+ 32 dt) .. + 3
  const int tr_base = (4 * (i16 >> 2) + 2 * g) * C::PITCH + 32 * gh + 8 * (i16 & 3);
  // the wave's allocation staging buffers (block b at + 2048 b)
  char* ebuf = ctl + C::EBUF_OFF + wave * (kNB * 2048);
  const int erow = 8 * (col & 3) + (col >> 2);
  const int ew0 = erow * 64 + (((2 * g) ^ (col & 3)) * 16);
  const int ew1 = erow * 64 + (((2 * g + 1) ^ (col & 3)) * 16);
  int er_off[2];        // GEMM2 A operand: token 4 (i16 / 4) + 2 g + h (+ 16 kk), prototypes 16 gh + 4 (i16 % 4) ..
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int x = 2 * g + h;                         // token % 4
    const int row = 8 * x + (i16 >> 2);              // 8 (t % 4) + t / 4 at kk = 0
    const int chunk = 2 * gh + ((i16 & 3) >> 1);
    er_off[h] = row * 64 + ((chunk ^ x) * 16) + 8 * (i16 & 1);
  }
  // Allocation staging round trip of one tile (both blocks, block b at
  // + 2048 b): the 16-byte writes (lane = token), then the transposing reads
  // (lane = prototype), in one asm block with one wait at the end.  A wave's
  // LDS operations complete in issue order, so the reads see the writes.  As
  // builtins, the compiler would put a wait for every outstanding load (all
  // direct-load prefetches) in front of them.
  const uint32_t a_w0 = lds_addr(ebuf + ew0), a_w1 = lds_addr(ebuf + ew1);
  const uint32_t a_r0 = lds_addr(ebuf + er_off[0]), a_r1 = lds_addr(ebuf + er_off[1]);
  auto stage_allocations = [&](const half8 (&w)[kNB][2], half8 (&ap)[kNB][2]) {
    static_assert(kNB == 2, "two blocks, at + 0 and + 2048");
    s16x4 r0, r1, r2, r3, r4, r5, r6, r7;
    asm volatile(
        "ds_write_b128 %8, %12\n\t"
        "ds_write_b128 %9, %13\n\t"
        "ds_write_b128 %8, %14 offset:2048\n\t"
        "ds_write_b128 %9, %15 offset:2048\n\t"
        "ds_read_b64_tr_b16 %0, %10\n\t"
        "ds_read_b64_tr_b16 %1, %11\n\t"
        "ds_read_b64_tr_b16 %2, %10 offset:256\n\t"
        "ds_read_b64_tr_b16 %3, %11 offset:256\n\t"
        "ds_read_b64_tr_b16 %4, %10 offset:2048\n\t"
        "ds_read_b64_tr_b16 %5, %11 offset:2048\n\t"
        "ds_read_b64_tr_b16 %6, %10 offset:2304\n\t"
        "ds_read_b64_tr_b16 %7, %11 offset:2304\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3), "=&v"(r4), "=&v"(r5), "=&v"(r6), "=&v"(r7)
        : "v"(a_w0), "v"(a_w1), "v"(a_r0), "v"(a_r1), "v"(w[0][0]), "v"(w[0][1]), "v"(w[1][0]), "v"(w[1][1])
        : "memory");
    const s16x4 r[8] = {r0, r1, r2, r3, r4, r5, r6, r7};
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const s16x4 lo = r[4 * b + 2 * kk], hi = r[4 * b + 2 * kk + 1];
        ap[b][kk] = __builtin_bit_cast(half8, s16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
      }
  };

  const int32_t* tile_base = ws_i32(ws, L.off_tile_base);
  float* part_u_all = ws_f32(ws, L.off_part_u);
  float* part_m_all = ws_f32(ws, L.off_part_m);
  const half2v ones = {(_Float16)1.0f, (_Float16)1.0f};

  // the group's tile range, segment by segment (one user each)
  int u = find_user(tile_base, L.R, ga);
  int32_t seq0 = 0;   // sequence number (within the group) of the segment's first tile; a multiple of 4
  for (;;) {
    const int32_t s0 = max(ga, tile_base[u]);
    const int32_t s1 = min(gb, tile_base[u + 1]);
    if (s1 > s0) {
      const int n = s1 - s0;                // tiles, a multiple of 4
      const int nst = n / kStageTiles;
      float16v U[kNB][C::DT];
#pragma unroll
      for (int b = 0; b < kNB; ++b)
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt) U[b][dt] = float16v{};
      float msum[kNB] = {};
      half8 e[4][kNB][2];                    // ring of normalised exponentials (fp16)
      float pl[4][kNB];                      // ... and the lane sums they were divided by
      uint64_t pw[(P >= 2) ? P / 2 : 1];     // exchange words in flight (wave 7)

      auto issue = [&](int ts, int b) {
        if (xw) return;
        char* base = lds + b * C::STAGE_BYTES;
        const int64_t tile0 = (int64_t)s0 + (int64_t)ts * kStageTiles;
#pragma unroll 1
        for (int i = wave; i < C::LOADS; i += NLW) {
          if (i < C::LOADS_ROWS) {
            // 16-byte slot 64 i + lane of the stage: row q / SLOTS, chunk q % SLOTS
            // (the padding chunk re-reads chunk 0 of its row)
            const int q = 64 * i + lane;
            const int row = q / C::SLOTS;
            int c = q - row * C::SLOTS;
            c = c == C::CPR ? 0 : c;
            const char* src = h16 + (tile0 * kTile + row) * (D * 2) + c * 16;
            __builtin_amdgcn_global_load_lds(src, (lds_ptr_t)(base + 1024 * i), 16, 0, 0);
          } else if (lane < 32) {
            const char* src = valg + tile0 * (kTile * 4) + lane * 16;
            __builtin_amdgcn_global_load_lds(src, (lds_ptr_t)(base + C::VAL_OFF), 16, 0, 0);
          }
        }
      };

      // ---- exchange-wave steps (tile with group sequence number sq; LDS
      // partial slot ps = sq % 4, ring slot zs = sq % 8) -------------------
      // publish the workgroup partial of a tile whose keep words are at vbase
      auto publish = [&](int32_t sq, int ps, int zs, const char* vbase) {
        // every wave has stored its partial of this tile (progress words)
        const uint32_t want = (uint32_t)(sq + 1);
        static_assert(kWaves == 4, "one 16-byte read of progress words");
        const u32x4* prog = reinterpret_cast<const u32x4*>(prog_words + ps * kWaves);
        int n_spin = 0;
        for (;;) {
          cbar();
          const u32x4 a = prog[0];
          cbar();
          if (a[0] == want && a[1] == want && a[2] == want && a[3] == want) break;
          if (aborted()) break;
          if (++n_spin > kSpinMax) { give_up(); break; }
          __builtin_amdgcn_s_sleep(1);
        }
        const float* pp = part + (ps * kTile + col) * kWaves;
        float v;
        if (!EXACT) {
          v = 0.f;
#pragma unroll
          for (int w = 0; w < kWaves; ++w) v += pp[w];
        } else {
          v = -INFINITY;
#pragma unroll
          for (int w = 0; w < kWaves; ++w) v = log_add_exp2(v, pp[w]);
        }
        const bool keep = reinterpret_cast<const uint32_t*>(vbase)[col] != 0u;
        if (!keep) v = EXACT ? -INFINITY : INFINITY;
        if (P == 1) {
          // the workgroup holds every prototype: its partial is the total
          if (g == 0) {
            float r;
            if (!EXACT) r = keep ? kShift * __builtin_amdgcn_rcpf(v) : 0.f;
            else r = keep ? v : INFINITY;
            zring[zs * kTile + col] = r;
          }
          if (lane == 0) lds_flag_store(ztag + zs, want);
        } else if (g == 0) {
          const uint64_t word = ((uint64_t)want << 32) | (uint64_t)__float_as_uint(v);
          __hip_atomic_store(xbuf + (zs * kTile + col) * P + pb, word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      };
      auto poll_issue = [&](int zs) {
        if (P == 1) return;
        const uint64_t* src = xbuf + (zs * kTile + col) * P + g * (P / 2);
#pragma unroll
        for (int q = 0; q < P / 2; ++q) pw[q] = __hip_atomic_load(src + q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      };
      auto poll_finish = [&](int32_t sq, int zs) {
        if (P == 1) return;
        const uint32_t tag = (uint32_t)(sq + 1);
        int n_spin = 0;
        for (;;) {
          bool ok = true;
#pragma unroll
          for (int q = 0; q < P / 2; ++q) ok = ok && ((uint32_t)(pw[q] >> 32) == tag);
          if (__all(ok)) break;
          if (aborted()) break;
          if (++n_spin > kPollMax) { give_up(); break; }
          __builtin_amdgcn_s_sleep(2);
          poll_issue(zs);
        }
        float v;
        if (!EXACT) {
          v = 0.f;
#pragma unroll
          for (int q = 0; q < P / 2; ++q) v += __uint_as_float((uint32_t)pw[q]);
          const HalfPair hp = lane_halves(v);
          v = hp.lo + hp.hi;
        } else {
          v = -INFINITY;
#pragma unroll
          for (int q = 0; q < P / 2; ++q) v = log_add_exp2(v, __uint_as_float((uint32_t)pw[q]));
          const HalfPair hp = lane_halves(v);
          v = log_add_exp2(hp.lo, hp.hi);
        }
        if (g == 0) {
          float r;
          if (!EXACT) r = (v == INFINITY) ? 0.f : kShift * __builtin_amdgcn_rcpf(v);
          else r = (v == -INFINITY) ? INFINITY : v;
          zring[zs * kTile + col] = r;
        }
        if (lane == 0) lds_flag_store(ztag + zs, tag);
      };

      // ---- one iteration ---------------------------------------------------
      // GEMM1 of local tile i (stage buffer B1, tile t1 of its stage) when G1,
      // GEMM2 of tile i - 3 (buffer B2, tile t2) when CONS.  zs8 = the group
      // sequence number of tile i mod 8 (sq = seq0 + i with seq0 and the
      // stage start multiples of 4, so sq mod 4 = t1).
      auto iter = [&](int i, int B1, auto t1c, int B2, int t2, auto g1c, auto consc, int zs8) {
        constexpr int t1 = decltype(t1c)::value;
        constexpr bool G1 = decltype(g1c)::value, CONS = decltype(consc)::value;
        constexpr int ER = t1;                 // ring slot of tile i
        constexpr int EC = (t1 + 1) & 3;       // ring slot of tile i - 3
        const int32_t sq = seq0 + i;
        // exchange wave: publish tile i - 1 (keep words: tile t1 - 1 of B1, or
        // tile 3 of the previous buffer)
        if (xw && i >= 1 && i - 1 < n) {
          const int VB = t1 > 0 ? B1 : (B1 + kBufs - 1) % kBufs;
          constexpr int VT = t1 > 0 ? t1 - 1 : kStageTiles - 1;
          publish(sq - 1, (t1 + 3) & 3, (zs8 + 7) & 7, lds + VB * C::STAGE_BYTES + C::VAL_OFF + VT * kTile * 4);
        }
        // wait until 2^14 / Z of tile i - 3 is in the ring
        const int zc = (zs8 + 5) & 7;
        if (CONS) {
          const uint32_t want = (uint32_t)(sq - 2);
          int n_spin = 0;
          while (lds_flag_load(ztag + zc) != want) {
            if (aborted()) break;
            if (++n_spin > kSpinMax) { give_up(); break; }
            __builtin_amdgcn_s_sleep(1);
          }
        }

        // ---- main block.  Region 1: GEMM1(i) with the allocations of tile
        // i - 3 (scale, staging round trip) under its MFMAs.  Region 2: GEMM2
        // of tile i - 3 with the exponentials of tile i under its MFMAs.
        __builtin_amdgcn_sched_barrier(0);
        half8 ha[C::S];
        if (G1) {
          const char* rows = lds + (B1 * C::STAGE_BYTES + t1 * C::TILE_BYTES + ha_base);
#pragma unroll
          for (int s = 0; s < C::S; ++s) ha[s] = *reinterpret_cast<const half8*>(rows + 32 * s);
        }
        half8 ap[kNB][2];
        if (CONS) {
          const float r = zring[zc * kTile + col];
          half8 w[kNB][2];
#pragma unroll
          for (int b = 0; b < kNB; ++b) {
            float sc;
            if (!EXACT) sc = pl[EC][b] * r;
            else sc = __builtin_amdgcn_exp2f(pl[EC][b] - r + 14.0f);
            const _Float16 hs = (_Float16)sc;
            w[b][0] = e[EC][b][0] * hs;
            w[b][1] = e[EC][b][1] * hs;
          }
          stage_allocations(w, ap);
        }
        float16v acc[kNB];
#pragma unroll
        for (int b = 0; b < kNB; ++b) acc[b] = float16v{};
        if (G1) {
#pragma unroll
          for (int s = 0; s < C::S; ++s)
#pragma unroll
            for (int b = 0; b < kNB; ++b) acc[b] = mfma32x32x16(qf[b][s], ha[s], acc[b]);
        }
        if (CONS) {
#pragma unroll
          for (int b = 0; b < kNB; ++b)
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                const half2v pr = {ap[b][kk][2 * q], ap[b][kk][2 * q + 1]};
                msum[b] = __builtin_amdgcn_fdot2(pr, ones, msum[b], false);
              }
        }
        if (G1 && CONS) {
          __builtin_amdgcn_sched_group_barrier(0x100, C::S + 1, 0);   // GEMM1 operands, ring value
#pragma unroll
          for (int q = 0; q < kNB * C::S; ++q) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);        // 1 MFMA
            __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);        // 2 VALU
            __builtin_amdgcn_sched_group_barrier(0x300, 1, 0);        // 1 LDS read or write
          }
        }
        __builtin_amdgcn_sched_barrier(0);
        if (CONS) {
          half8 hb[2][C::DT];
          tile_tr_reads<D>(lds_addr(lds + (B2 * C::STAGE_BYTES + t2 * C::TILE_BYTES + tr_base)), hb);
#pragma unroll
          for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
              for (int b = 0; b < kNB; ++b) U[b][dt] = mfma32x32x16(ap[b][kk], hb[kk][dt], U[b][dt]);
        }
        if (G1) {
          float pv[kNB];
#pragma unroll
          for (int b = 0; b < kNB; ++b) {
            float E[16];
            if (!EXACT) {
              float s0v = 0.f, s1v = 0.f;
#pragma unroll
              for (int r = 0; r < 16; r += 2) {
                E[r] = __builtin_amdgcn_exp2f(acc[b][r]);
                E[r + 1] = __builtin_amdgcn_exp2f(acc[b][r + 1]);
                s0v += E[r];
                s1v += E[r + 1];
              }
              pv[b] = s0v + s1v;
              pl[ER][b] = pv[b];
            } else {
              float m = acc[b][0];
#pragma unroll
              for (int r = 1; r < 16; ++r) m = fmaxf(m, acc[b][r]);
              float s0v = 0.f, s1v = 0.f;
#pragma unroll
              for (int r = 0; r < 16; r += 2) {
                E[r] = __builtin_amdgcn_exp2f(acc[b][r] - m);
                E[r + 1] = __builtin_amdgcn_exp2f(acc[b][r + 1] - m);
                s0v += E[r];
                s1v += E[r + 1];
              }
              pv[b] = s0v + s1v;
              pl[ER][b] = m + log2f(pv[b]);
            }
            const float rp = __builtin_amdgcn_rcpf(pv[b]);
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                const float2v v = {E[8 * hh + 2 * q] * rp, E[8 * hh + 2 * q + 1] * rp};
                const half2v hv = __builtin_convertvector(v, half2v);
                e[ER][b][hh][2 * q] = hv[0];
                e[ER][b][hh][2 * q + 1] = hv[1];
              }
          }
          // the wave's partial over its 64 prototypes, into LDS slot t1
          float wpart;
          if (!EXACT) {
            const HalfPair hp = lane_halves(pv[0] + pv[1]);
            wpart = hp.lo + hp.hi;
          } else {
            const HalfPair hp = lane_halves(log_add_exp2(pl[ER][0], pl[ER][1]));
            wpart = log_add_exp2(hp.lo, hp.hi);
          }
          if (g == 0) part[(t1 * kTile + col) * kWaves + wave] = wpart;
        }
        if (G1 && CONS) {
#pragma unroll
          for (int q = 0; q < 2 * C::DT; ++q) {
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);        // 2 transposing reads
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);        // 1 MFMA
            __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);        // 4 VALU
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);        // 1 MFMA
            __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);        // 4 VALU
          }
        }
        __builtin_amdgcn_sched_barrier(0);
        if (G1 && lane == 0) lds_flag_store(prog_words + t1 * kWaves + wave, (uint32_t)(sq + 1));

        // exchange wave: Z of tile i - 2 into the ring, then poll tile i - 1
        if (xw) {
          if (i - 2 >= 0 && i - 2 < n) poll_finish(sq - 2, (zs8 + 6) & 7);
          if (i - 1 >= 0 && i - 1 < n) poll_issue((zs8 + 7) & 7);
        }
      };

      // ---- stages ------------------------------------------------------------
      using I0 = std::integral_constant<int, 0>;
      using I1 = std::integral_constant<int, 1>;
      using I2 = std::integral_constant<int, 2>;
      using I3 = std::integral_constant<int, 3>;
      using T = std::true_type;
      using Fl = std::false_type;
      auto stage_head = [&](int st) {
        if (!xw) {
          if (st + 1 < nst) {
            if (my_loads == LMAX) __builtin_amdgcn_s_waitcnt(waitcnt_vm(LMAX));
            else __builtin_amdgcn_s_waitcnt(waitcnt_vm(LMIN));
          } else {
            __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
          }
        }
        lds_barrier();     // stage st is in LDS; stage st - 2's buffer is free
        if (st + 2 < nst) issue(st + 2, (st + 2) % kBufs);
      };

      issue(0, 0);
      if (nst > 1) issue(1, 1);
      {  // stage 0: no tile to consume before tile 3
        stage_head(0);
        const int zb = (seq0 & 4);
        iter(0, 0, I0{}, 0, 0, T{}, Fl{}, zb + 0);
        iter(1, 0, I1{}, 0, 0, T{}, Fl{}, zb + 1);
        iter(2, 0, I2{}, 0, 0, T{}, Fl{}, zb + 2);
        iter(3, 0, I3{}, 0, 0, T{}, T{}, zb + 3);
      }
      for (int st = 1; st < nst; ++st) {
        stage_head(st);
        const int B = st % kBufs, Bp = (st + kBufs - 1) % kBufs;
        const int i0 = kStageTiles * st;
        const int zb = (seq0 + i0) & 4;
        iter(i0 + 0, B, I0{}, Bp, 1, T{}, T{}, zb + 0);
        iter(i0 + 1, B, I1{}, Bp, 2, T{}, T{}, zb + 1);
        iter(i0 + 2, B, I2{}, Bp, 3, T{}, T{}, zb + 2);
        iter(i0 + 3, B, I3{}, B, 0, T{}, T{}, zb + 3);
      }
      {  // drain: tiles n-3 .. n-1 are tiles 1..3 of the last stage (buffer Bl);
         // iteration n also publishes tile n-1, whose keep words iter() finds
         // in "tile 3 of the buffer before B1" with B1 = Bl + 1
        const int Bl = (nst - 1) % kBufs, Bn = (Bl + 1) % kBufs;
        const int zb = (seq0 + n) & 4;
        iter(n + 0, Bn, I0{}, Bl, 1, Fl{}, T{}, zb + 0);
        iter(n + 1, Bn, I1{}, Bl, 2, Fl{}, T{}, zb + 1);
        iter(n + 2, Bn, I2{}, Bl, 3, Fl{}, T{}, zb + 2);
      }

      float* part_u = part_u_all + (int64_t)(group + u) * L.k * D;
      float* part_m = part_m_all + (int64_t)(group + u) * L.k;
#pragma unroll
      for (int b = 0; b < kNB; ++b) {
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            part_u[(int64_t)(p0 + 32 * b + acc_row(r, g)) * D + 32 * dt + col] = U[b][dt][r];
        const float m = msum[b] + __shfl_xor(msum[b], 32);
        if (g == 0) part_m[p0 + 32 * b + col] = m;
      }
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
      lds_barrier();     // every wave is done with the stage buffers
      seq0 += n;
    }
    if (s1 >= gb) break;
    ++u;
  }
  // the last segment ended with a barrier: every wave is past its waits
  if (tid == 0 && aborted()) atomicOr(ws_i32(ws, L.off_hdr) + kHdrErr, kErrExchange);
}

// Grid: groups x P workgroups of 8 waves, launched cooperatively (all
// co-resident).  Workgroup x sits on XCD x % 8; the P workgroups of a group
// are consecutive slots x / 8 of one XCD.
template <int D, int P>
__global__ __launch_bounds__(kWaves * 64) void fused_accum(Layout L, void* ws) {
  __shared__ __attribute__((aligned(1024))) char lds[F<D>::ROWS_LDS];
  __shared__ __attribute__((aligned(1024))) char ctl[F<D>::CTL_LDS];
  const int32_t* hdr = ws_i32(ws, L.off_hdr);
  const int x = blockIdx.x, xcd = x & 7, slotw = x >> 3;
  const int group = xcd + 8 * (slotw / P);
  const int pb = slotw % P;
  const int G = L.groups;
  const int32_t T = hdr[kHdrTiles];
  const int32_t Tg = (T + 4 * G - 1) / (4 * G) * 4;
  const int32_t ga = group * Tg;
  const int32_t gb = min(T, ga + Tg);
  if (ga >= gb) return;  // uniform over the group
  // |q_j . h_t| <= qmax hmax: below 100 no 2^L can overflow or leave the
  // normal range, and plain sums are exact enough
  const float bound = query_norm_max(L, ws) * __int_as_float(hdr[kHdrHmax]);
  if (bound < 100.0f)
    fused_body<D, P, false>(L, ws, lds, ctl, group, pb, ga, gb);
  else
    fused_body<D, P, true>(L, ws, lds, ctl, group, pb, ga, gb);
}

bool fused_shape_ok(const Layout& L) {
  if (L.dtype != 0 || (L.d != 64 && L.d != 128)) return false;
  const int P = L.k / kFusedProtos;
  return L.k % kFusedProtos == 0 && (P == 1 || P == 2 || P == 4 || P == 8 || P == 16);
}

namespace {
template <int D, int P>
const void* kernel_of() {
  return reinterpret_cast<const void*>(&fused_accum<D, P>);
}
template <int D>
const void* kernel_p(int P) {
  switch (P) {
    case 1: return kernel_of<D, 1>();
    case 2: return kernel_of<D, 2>();
    case 4: return kernel_of<D, 4>();
    case 8: return kernel_of<D, 8>();
    default: return kernel_of<D, 16>();
  }
}
const void* fused_kernel(const Layout& L) {
  const int P = L.k / kFusedProtos;
  return L.d == 128 ? kernel_p<128>(P) : kernel_p<64>(P);
}
}  // namespace

bool fused_fits_device(const Layout& L, int device) {
  int coop = 0, cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, device) != hipSuccess || !coop) return false;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess) return false;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fused_kernel(L), kWaves * 64, 0) != hipSuccess)
    return false;
  return (int64_t)cus * per_cu >= (int64_t)L.groups * (L.k / kFusedProtos);
}

hipError_t launch_fused(const Layout& L, void* ws, hipStream_t stream) {
  Layout Lc = L;
  void* wsp = ws;
  void* args[] = {&Lc, &wsp};
  return hipLaunchCooperativeKernel(fused_kernel(L), dim3(L.groups * (L.k / kFusedProtos)), dim3(kWaves * 64),
                                    args, 0, stream);
}

}  // namespace sa
