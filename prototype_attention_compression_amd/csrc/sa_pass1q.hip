// sa_pass1q.hip — FlashSA pass 1 with the queries resident in registers
// (gfx950, bf16 inputs, k = 256, 512 or 1024).
//
// Same outputs as pass1_lse (the per-token base-2 logsumexp over ALL k
// prototypes, SequenceO1 blog "How it works" item 1 and review FAQ on SA,
// delivered as pass 2's -l fp16 pairs, and the fp16 token rows), computed
// the other way round: instead of streaming the k x d queries through LDS
// for every 256 tokens, each workgroup keeps all k query rows in registers
// (8 waves x k/8 rows: 128 registers per lane at k = 1024) and streams its
// contiguous range of tokens through LDS once.  A token's logsumexp is then
// complete inside the workgroup: 8 per-wave partials, summed through LDS.
//
// Per 32-token tile:
//   * conversion (all 512 threads, one 16-byte chunk each): the bf16 row
//     chunk loaded two tiles earlier is widened to fp16 (exact for
//     magnitudes in [2^-17, 65504]; a kept value beyond that range raises
//     a device error bit), written to LDS and to the fp16 row buffer pass 2
//     reads; masked tokens and padding rows are zero (a padding slot loads
//     the workspace's zero row, a masked token's chunk is cleared).  The row
//     norms decide, per tile, whether any logit can reach |L| >= 100
//     (Cauchy-Schwarz with the largest query norm): then the tile takes the
//     exact form (running maximum, rescaled sums), else plain sums of 2^L;
//   * compute (each wave: its k/8 prototypes, NBW blocks of 32): 8 16-byte
//     operand reads, NBW x 8 fp16 MFMAs (lane = token, so the sum over
//     prototypes stays in the lane), exponentials and sums;
//   * the first four waves turn 8 tokens each of the previous tile from 8
//     partials into -l pairs.
// One barrier per tile; three LDS tile buffers (convert t+1 while computing
// t); the global loads run two tiles ahead in registers.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "sa_device.h"
#include "sa_launch.h"

namespace sa {

namespace {

constexpr int kBufs = 3;
constexpr int kWGs = 256;          // persistent grid: workgroups per CU x 256 CUs

template <int D>
struct Q1 {
  static constexpr int S = D / 16;                 // MFMA K steps over d
  static constexpr int CPR = D / 8;                // 16-B chunks per row
  static constexpr int PITCH = (CPR + 1) * 16;     // padded LDS row
  static constexpr int TILE_BYTES = kTile * PITCH;
  static constexpr int CHUNKS = kTile * CPR;       // 16-B chunks per tile (<= 512)
};

// log2 of x >= 2^-126 (no denormal inputs): the hardware instruction alone.
// Every logarithm here is of a sum that holds a term of at least 2^-100 (the
// fast form: every logit above -100) or of exactly 1 (the max-shifted form).
__device__ __forceinline__ float log2_normal(float x) { return __builtin_amdgcn_logf(x); }

__device__ __forceinline__ float log_add_exp2(float a, float b) {
  const float m = fmaxf(a, b);
  if (m == -INFINITY) return -INFINITY;
  return m + log2_normal(__builtin_amdgcn_exp2f(a - m) + __builtin_amdgcn_exp2f(b - m));
}

// Issue priority of the calling wave (0..3; the instruction takes a
// constant).
__device__ __forceinline__ void wave_priority(int p) {
  switch (p) {
    case 0: __builtin_amdgcn_s_setprio(0); break;
    case 1: __builtin_amdgcn_s_setprio(1); break;
    case 2: __builtin_amdgcn_s_setprio(2); break;
    default: __builtin_amdgcn_s_setprio(3); break;
  }
}

// value of lane l % 32 (lo) and of lane l % 32 + 32 (hi), in every lane
struct HalfPair {
  float lo, hi;
};
__device__ __forceinline__ HalfPair lane_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return {__uint_as_float(r[0]), __uint_as_float(r[1])};
}

}  // namespace

template <int D, int NBW, bool MASKED, int W>
__global__ __launch_bounds__(W * 64, NBW == 1 ? 4 : 2) void pass1_qres(const uint16_t* __restrict__ H,
                                                          const int64_t* __restrict__ offsets,
                                                          const uint8_t* __restrict__ mask,
                                                          const int32_t* __restrict__ tile_base, Layout L,
                                                          void* __restrict__ ws) {
  using C = Q1<D>;
  __shared__ __attribute__((aligned(1024))) char rows[kBufs][C::TILE_BYTES];
  static_assert(W % 4 == 0 && kTile % W == 0, "wave count");
  __shared__ float part[2][kTile][W];
  // one byte per wave: "a logit of this wave's chunks may reach 100"
  static_assert(W == 4 || W == 8, "exact bytes read as one word");
  __shared__ __attribute__((aligned(8))) uint8_t exact_bytes[kBufs][W];
  // masked batches: whether each token of the tile is kept (unmasked ones
  // use the tile's token count, a scalar)
  __shared__ uint32_t keep_words[MASKED ? kBufs : 1][kTile];
  // A word per lane for the stores of lanes whose value another lane
  // already stores: the store address is a select, not a branch, and no two
  // lanes of a store share an address (same-address LDS stores serialise).
  __shared__ uint32_t spare[W * 64];

  const int32_t* hdr = ws_i32(ws, L.off_hdr);
  const int32_t T = hdr[kHdrTiles];
  const int32_t per = (T + gridDim.x - 1) / gridDim.x;
  const int32_t ta = blockIdx.x * per;
  const int32_t tb = min(T, ta + per);
  if (ta >= tb) return;  // uniform
  const int n = tb - ta;
  const float qmax = query_norm_max(L, ws);
  const float lim2 = 10000.0f / fmaxf(qmax * qmax, 1e-30f);   // |h|^2 >= lim2  <=>  qmax |h| >= 100
  const float lim2c = lim2 / (float)C::CPR;   // the same against a chunk's squared norm (CPR: power of two)

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar branches on it
  const int col = lane & 31, g = lane >> 5;

  // A operands: the wave's NBW blocks of 32 query rows (lane = prototype row)
  const _Float16* q16 = ws_f16(ws, L.off_q16);
  half8 qf[NBW][C::S];
#pragma unroll
  for (int b = 0; b < NBW; ++b)
#pragma unroll
    for (int s = 0; s < C::S; ++s)
      qf[b][s] = *reinterpret_cast<const half8*>(q16 + (int64_t)((wave * NBW + b) * 32 + col) * D + 16 * s + 8 * g);

  _Float16* h16 = ws_f16(ws, L.off_h16);
  uint32_t* nl = reinterpret_cast<uint32_t*>(ws_i32(ws, L.off_nl));
  const uint16_t* zrow = reinterpret_cast<const uint16_t*>(ws_i32(ws, L.off_zrow));

  // conversion role of this thread: chunk q of a tile (row q / CPR, chunk q %
  // CPR); at d = 128 every thread has one
  constexpr bool kAllConvert = C::CHUNKS == W * 64;
  const bool conv = kAllConvert || tid < C::CHUNKS;
  const int crow = tid / C::CPR, cch = tid % C::CPR;
  // Forward walk over the tiles being loaded (tile index increases).  The
  // user lookup reads only kernel arguments the kernel never writes, so it
  // compiles to scalar loads.  The row chunk (and mask byte) load is issued
  // unconditionally from an address clamped into the same user's rows, with
  // whether the slot is live kept aside: no load sits behind a branch, so
  // the compiler's wait before the conversion two tiles later counts only
  // what was issued after it instead of draining the prefetches and stores.
  // A slot that holds no token (a padding slot: tiles are rounded up to a
  // multiple of kUserTileAlign, so it may lie past the end of H) reads the
  // workspace's zero row, and its mask byte (masked batches) from the user's
  // first token: a user with tiles has at least one.  `cnt` is the tile's
  // token count (scalar; 0 past the workgroup's range).
  // The current user's tile base and token range stay in registers and are
  // read again only when the walk crosses into the next user (a workgroup's
  // range meets a few users), so a load waits on no scalar memory read.
  int lu = find_user(tile_base, L.R, ta);
  int32_t u_tile0 = tile_base[lu], u_tile1 = tile_base[lu + 1];
  int64_t u_first = offsets[lu], u_end = offsets[lu + 1];
  // the user's tiles that hold tokens, and the token count of the last one
  // (32-bit scalar arithmetic per tile)
  auto user_tiles = [&](int32_t& nt, int32_t& last) {
    const int64_t n_u = u_end - u_first;
    nt = (int32_t)((n_u + kTile - 1) / kTile);
    last = (int32_t)(n_u - (int64_t)(nt - 1) * kTile);
  };
  int32_t u_nt, u_last;
  user_tiles(u_nt, u_last);
  auto load = [&](int32_t tile, u32x4& raw, uint32_t& mb, bool& in, int32_t& cnt) {
    const bool live = tile < tb;               // uniform
    const int32_t tl = live ? tile : tb - 1;   // a tile of this workgroup
    if (tl >= u_tile1) {                       // uniform
      do ++lu; while (tl >= tile_base[lu + 1]);
      u_tile0 = tile_base[lu];
      u_tile1 = tile_base[lu + 1];
      u_first = offsets[lu];
      u_end = offsets[lu + 1];
      user_tiles(u_nt, u_last);
    }
    const int64_t first = u_first;
    const int32_t trel = tl - u_tile0;
    cnt = !live ? 0 : (trel < u_nt - 1 ? kTile : (trel == u_nt - 1 ? u_last : 0));
    const int64_t tok = first + (int64_t)trel * kTile + crow;
    in = live && conv && tok < u_end;
    const uint16_t* row = in ? H + tok * D : zrow;
    raw = reinterpret_cast<const u32x4*>(row)[cch];
    if constexpr (MASKED) mb = mask[in ? tok : first];
    else mb = 1u;
  };
  // Kept values outside fp16's finite range raise a device error bit once
  // the tiles are done.  Inside the loop only the chunk's squared norm is
  // tested (no branch): a kept value beyond 65504, or inf or NaN, makes it
  // exceed 65504^2 or NaN.  A wave that saw such a chunk reads its chunks
  // again after the loop and tests every value (a slow path that only
  // such inputs take).
  constexpr float kF16MaxSq = 65504.0f * 65504.0f;   // exact in fp32
  uint64_t range_sus = 0ull;
  uint32_t range_bad = 0u;
  // A buffer view of this workgroup's fp16 rows, tiles [ta, tb): the
  // hardware's range check drops the stores of conversions past the last
  // tile, so the row store needs no branch.
  const __amdgpu_buffer_rsrc_t h16_rows = __builtin_amdgcn_make_buffer_rsrc(
      h16 + (int64_t)ta * kTile * D, (short)0, n * kTile * D * 2, kBufferRsrcWord3);
  // the same for the -l pairs of tiles [ta, tb)
  const __amdgpu_buffer_rsrc_t nl_view =
      __builtin_amdgcn_make_buffer_rsrc(nl + (int64_t)ta * kTile, (short)0, n * kTile * 4, kBufferRsrcWord3);
  // widen, store to LDS buffer b and to the fp16 rows; keep words (masked
  // batches) and the per-wave "some logit may reach 100" bit.  A masked
  // token's row becomes zero here (whatever it held, NaN included).  Runs for every iteration,
  // past the last tile too (into a buffer nobody reads; the row store is
  // dropped), so that consuming the prefetched registers never sits behind
  // a branch.  The exact/fast decision needs a bound on each row's norm: CPR
  // times the largest squared norm of the row's 8-value chunks bounds it, so
  // no exchange between lanes is needed.  At d = 128 the body has no branch,
  // which lets it run interleaved with the previous tile's MFMAs.
  auto convert = [&](int32_t tile, int b, const u32x4& raw_in, uint32_t mb, bool in) {
    // unmasked: a slot without a token already holds the zero row
    const bool keep = MASKED ? in && mb != 0u : true;
    const u32x4 raw = !MASKED || keep ? raw_in : u32x4{0u, 0u, 0u, 0u};
    const half8 hv = bf16x8_to_f16x8(raw);
    float n2 = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // (the element goes through a named scalar: hipcc lowers a bit cast
      // taken directly from a vector element to a read of element 0)
      const uint32_t w = raw[i];
      const bf16x2 x = __builtin_bit_cast(bf16x2, w);
      n2 = __builtin_amdgcn_fdot2_f32_bf16(x, x, n2, false);
    }
    if (conv) {   // uniform: true for every thread at d = 128
      *reinterpret_cast<half8*>(&rows[b][crow * C::PITCH + 16 * cch]) = hv;
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, hv), h16_rows,
                                             ((tile - ta) * kTile + crow) * (D * 2) + 16 * cch, 0, 0);
      if constexpr (MASKED) {
        uint32_t* kw = cch == 0 ? &keep_words[b][crow] : &spare[tid];
        *kw = keep ? 1u : 0u;
      }
    }
    range_sus |= __ballot(!(n2 <= kF16MaxSq));
    const bool big = conv && keep && n2 >= lim2c;
    const uint32_t eb = __ballot(big) != 0ull ? 1u : 0u;   // uniform over the wave
    *(lane == 0 ? &exact_bytes[b][wave] : reinterpret_cast<uint8_t*>(&spare[tid])) = (uint8_t)eb;
  };

  // whether some wave flagged tile buffer b for the exact form
  auto tile_exact = [&](int b) {
    if constexpr (W == 8) return *reinterpret_cast<const uint64_t*>(&exact_bytes[b][0]) != 0ull;
    else return *reinterpret_cast<const uint32_t*>(&exact_bytes[b][0]) != 0u;
  };

  // partial of tile j (buffer b) into LDS slot j % 2
  const int hbase = col * C::PITCH + 16 * g;
  // exact form: fold one block's 16 logits into the running maximum m and
  // the sum p (rescaled when the maximum grows)
  auto exact_block = [&](const float16v& a, float& m, float& p) {
    float mb = a[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mb = fmaxf(mb, a[r]);
    const float mn = fmaxf(m, mb);
    p *= __builtin_amdgcn_exp2f(m - mn);
#pragma unroll
    for (int r = 0; r < 16; ++r) p += __builtin_amdgcn_exp2f(a[r] - mn);
    m = mn;
  };
  // the wave's partial (sum of 2^L, or its log2 in the exact form) of the
  // lane's token over its blocks, combined over the two lane halves
  auto block_partials = [&](bool exact, const float16v (&a)[NBW]) {
    if (!exact) {
      float p0 = 0.f, p1 = 0.f;
#pragma unroll
      for (int bl = 0; bl < NBW; ++bl)
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          p0 += __builtin_amdgcn_exp2f(a[bl][r]);
          p1 += __builtin_amdgcn_exp2f(a[bl][r + 1]);
        }
      const HalfPair hp = lane_halves(p0 + p1);
      return hp.lo + hp.hi;
    }
    float m = -INFINITY, p = 0.f;
#pragma unroll
    for (int bl = 0; bl < NBW; ++bl) exact_block(a[bl], m, p);
    const HalfPair hp = lane_halves(m + log2_normal(p));
    return log_add_exp2(hp.lo, hp.hi);
  };

  // `mid` (the next tile's conversion) runs after the first block's MFMAs
  // are issued, in the same basic block, so its VALU work fills the MFMA
  // pipeline's gaps instead of a phase of its own
  auto compute = [&](int j, int b, auto&& mid) {
    // the operand reads go out before the exact-mode bits are read, so the
    // two LDS round trips overlap
    half8 ha[C::S];
    if constexpr (NBW > 1) {
#pragma unroll
      for (int s = 0; s < C::S; ++s) ha[s] = *reinterpret_cast<const half8*>(&rows[b][hbase + 32 * s]);
    }
    const bool exact = tile_exact(b);
    float wpart;
    if constexpr (NBW == 1) {
      // one block: each 16-byte operand read (8 features of the lane's
      // token) feeds one MFMA as soon as it lands, so only a read or two is
      // live (under 128 registers: two workgroups share a CU)
      float16v a[NBW];
#pragma unroll
      for (int bl = 0; bl < NBW; ++bl) a[bl] = float16v{};
#pragma unroll
      for (int s = 0; s < C::S; ++s) {
        const half8 h = *reinterpret_cast<const half8*>(&rows[b][hbase + 32 * s]);
#pragma unroll
        for (int bl = 0; bl < NBW; ++bl) a[bl] = mfma32x32x16(qf[bl][s], h, a[bl]);
      }
      mid();
      wpart = block_partials(exact, a);
    } else {
      // block-major MFMA chains over the tile's operands held in registers:
      // the exponentials of block b run under the MFMAs of block b + 1.
      // A wave's issue priority falls block by block (NBW - 1 - b): of the
      // two waves sharing a SIMD, the one ahead yields to the one behind, so
      // both stay busy until the tile's end instead of the older wave
      // finishing first and the other running alone (measured: the two
      // waves' compute ends 0.2 instead of 1.5 thousand cycles apart).
      // Block 0's MFMAs and the conversion come before the branch on the
      // tile's form: with the conversion inside both branches the compiler
      // hoists it above them, ahead of the first MFMA.
      wave_priority(NBW - 1);
      float16v a0 = float16v{};
#pragma unroll
      for (int s = 0; s < C::S; ++s) a0 = mfma32x32x16(qf[0][s], ha[s], a0);
      mid();
      if (!exact) {
        float p0 = 0.f, p1 = 0.f;
#pragma unroll
        for (int bl = 0; bl < NBW; ++bl) {
          float16v a = a0;
          if (bl > 0) {
            wave_priority(NBW - 1 - bl);
            a = float16v{};
#pragma unroll
            for (int s = 0; s < C::S; ++s) a = mfma32x32x16(qf[bl][s], ha[s], a);
          }
#pragma unroll
          for (int r = 0; r < 16; r += 2) {
            p0 += __builtin_amdgcn_exp2f(a[r]);
            p1 += __builtin_amdgcn_exp2f(a[r + 1]);
          }
        }
        const HalfPair hp = lane_halves(p0 + p1);
        wpart = hp.lo + hp.hi;
      } else {
        float m = -INFINITY, p = 0.f;
#pragma unroll
        for (int bl = 0; bl < NBW; ++bl) {
          float16v a = a0;
          if (bl > 0) {
            wave_priority(NBW - 1 - bl);
            a = float16v{};
#pragma unroll
            for (int s = 0; s < C::S; ++s) a = mfma32x32x16(qf[bl][s], ha[s], a);
          }
          exact_block(a, m, p);
        }
        const HalfPair hp = lane_halves(m + log2_normal(p));
        wpart = log_add_exp2(hp.lo, hp.hi);
      }
    }
    // both lane halves hold the same value; the upper half's store is spare
    float* pw = g == 0 ? &part[j & 1][col][wave] : reinterpret_cast<float*>(&spare[tid]);
    *pw = wpart;
    return exact;
  };

  // -l pairs of tile j (buffer b) from its W partials.  Only the first
  // W / 2 waves finalize, TPW = kTile / (W / 2) tokens each.
  // Waves w and w + W / 2 share a SIMD, and the first of the pair, which the
  // arbiter favours at equal priority, finishes its MFMAs before the second;
  // its finalize then partly fills that gap instead of lengthening the
  // second wave's path to the next barrier (measured faster than a finalize
  // spread over all waves).
  auto finalize = [&](int j, int b, bool exact, int32_t cnt) {
    constexpr int FW = W / 2;
    constexpr int TPW = kTile / FW;   // tokens per finalizing wave
    static_assert(TPW * FW == kTile && TPW <= 64, "tokens per wave");
    if (wave >= FW) return;           // uniform
    // every lane works (no branch): lanes with equal lane % TPW store the
    // same value to the same word
    const int tok = wave * TPW + (lane % TPW);
    bool keep;
    if constexpr (MASKED) keep = keep_words[b][tok] != 0u;
    else keep = tok < cnt;
    const float* pp = part[j & 1][tok];
    float lse;
    if (!exact) {
      float s = 0.f;
#pragma unroll
      for (int w = 0; w < W; ++w) s += pp[w];
      lse = log2_normal(s);
    } else {
      lse = -INFINITY;
#pragma unroll
      for (int w = 0; w < W; ++w) lse = log_add_exp2(lse, pp[w]);
    }
    // -l = 14 - lse as an fp16 pair (hi, lo) with hi + lo = -l to ~2^-16
    const float nlv = keep ? kAllocShift - lse : -60000.0f;
    const _Float16 hi = (_Float16)nlv;
    const _Float16 lo = keep ? (_Float16)(nlv - (float)hi) : (_Float16)0.0f;
    const half2v pr = {hi, lo};
    // lanes past TPW computed duplicates: their byte offset lies past the
    // view's end, so the hardware drops their stores
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, pr), nl_view,
                                          lane < TPW ? (j * kTile + tok) * 4 : 0x7FFFFFF0, 0, 0);
  };

  // prologue: tiles 0 and 1 loaded, tile 0 converted into buffer 0
  u32x4 raw[2];
  uint32_t mb[2];
  bool in[2];
  int32_t cnt[2];
  load(ta, raw[0], mb[0], in[0], cnt[0]);
  load(ta + 1, raw[1], mb[1], in[1], cnt[1]);
  convert(ta, 0, raw[0], mb[0], in[0]);
  // token counts of the tiles being finalized and computed
  int32_t cnt_fin = 0, cnt_cmp = cnt[0];
  load(ta + 2, raw[0], mb[0], in[0], cnt[0]);

  // iteration j: compute tile j with the conversion of tile j + 1 (loaded two
  // iterations ago) into buffer (j + 1) % 3 interleaved, finalize tile j - 1,
  // then load tile j + 3.  The wait for tile j + 1's registers counts vector memory
  // operations in issue order; with the newest load the last one issued
  // before it, that load stays in flight across the wait.
  // exact-mode decision of the previous tile, for its finalize
  bool ex_prev = false;
  auto iteration = [&](int j, auto oddc) {
    constexpr int R = decltype(oddc)::value;   // raw slot of tile j + 1
    lds_barrier();
    const int b = j % kBufs;
    const bool ex = compute(j, b, [&] { convert(ta + j + 1, (j + 1) % kBufs, raw[R], mb[R], in[R]); });
    if (j >= 1) finalize(j - 1, (j + kBufs - 1) % kBufs, ex_prev, cnt_fin);
    ex_prev = ex;
    cnt_fin = cnt_cmp;
    cnt_cmp = cnt[R];
    load(ta + j + 3, raw[R], mb[R], in[R], cnt[R]);
  };
  int j = 0;
  for (; j + 1 < n; j += 2) {
    iteration(j, std::integral_constant<int, 1>{});
    iteration(j + 1, std::integral_constant<int, 0>{});
  }
  if (j < n) iteration(j, std::integral_constant<int, 1>{});
  lds_barrier();
  finalize(n - 1, (n - 1) % kBufs, ex_prev, cnt_fin);
  if (range_sus != 0ull) {   // uniform over the wave
    lu = find_user(tile_base, L.R, ta);
    u_tile0 = tile_base[lu];
    u_tile1 = tile_base[lu + 1];
    u_first = offsets[lu];
    u_end = offsets[lu + 1];
    user_tiles(u_nt, u_last);
    for (int32_t t = ta; t < tb; ++t) {
      u32x4 r;
      uint32_t m;
      bool i;
      int32_t c;
      load(t, r, m, i, c);
      if (i && m != 0u) range_bad |= bf16x8_range_bits(r);
    }
  }
  if (__ballot(range_bad != 0u) != 0ull && lane == 0) atomicOr(ws_i32(ws, L.off_hdr) + kHdrErr, kErrRange);
}

bool pass1q_ok(const Layout& L) {
  return L.dtype == 0 && (L.d == 64 || L.d == 128) && (L.k == 256 || L.k == 512 || L.k == 1024);
}

hipError_t launch_pass1q(const Layout& L, const void* H, const int64_t* offsets, const uint8_t* mask, void* ws,
                         hipStream_t stream) {
  // 8 waves x k/8 prototypes.  At k = 256 (under 128 registers) two
  // workgroups share a CU: four waves per SIMD, with independent barriers,
  // hide the exponentials and row conversion that two waves per SIMD leave
  // exposed (measured 24% faster).  Sixteen-wave workgroups were slower: one
  // barrier per tile across 16 waves, and half of them idle in the
  // conversion.
  const int per_cu = L.k == 256 ? 2 : 1;
  const int grid = L.tiles_max < kWGs * per_cu ? L.tiles_max : kWGs * per_cu;
  if (grid == 0) return hipSuccess;
  const int32_t* tile_base = reinterpret_cast<const int32_t*>(static_cast<char*>(ws) + L.off_tile_base);
#define SA_P1Q(DD, NN, WW)                                                                                 \
  do {                                                                                                     \
    if (mask != nullptr)                                                                                   \
      hipLaunchKernelGGL((pass1_qres<DD, NN, true, WW>), dim3(grid), dim3(WW * 64), 0, stream,            \
                         (const uint16_t*)H, offsets, mask, tile_base, L, ws);                             \
    else                                                                                                   \
      hipLaunchKernelGGL((pass1_qres<DD, NN, false, WW>), dim3(grid), dim3(WW * 64), 0, stream,           \
                         (const uint16_t*)H, offsets, mask, tile_base, L, ws);                             \
  } while (0)
  if (L.d == 128) {
    if (L.k == 256) SA_P1Q(128, 1, 8);
    else if (L.k == 512) SA_P1Q(128, 2, 8);
    else SA_P1Q(128, 4, 8);
  } else {
    if (L.k == 256) SA_P1Q(64, 1, 8);
    else if (L.k == 512) SA_P1Q(64, 2, 8);
    else SA_P1Q(64, 4, 8);
  }
#undef SA_P1Q
  return hipGetLastError();
}

}  // namespace sa
