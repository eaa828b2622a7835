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
//     magnitudes in [2^-17, 65504]), written to LDS and to the fp16 row
//     buffer pass 2 reads; masked tokens and padding rows are zero.  The row
//     norms decide, per tile, whether any logit can reach |L| >= 100
//     (Cauchy-Schwarz with the largest query norm): then the tile takes the
//     exact form (running maximum, rescaled sums), else plain sums of 2^L;
//   * compute (each wave: its k/8 prototypes, NBW blocks of 32): 8 16-byte
//     operand reads, NBW x 8 fp16 MFMAs (lane = token, so the sum over
//     prototypes stays in the lane), exponentials and sums;
//   * every wave turns 4 tokens of the previous tile from 8 partials into
//     -l pairs.
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

__device__ __forceinline__ float log_add_exp2(float a, float b) {
  const float m = fmaxf(a, b);
  if (m == -INFINITY) return -INFINITY;
  return m + log2f(__builtin_amdgcn_exp2f(a - m) + __builtin_amdgcn_exp2f(b - m));
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
  __shared__ __attribute__((aligned(16))) uint32_t exact_bits[kBufs][W];
  __shared__ uint32_t keep_words[kBufs][kTile];

  const int32_t* hdr = ws_i32(ws, L.off_hdr);
  const int32_t T = hdr[kHdrTiles];
  const int32_t per = (T + gridDim.x - 1) / gridDim.x;
  const int32_t ta = blockIdx.x * per;
  const int32_t tb = min(T, ta + per);
  if (ta >= tb) return;  // uniform
  const int n = tb - ta;
  const float qmax = __int_as_float(hdr[kHdrQmax]);
  const float lim2 = 10000.0f / fmaxf(qmax * qmax, 1e-30f);   // |h|^2 >= lim2  <=>  qmax |h| >= 100

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

  // conversion role of this thread: chunk q of a tile (row q / CPR, chunk q % CPR)
  const bool conv = tid < C::CHUNKS;
  const int crow = tid / C::CPR, cch = tid % C::CPR;
  // Forward walk over the tiles being loaded (tile index increases).  The
  // user lookup reads only kernel arguments the kernel never writes, so it
  // compiles to scalar loads.  The row chunk (and mask byte) load is issued
  // unconditionally from an address clamped into the same user's rows, with
  // whether the slot is live kept aside: no load sits behind a branch, so
  // the compiler's wait before the conversion two tiles later counts only
  // what was issued after it instead of draining the prefetches and stores.
  int lu = find_user(tile_base, L.R, ta);
  auto load = [&](int32_t tile, u32x4& raw, uint32_t& mb, bool& in) {
    const bool live = tile < tb;               // uniform
    const int32_t tl = live ? tile : tb - 1;   // a tile of this workgroup
    while (tl >= tile_base[lu + 1]) ++lu;      // uniform
    const int64_t t0 = offsets[lu] + (int64_t)(tl - tile_base[lu]) * kTile;
    const int64_t tok = t0 + crow;
    in = live && conv && tok < offsets[lu + 1];
    const int64_t tc = in ? tok : t0;          // t0 is a token of user lu
    raw = reinterpret_cast<const u32x4*>(H + tc * D)[cch];
    if constexpr (MASKED) mb = mask[tc];
    else mb = 1u;
  };
  // widen, store to LDS buffer b and to the fp16 rows; keep words and the
  // per-wave "some logit may reach 100" bit.  A dropped token's row becomes
  // zero here (whatever it held, NaN included).  Runs for every iteration,
  // past the last tile too (into a buffer nobody reads, no global store), so
  // that consuming the prefetched registers never sits behind a branch.
  auto convert = [&](int32_t tile, int b, const u32x4& raw_in, uint32_t mb, bool in) {
    const bool keep = in && mb != 0u;
    const u32x4 raw = keep ? raw_in : u32x4{0u, 0u, 0u, 0u};
    const half8 hv = bf16x8_to_f16x8(raw);
    float n2 = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float v = (float)hv[e];
      n2 = fmaf(v, v, n2);
    }
#pragma unroll
    for (int o = 1; o < C::CPR; o <<= 1) n2 += __shfl_xor(n2, o);
    if (conv) {
      *reinterpret_cast<half8*>(&rows[b][crow * C::PITCH + 16 * cch]) = hv;
      if (tile < tb) *reinterpret_cast<half8*>(h16 + ((int64_t)tile * kTile + crow) * D + 8 * cch) = hv;
      if (cch == 0) keep_words[b][crow] = keep ? 1u : 0u;
    }
    const bool big = conv && keep && n2 >= lim2;
    const uint64_t bal = __ballot(big);
    if (lane == 0) exact_bits[b][wave] = bal != 0 ? 1u : 0u;
  };

  // whether some wave flagged tile buffer b for the exact form
  auto tile_exact = [&](int b) {
    uint32_t any = 0u;
#pragma unroll
    for (int w = 0; w < W; w += 4) {
      const u32x4 e = *reinterpret_cast<const u32x4*>(&exact_bits[b][w]);
      any |= e[0] | e[1] | e[2] | e[3];
    }
    return any != 0u;
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
    const HalfPair hp = lane_halves(m + log2f(p));
    return log_add_exp2(hp.lo, hp.hi);
  };

  auto compute = [&](int j, int b) {
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
      wpart = block_partials(exact, a);
    } else {
      // block-major MFMA chains over the tile's operands held in registers:
      // the exponentials of block b run under the MFMAs of block b + 1
      half8 ha[C::S];
#pragma unroll
      for (int s = 0; s < C::S; ++s) ha[s] = *reinterpret_cast<const half8*>(&rows[b][hbase + 32 * s]);
      if (!exact) {
        float p0 = 0.f, p1 = 0.f;
#pragma unroll
        for (int bl = 0; bl < NBW; ++bl) {
          float16v a = float16v{};
#pragma unroll
          for (int s = 0; s < C::S; ++s) a = mfma32x32x16(qf[bl][s], ha[s], a);
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
          float16v a = float16v{};
#pragma unroll
          for (int s = 0; s < C::S; ++s) a = mfma32x32x16(qf[bl][s], ha[s], a);
          exact_block(a, m, p);
        }
        const HalfPair hp = lane_halves(m + log2f(p));
        wpart = log_add_exp2(hp.lo, hp.hi);
      }
    }
    if (g == 0) part[j & 1][col][wave] = wpart;
  };

  // -l pairs of tile j (buffer b) from its 8 partials: wave w, lanes 0..3,
  // tokens 4 w .. 4 w + 3
  auto finalize = [&](int j, int b) {
    constexpr int TPW = kTile / W;   // tokens per wave
    if (lane >= TPW) return;
    const int tok = wave * TPW + lane;
    const bool exact = tile_exact(b);
    const float* pp = part[j & 1][tok];
    float lse;
    if (!exact) {
      float s = 0.f;
#pragma unroll
      for (int w = 0; w < W; ++w) s += pp[w];
      lse = log2f(s);
    } else {
      lse = -INFINITY;
#pragma unroll
      for (int w = 0; w < W; ++w) lse = log_add_exp2(lse, pp[w]);
    }
    const bool keep = keep_words[b][tok] != 0u;
    // -l = 14 - lse as an fp16 pair (hi, lo) with hi + lo = -l to ~2^-16
    const float nlv = keep ? kAllocShift - lse : -60000.0f;
    const _Float16 hi = (_Float16)nlv;
    const _Float16 lo = keep ? (_Float16)(nlv - (float)hi) : (_Float16)0.0f;
    const half2v pr = {hi, lo};
    nl[(int64_t)(ta + j) * kTile + tok] = __builtin_bit_cast(uint32_t, pr);
  };

  // prologue: tiles 0 and 1 loaded, tile 0 converted into buffer 0
  u32x4 raw[2];
  uint32_t mb[2];
  bool in[2];
  load(ta, raw[0], mb[0], in[0]);
  load(ta + 1, raw[1], mb[1], in[1]);
  convert(ta, 0, raw[0], mb[0], in[0]);
  load(ta + 2, raw[0], mb[0], in[0]);

  // iteration j: convert tile j + 1 (loaded two iterations ago) into buffer
  // (j + 1) % 3, finalize tile j - 1, compute tile j, then load tile j + 3.  The wait for tile j + 1's registers counts vector memory
  // operations in issue order; with the newest load the last one issued
  // before it, that load stays in flight across the wait.
  auto iteration = [&](int j, auto oddc) {
    constexpr int R = decltype(oddc)::value;   // raw slot of tile j + 1
    lds_barrier();
    const int b = j % kBufs;
    convert(ta + j + 1, (j + 1) % kBufs, raw[R], mb[R], in[R]);
    if (j >= 1) finalize(j - 1, (j + kBufs - 1) % kBufs);
    compute(j, b);
    load(ta + j + 3, raw[R], mb[R], in[R]);
  };
  int j = 0;
  for (; j + 1 < n; j += 2) {
    iteration(j, std::integral_constant<int, 1>{});
    iteration(j + 1, std::integral_constant<int, 0>{});
  }
  if (j < n) iteration(j, std::integral_constant<int, 1>{});
  lds_barrier();
  finalize(n - 1, (n - 1) % kBufs);
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
