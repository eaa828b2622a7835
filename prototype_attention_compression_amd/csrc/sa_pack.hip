// sa_pack.hip — token packing for the one-pass FlashSA path (bf16 inputs).
//
// Writes every tile of every user in the form the one-pass kernel streams:
//   * the fp16 token rows (bf16 widened exactly; masked tokens and the
//     padding rows of a user's last tiles are zero, so NaN in a dropped row
//     cannot reach the sums — a dropped token takes no part at all, as the
//     per-token softmax over prototypes of the SequenceO1 blog, "How it
//     works" item 1, is only defined for kept history items);
//   * one word per token: 1 if it takes part, else 0;
//   * the largest row norm |h_t| of a kept token (header word), which with
//     the largest query norm bounds every logit (Cauchy-Schwarz) and picks
//     the exponent-range mode of the one-pass kernel.
// Memory-bound: 2 bytes read and 2 written per element.  A persistent grid
// of at most kPackWGs workgroups walks contiguous tile ranges (the user of a
// tile advances monotonically, no search per tile) and raises the norm
// maximum with one atomic per workgroup.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "sa_device.h"
#include "sa_launch.h"

namespace sa {

namespace {
constexpr int kPackWGs = 2048;
}

template <int D>
__global__ __launch_bounds__(256) void pack_rows(const uint16_t* __restrict__ H, const int64_t* __restrict__ offsets,
                                                 const uint8_t* __restrict__ mask, Layout L, void* ws) {
  constexpr int CPR = D / 8;                 // 16-byte chunks per row
  constexpr int PER = kTile * CPR / 256;     // chunks per thread per tile (2 or 1)
  __shared__ float red[4];
  int32_t* hdr = ws_i32(ws, L.off_hdr);
  const int32_t T = hdr[kHdrTiles];
  const int32_t per_wg = (T + gridDim.x - 1) / gridDim.x;
  const int32_t ta = blockIdx.x * per_wg;
  const int32_t tb = min(T, ta + per_wg);
  const int tid = threadIdx.x;
  float nmax = 0.f;
  uint32_t range_bad = 0u;   // kept values outside fp16's finite range
  if (ta < tb) {
    const int32_t* tile_base = ws_i32(ws, L.off_tile_base);
    _Float16* h16 = ws_f16(ws, L.off_h16);
    uint32_t* valid = reinterpret_cast<uint32_t*>(ws_i32(ws, L.off_nl));
    int u = find_user(tile_base, L.R, ta);
    int32_t ub = tile_base[u + 1];
    for (int32_t tile = ta; tile < tb; ++tile) {
      while (tile >= ub) {   // uniform: the next user with tiles
        ++u;
        ub = tile_base[u + 1];
      }
      const int64_t tok0 = offsets[u] + (int64_t)(tile - tile_base[u]) * kTile;
      const int64_t tok1 = offsets[u + 1];
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int q = tid + 256 * i;
        const int row = q / CPR, c = q % CPR;
        const int64_t tok = tok0 + row;
        u32x4 raw = {0u, 0u, 0u, 0u};
        bool keep = false;
        if (tok < tok1) {
          keep = (mask == nullptr) || (mask[tok] != 0);
          if (keep) raw = reinterpret_cast<const u32x4*>(H + tok * D)[c];
        }
        range_bad |= bf16x8_range_bits(raw);
        const half8 hv = bf16x8_to_f16x8(raw);
        *reinterpret_cast<half8*>(h16 + ((int64_t)tile * kTile + row) * D + 8 * c) = hv;
        if (c == 0) valid[(int64_t)tile * kTile + row] = keep ? 1u : 0u;
        // squared norm of the fp16 row: its CPR chunks are CPR consecutive
        // lanes of one wave (CPR divides 64)
        float n2 = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float v = (float)hv[e];
          n2 = fmaf(v, v, n2);
        }
#pragma unroll
        for (int o = 1; o < CPR; o <<= 1) n2 += __shfl_xor(n2, o);
        nmax = fmaxf(nmax, n2);
      }
    }
  }
  if (__ballot(range_bad != 0u) != 0ull && (tid & 63) == 0) atomicOr(hdr + kHdrErr, kErrRange);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) nmax = fmaxf(nmax, __shfl_xor(nmax, o));
  if ((tid & 63) == 0) red[tid >> 6] = nmax;
  __syncthreads();
  // non-negative floats order like their bit patterns
  if (tid == 0) {
    const float m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    if (m > 0.f) atomicMax(hdr + kHdrHmax, __float_as_int(sqrtf(m)));
  }
}

hipError_t launch_pack(const Layout& L, const void* H, const int64_t* offsets, const uint8_t* mask, void* ws,
                       hipStream_t stream) {
  const int grid = L.tiles_max < kPackWGs ? L.tiles_max : kPackWGs;
  if (grid == 0) return hipSuccess;
  if (L.d == 128)
    hipLaunchKernelGGL(pack_rows<128>, dim3(grid), dim3(256), 0, stream, (const uint16_t*)H, offsets, mask, L, ws);
  else
    hipLaunchKernelGGL(pack_rows<64>, dim3(grid), dim3(256), 0, stream, (const uint16_t*)H, offsets, mask, L, ws);
  return hipGetLastError();
}

}  // namespace sa
