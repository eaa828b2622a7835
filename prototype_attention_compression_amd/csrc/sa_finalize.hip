// sa_finalize.hip — chunk reduction and prototype-wise normalisation.
//
// For user u and a block of 32 prototypes, sums the partials
// U_c[j, :] = sum_t A[j,t] h_t and m_c[j] over the user's partial slots in
// slot order (a fixed order: the result is bitwise repeatable), then writes
//     S_u[j, :] = (U[j, :] / m_j) Wv,   mass[u, j] = m_j
// i.e. the mass-normalised allocation-weighted mean of the value rows
// v_t = h_t Wv (SequenceO1 blog "How it works" item 1: the k x d sketch of
// softly assigned items; the division by the prototype's total mass is the
// prototype-wise normalisation read as a weighted mean).  Applying Wv after
// the reduction equals summing A v_t because the projection is linear.  A
// prototype with zero mass (every allocation underflowed, or an empty user)
// gets a zero row.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "sa_device.h"
#include "sa_launch.h"
#include "sa_slots.h"

namespace sa {

namespace {
constexpr int kSlotBatch = 4;   // partial slots whose loads are in flight together
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
}  // namespace

template <typename T>
__device__ __forceinline__ float wv_value(T v);
template <>
__device__ __forceinline__ float wv_value<uint16_t>(uint16_t v) {
  return __uint_as_float(((uint32_t)v) << 16);
}
template <>
__device__ __forceinline__ float wv_value<float>(float v) {
  return v;
}

// One workgroup = one user and kFinRows prototypes.  Wv (D x D) is staged in
// LDS once per workgroup with all of its 16-byte loads in flight together, and
// the partial slots are read kSlotBatch at a time (the sums still run in slot
// order): both loops would otherwise wait on one global load per step.
template <int D, typename T>
__global__ __launch_bounds__(256) void finalize(const T* __restrict__ Wv, Layout L, void* ws, float* __restrict__ S,
                                                float* __restrict__ mass, float* __restrict__ Sbar,
                                                float mass_scale, int presummed) {
  constexpr int PER = kFinRows * D / 256;   // elements per thread
  constexpr int RPI = 256 / D;              // rows per output pass
  constexpr int WCH = D * D * (int)sizeof(T) / 16 / 256;   // 16-byte chunks of Wv per thread
  static_assert(WCH * 256 * 16 == D * D * (int)sizeof(T), "whole chunks");
  constexpr bool kMfma = std::is_same<T, uint16_t>::value;
  // bf16 Wv: staged transposed, Wv^T[n][k] with a padded pitch, as the B
  // operand of the value projection on MFMAs; fp32 Wv: staged as it is
  constexpr int WP = kMfma ? D + 8 : D;
  __shared__ float sh[kFinRows][D + 1];
  __shared__ float ms[kFinRows];
  __shared__ __attribute__((aligned(16))) T wsh[D * WP];
  const int nrb = L.k / kFinRows;
  const int u = blockIdx.x / nrb, rb = blockIdx.x % nrb;
  const int j0 = rb * kFinRows;
  const int tid = threadIdx.x;
  {
    u32x4 w[WCH];
    if constexpr (kMfma) {
      // thread chunk i: row k = q % D, columns n0 .. n0 + 7 (n0 = 8 (q / D)),
      // so the lanes of a wave write consecutive k of one transposed row:
      // no LDS bank conflicts
#pragma unroll
      for (int i = 0; i < WCH; ++i) {
        const int q = tid + 256 * i, k = q % D, n0 = 8 * (q / D);
        w[i] = reinterpret_cast<const u32x4*>(Wv)[k * (D / 8) + n0 / 8];
      }
#pragma unroll
      for (int i = 0; i < WCH; ++i) {
        const int q = tid + 256 * i, k = q % D, n0 = 8 * (q / D);
#pragma unroll
        for (int e = 0; e < 8; ++e)
          wsh[(n0 + e) * WP + k] = (uint16_t)(w[i][e >> 1] >> (16 * (e & 1)));
      }
    } else {
#pragma unroll
      for (int i = 0; i < WCH; ++i) w[i] = reinterpret_cast<const u32x4*>(Wv)[tid + 256 * i];
#pragma unroll
      for (int i = 0; i < WCH; ++i) reinterpret_cast<u32x4*>(wsh)[tid + 256 * i] = w[i];
    }
  }
  // the user's partial-sum slots, or the heads of their pre-summed
  // sub-ranges (sa_slots.h), added in slot order
  int c0, c1;
  user_slots(L, ws, u, c0, c1);
  const int n = c1 - c0;
  const bool pre = presummed && n > kPreMin;
  const float* part_u = ws_f32(ws, L.off_part_u);
  const float* part_m = ws_f32(ws, L.off_part_m);

  // thread tid owns the 16-byte pieces tid + 256 i (i < V4) of the 32-row
  // block: elements 4 (tid + 256 i) .. + 3, one 16-byte load per piece
  constexpr int V4 = PER / 4;
  static_assert(V4 * 4 == PER, "whole pieces");
  f32x4 acc[V4];
#pragma unroll
  for (int i = 0; i < V4; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto slot_block = [&](int c) {
    return reinterpret_cast<const f32x4*>(part_u + ((int64_t)c * L.k + j0) * D);
  };
  if (pre) {
    f32x4 v[kPreSplit][V4];
#pragma unroll
    for (int q = 0; q < kPreSplit; ++q) {
      const f32x4* base = slot_block(sub_head(c0, n, q));
#pragma unroll
      for (int i = 0; i < V4; ++i) v[q][i] = base[tid + 256 * i];
    }
#pragma unroll
    for (int q = 0; q < kPreSplit; ++q)
#pragma unroll
      for (int i = 0; i < V4; ++i) acc[i] += v[q][i];
  } else {
    int c = c0;
    for (; c + kSlotBatch <= c1; c += kSlotBatch) {
      f32x4 v[kSlotBatch][V4];
#pragma unroll
      for (int q = 0; q < kSlotBatch; ++q) {
        const f32x4* base = slot_block(c + q);
#pragma unroll
        for (int i = 0; i < V4; ++i) v[q][i] = base[tid + 256 * i];
      }
#pragma unroll
      for (int q = 0; q < kSlotBatch; ++q)
#pragma unroll
        for (int i = 0; i < V4; ++i) acc[i] += v[q][i];
    }
    for (; c < c1; ++c) {
      const f32x4* base = slot_block(c);
#pragma unroll
      for (int i = 0; i < V4; ++i) acc[i] += base[tid + 256 * i];
    }
  }
  if (tid < kFinRows) {
    float m = 0.f;
    if (pre) {
      for (int q = 0; q < kPreSplit; ++q) m += part_m[(int64_t)sub_head(c0, n, q) * L.k + j0 + tid];
    } else {
      for (int cc = c0; cc < c1; ++cc) m += part_m[(int64_t)cc * L.k + j0 + tid];
    }
    ms[tid] = m;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < V4; ++i) {
    const int e = 4 * (tid + 256 * i), j = e / D, a = e % D;   // one row per piece (D % 4 == 0)
    const float m = ms[j];
    f32x4 v;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      v[c] = m > 0.f ? acc[i][c] / m : 0.f;
      sh[j][a + c] = v[c];
    }
    if (Sbar != nullptr)   // the mass-normalised rows
      *reinterpret_cast<f32x4*>(Sbar + ((int64_t)u * L.k + j0) * D + e) = v;
  }
  __syncthreads();
  float* dst = S + ((int64_t)u * L.k + j0) * D;
  if constexpr (kMfma) {
    // S rows = Sbar rows x Wv: wave w takes output columns 32 w .. 32 w + 31
    // (D = 64: waves 0 and 1).  Wv is exact in bf16; each fp32 Sbar value is
    // split into three bf16 terms hi + mid + lo (24 significant bits, as
    // fp32), so the products carry fp32 accuracy with fp32 sums.
    const int lane = tid & 63, wave = tid >> 6, col = lane & 31, g = lane >> 5;
    if (32 * wave < D) {   // uniform over the wave
      float16v acc = float16v{};
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        const int k0 = 16 * ks + 8 * g;
        bf16x8 hi, mid, lo;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float x = sh[col][k0 + e];
          const __bf16 h = (__bf16)x;
          const float r1 = x - (float)h;
          const __bf16 m1 = (__bf16)r1;
          hi[e] = h;
          mid[e] = m1;
          lo[e] = (__bf16)(r1 - (float)m1);
        }
        const bf16x8 b = *reinterpret_cast<const bf16x8*>(&wsh[(32 * wave + col) * WP + k0]);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(hi, b, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(mid, b, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lo, b, acc, 0, 0, 0);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) dst[(int64_t)acc_row(r, g) * D + 32 * wave + col] = acc[r];
    }
  } else {
    const int cl = tid % D, jr = tid / D;
    float out[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) out[i] = 0.f;
#pragma unroll 4
    for (int a = 0; a < D; ++a) {
      const float w = wv_value<T>(wsh[a * D + cl]);
#pragma unroll
      for (int i = 0; i < PER; ++i) out[i] = fmaf(sh[jr + RPI * i][a], w, out[i]);
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) dst[(int64_t)(jr + RPI * i) * D + cl] = out[i];
  }
  if (mass != nullptr && tid < kFinRows) mass[(int64_t)u * L.k + j0 + tid] = ms[tid] * mass_scale;
}

// Pre-reduction for users with many slots: workgroup (user, 32-row block,
// sub-range s) adds the slots of sub-range s in order and writes the sum to
// the sub-range's first slot (sub-ranges are disjoint, so workgroups never
// touch each other's slots).
template <int D>
__global__ __launch_bounds__(256) void presum_slots(Layout L, void* ws) {
  constexpr int PER = kFinRows * D / 256;
  const int nrb = L.k / kFinRows;
  const int sidx = blockIdx.x % kPreSplit, ub = blockIdx.x / kPreSplit;
  const int u = ub / nrb, rb = ub % nrb;
  const int j0 = rb * kFinRows;
  const int tid = threadIdx.x;
  int c0, c1;
  user_slots(L, ws, u, c0, c1);
  const int n = c1 - c0;
  if (n <= kPreMin) return;   // uniform over the workgroup
  const int a = sub_head(c0, n, sidx), b = sub_head(c0, n, sidx + 1);
  float* part_u = ws_f32(ws, L.off_part_u);
  float* part_m = ws_f32(ws, L.off_part_m);
  // 16-byte pieces tid + 256 i of the 32-row block, as in finalize
  constexpr int V4 = PER / 4;
  static_assert(V4 * 4 == PER, "whole pieces");
  auto slot_block = [&](int c) { return reinterpret_cast<f32x4*>(part_u + ((int64_t)c * L.k + j0) * D); };
  f32x4 acc[V4];
#pragma unroll
  for (int i = 0; i < V4; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  int c = a;
  for (; c + kSlotBatch <= b; c += kSlotBatch) {
    f32x4 v[kSlotBatch][V4];
#pragma unroll
    for (int q = 0; q < kSlotBatch; ++q) {
      const f32x4* base = slot_block(c + q);
#pragma unroll
      for (int i = 0; i < V4; ++i) v[q][i] = base[tid + 256 * i];
    }
#pragma unroll
    for (int q = 0; q < kSlotBatch; ++q)
#pragma unroll
      for (int i = 0; i < V4; ++i) acc[i] += v[q][i];
  }
  for (; c < b; ++c) {
    const f32x4* base = slot_block(c);
#pragma unroll
    for (int i = 0; i < V4; ++i) acc[i] += base[tid + 256 * i];
  }
  float m = 0.f;
  if (tid < kFinRows)
    for (int cc = a; cc < b; ++cc) m += part_m[(int64_t)cc * L.k + j0 + tid];
  __syncthreads();   // every read of slot a is done before it is overwritten
  f32x4* dst = slot_block(a);
#pragma unroll
  for (int i = 0; i < V4; ++i) dst[tid + 256 * i] = acc[i];
  if (tid < kFinRows) part_m[(int64_t)a * L.k + j0 + tid] = m;
}

hipError_t launch_presum(const Layout& L, void* ws, hipStream_t stream) {
  if (!presum_launch(L)) return hipSuccess;
  const int64_t grid = (int64_t)L.R * (L.k / kFinRows) * kPreSplit;
  if (L.d == 128)
    hipLaunchKernelGGL((presum_slots<128>), dim3((unsigned)grid), dim3(256), 0, stream, L, ws);
  else
    hipLaunchKernelGGL((presum_slots<64>), dim3((unsigned)grid), dim3(256), 0, stream, L, ws);
  return hipGetLastError();
}

hipError_t launch_finalize(const Layout& L, const void* Wv, void* ws, float* S, float* mass, float* Sbar,
                           hipStream_t stream) {
  const int64_t grid = (int64_t)L.R * (L.k / kFinRows);
  if (grid == 0) return hipSuccess;
  const int pre = presum_launch(L) ? 1 : 0;
  if (pre && launch_presum(L, ws, stream) != hipSuccess) return hipErrorLaunchFailure;
  if (L.dtype == 0) {
    const float scale = 1.0f / 16384.0f;  // allocations were scaled by 2^14
    if (L.d == 128)
      hipLaunchKernelGGL((finalize<128, uint16_t>), dim3((unsigned)grid), dim3(256), 0, stream,
                         (const uint16_t*)Wv, L, ws, S, mass, Sbar, scale, pre);
    else
      hipLaunchKernelGGL((finalize<64, uint16_t>), dim3((unsigned)grid), dim3(256), 0, stream,
                         (const uint16_t*)Wv, L, ws, S, mass, Sbar, scale, pre);
  } else {
    if (L.d == 128)
      hipLaunchKernelGGL((finalize<128, float>), dim3((unsigned)grid), dim3(256), 0, stream, (const float*)Wv, L,
                         ws, S, mass, Sbar, 1.0f, pre);
    else
      hipLaunchKernelGGL((finalize<64, float>), dim3((unsigned)grid), dim3(256), 0, stream, (const float*)Wv, L,
                         ws, S, mass, Sbar, 1.0f, pre);
  }
  return hipGetLastError();
}

}  // namespace sa
