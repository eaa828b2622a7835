// sa_probe.hip — a measurement helper beside the compression kernels: a loop
// of fp16 32x32x16 MFMAs with no memory traffic, timed by the caller.  It
// shows how fast the matrix cores of this part run on a given kind of operand
// data.  The part is power-limited, so its clock under load, and with it the
// MFMA rate, depends on how many operand bits toggle: the rate on random data
// is the practical ceiling for the sketch kernels, whose operands are token
// rows and queries.
//
// 512 workgroups of 4 waves (two waves per SIMD on 256 CUs).  Each wave runs
// `iters` x 8 MFMAs over four independent accumulator chains, with its
// operands in 8 register pairs, so consecutive instructions read different
// data.  Operand kinds: 0 zeros, 1 one constant value (1/64), 2 uniform
// values in [-1, 1) drawn per lane and register from a 32-bit integer hash
// (the finalising mix of MurmurHash3, Appleby).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sa.h"
#include "sa_device.h"

namespace sa {

namespace {

constexpr int kProbeWGs = 512;

__device__ __forceinline__ uint32_t mix32(uint32_t x) {
  x ^= x >> 16;
  x *= 0x85ebca6bu;
  x ^= x >> 13;
  x *= 0xc2b2ae35u;
  x ^= x >> 16;
  return x;
}

__device__ __forceinline__ float probe_value(int kind, uint32_t key) {
  if (kind == 0) return 0.f;
  if (kind == 1) return 0.015625f;
  return (float)(mix32(key) & 0xFFFFu) * (1.0f / 32768.0f) - 1.0f;
}

}  // namespace

__global__ __launch_bounds__(256, 2) void probe_mfma(int kind, int iters, float* __restrict__ sink) {
  const uint32_t gid = blockIdx.x * 256 + threadIdx.x;
  half8 a[8], b[8];
#pragma unroll
  for (int q = 0; q < 8; ++q)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t key = (gid * 8u + (uint32_t)q) * 16u + (uint32_t)e;
      a[q][e] = (_Float16)probe_value(kind, key);
      b[q][e] = (_Float16)probe_value(kind, key + 8u);
    }
  float16v acc[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) acc[c] = float16v{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[q & 3] = mfma32x32x16(a[q], b[7 - q], acc[q & 3]);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  sink[gid] = s;
}

}  // namespace sa

extern "C" sa_status sa_probe_mfma(int32_t operands, int32_t iters, float* sink, void* stream) {
  if (sink == nullptr || operands < 0 || operands > 2 || iters < 1 || iters > 1000000) return SA_E_INVALID;
  static_assert(sa::kProbeWGs * 256 == SA_PROBE_SINK_FLOATS, "sink size");
  hipLaunchKernelGGL(sa::probe_mfma, dim3(sa::kProbeWGs), dim3(256), 0, (hipStream_t)stream, (int)operands,
                     (int)iters, sink);
  return hipGetLastError() == hipSuccess ? SA_OK : SA_E_HIP;
}
