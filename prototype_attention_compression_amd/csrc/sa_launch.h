// sa_launch.h — host-side launchers of the libsa kernels (one per kernel
// file), called in stream order by sa_compress.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sa_layout.h"

namespace sa {

// queries + ragged schedule
hipError_t launch_prep(const Layout& L, const void* P, const void* Wk, const int64_t* offsets, void* ws,
                       hipStream_t stream);
// bf16 path, pass 1: per-token logsumexp and fp16 token rows
hipError_t launch_pass1(const Layout& L, const void* H, const int64_t* offsets, const uint8_t* mask,
                        void* ws, hipStream_t stream);
// bf16 path, pass 1 with the queries resident in registers (k = 256, 512,
// 1024): logsumexp and fp16 token rows
bool pass1q_ok(const Layout& L);
hipError_t launch_pass1q(const Layout& L, const void* H, const int64_t* offsets, const uint8_t* mask, void* ws,
                         hipStream_t stream);
// bf16 path, pass 2: allocations, per-chunk sums of A h and masses
hipError_t launch_pass2(const Layout& L, void* ws, hipStream_t stream);
// fp32 path, both passes
hipError_t launch_f32(const Layout& L, const void* H, const int64_t* offsets, const uint8_t* mask, void* ws,
                      hipStream_t stream);
// one-pass path: fp16 token rows, keep words and the largest row norm
hipError_t launch_pack(const Layout& L, const void* H, const int64_t* offsets, const uint8_t* mask, void* ws,
                       hipStream_t stream);
// one-pass path: shapes it is built for; whether the device holds its
// cooperative grid; the cooperative launch itself
bool fused_shape_ok(const Layout& L);
bool fused_fits_device(const Layout& L, int device);
hipError_t launch_fused(const Layout& L, void* ws, hipStream_t stream);
// partial-sum reduction, prototype-wise normalisation and the value projection
// Pre-reduction of the partial slots of users with many slots (sa_slots.h);
// launch_finalize runs it itself, the backward before its per-user step.
hipError_t launch_presum(const Layout& L, void* ws, hipStream_t stream);
hipError_t launch_finalize(const Layout& L, const void* Wv, void* ws, float* S, float* mass, float* Sbar,
                           hipStream_t stream);
// backward (bf16): per-user Z, c and scales from pass 2's partial sums and dS
hipError_t launch_bwd_user(const Layout& L, const void* Wv, const float* dS, const float* Sbar_in,
                           const float* mass_in, void* ws, hipStream_t stream);
// backward: token-major dH (and the per-token delta the E pass reads)
hipError_t launch_bwd_dh(const Layout& L, const int64_t* offsets, void* ws, float* dH, hipStream_t stream);
// backward: prototype-major partial E = sum_t dL h_t
hipError_t launch_bwd_e(const Layout& L, void* ws, hipStream_t stream);
// backward: E, dP, dWk and dWv from the partials
hipError_t launch_bwd_params(const Layout& L, const void* P, const void* Wk, const float* dS, void* ws, float* dP,
                             float* dWk, float* dWv, hipStream_t stream);
// the ragged schedule alone (tile prefix sums and the offsets check)
hipError_t launch_schedule(const Layout& L, const int64_t* offsets, void* ws, hipStream_t stream);
// sketch-branch target attention (schedule + attention kernel)
hipError_t launch_target_attention(const Layout& L, const void* Q, const int64_t* cand_offsets, const float* S,
                                   const int32_t* sketch_rows, int64_t sketch_count, void* ws, float* out, float* lse,
                                   hipStream_t stream);
// zero fill (used when the batch has no users)
hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t stream);
// dst[0] = the workspace's device error word
hipError_t launch_copy_error(const Layout& L, const void* ws, int32_t* dst, hipStream_t stream);

}  // namespace sa
