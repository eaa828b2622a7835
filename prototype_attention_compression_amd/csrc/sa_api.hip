// sa_api.hip — the C ABI of libsa (declared in include/sa.h): argument
// validation (pure host code, before any HIP call), workspace layout, and
// the stream-ordered launch sequence.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <mutex>

#include "sa.h"
#include "sa_launch.h"
#include "sa_layout.h"

namespace sa {
namespace {

constexpr size_t kAlign = 256;
constexpr int64_t kMaxTokens = (int64_t)1 << 31;
constexpr int64_t kMaxUsers = (int64_t)1 << 28;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return reinterpret_cast<uintptr_t>(p) % 16 == 0; }

sa_status check_problem(const sa_problem* p) {
  if (p == nullptr) return SA_E_INVALID;
  if (p->num_users < 0 || p->total_tokens < 0 || p->d <= 0 || p->k <= 0) return SA_E_INVALID;
  if ((p->flags & ~(SA_FLAG_TWO_PASS | SA_FLAG_ONE_PASS)) != 0) return SA_E_INVALID;
  if ((p->flags & SA_FLAG_TWO_PASS) && (p->flags & SA_FLAG_ONE_PASS)) return SA_E_INVALID;
  if (p->dtype != SA_BF16 && p->dtype != SA_F32) return SA_E_INVALID;
  if (p->d != 64 && p->d != 128) return SA_E_UNSUPPORTED;
  if (p->k % 64 != 0 || p->k > 4096) return SA_E_UNSUPPORTED;
  if (p->total_tokens >= kMaxTokens || p->num_users >= kMaxUsers) return SA_E_UNSUPPORTED;
  return SA_OK;
}

// The backward pass: bf16 inputs only; it always runs the two forward passes.
sa_status check_problem_bwd(const sa_problem* p) {
  sa_status st = check_problem(p);
  if (st != SA_OK) return st;
  if (p->dtype != SA_BF16 || (p->flags & SA_FLAG_ONE_PASS)) return SA_E_UNSUPPORTED;
  return SA_OK;
}

// pass-2 waves per workgroup: 8, 4 or 2, dividing k / 32 (k is a multiple of 64)
int pick_waves(int k) {
  const int blocks = k / kProtoPerWave;
  return blocks % 8 == 0 ? 8 : (blocks % 4 == 0 ? 4 : 2);
}

// Tiles per pass-2 chunk: enough chunks that chunks x prototype blocks fill
// the 256 compute units at least once, and no longer than 256 tiles (8192
// tokens) so per-chunk partial sums stay a small fraction of the traffic.
int pick_tiles_per_chunk(int64_t tiles_est, int n_pblocks, bool f32) {
  const int64_t want = (tiles_est * n_pblocks + 255) / 256;
  const int64_t lo = f32 ? 4 : 16, hi = f32 ? 64 : 256;
  const int64_t ct = want < lo ? lo : (want > hi ? hi : want);
  return (int)((ct + kUserTileAlign - 1) / kUserTileAlign * kUserTileAlign);
}

// `bwd`: also lay out the backward pass's buffers (sa_compress_backward)
Layout make_layout(const sa_problem& p, bool bwd = false) {
  Layout L;
  memset(&L, 0, sizeof(L));
  L.N = p.total_tokens;
  L.R = (int32_t)p.num_users;
  L.d = p.d;
  L.k = p.k;
  L.dtype = p.dtype;
  const bool f32 = p.dtype == SA_F32;
  L.waves = f32 ? 1 : pick_waves(p.k);
  L.n_pblocks = f32 ? p.k / 64 : p.k / (L.waves * kProtoPerWave);
  // sum_u A ceil(n_u / (32 A)) <= (N + (32 A - 1) R) / 32 for A = kUserTileAlign
  const int64_t span = (int64_t)kTile * kUserTileAlign;
  const int64_t tiles_max = (p.total_tokens + (span - 1) * p.num_users) / span * kUserTileAlign;
  L.tiles_max = (int32_t)tiles_max;
  L.tiles_per_chunk = pick_tiles_per_chunk(tiles_max, L.n_pblocks, f32);
  // sum_u ceil(t_u / CT) <= (tiles + (CT - 1) R) / CT
  L.chunks_max = (int32_t)((tiles_max + (int64_t)(L.tiles_per_chunk - 1) * p.num_users) / L.tiles_per_chunk);
  // the one-pass path: sized whenever its shape is built, used per call
  L.fused = 0;
  L.groups = 0;
  L.p2_groups = 0;
  int64_t parts = f32 ? L.chunks_max : 0;
  if (!f32) {
    L.p2_groups = std::max(1, kP2WGs / L.n_pblocks);
    parts = std::max<int64_t>(parts, (int64_t)L.p2_groups + p.num_users);
  }
  if (fused_shape_ok(L)) {
    L.groups = kFusedWGs / (p.k / kFusedProtos);
    parts = std::max<int64_t>(parts, (int64_t)L.groups + p.num_users);
  }
  L.parts_max = (int32_t)parts;
  const size_t R1 = (size_t)p.num_users + 1;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align_up(off + bytes);
    return o;
  };
  L.off_hdr = take(64 * sizeof(int32_t));
  L.off_tile_base = take(R1 * sizeof(int32_t));
  L.off_chunk_base = take(R1 * sizeof(int32_t));
  if (!f32) {
    L.off_q16 = take((size_t)p.k * p.d * 2);
    L.off_qpart = take((size_t)(p.k / 32) * sizeof(float));
    L.off_zrow = take(256);
    L.off_h16 = take((size_t)tiles_max * kTile * p.d * 2);
    // + 16 bytes: the pairs past the last tile that pass 2's -l pieces read
    L.off_nl = take((size_t)tiles_max * kTile * sizeof(uint32_t) + 16);
    if (L.groups > 0) L.off_xbuf = take((size_t)L.groups * kXSlots * kTile * (p.k / kFusedProtos) * sizeof(uint64_t));
  } else {
    L.off_q32 = take((size_t)p.k * p.d * sizeof(float));
    L.off_lse32 = take((size_t)tiles_max * kTile * sizeof(float));
  }
  L.off_part_u = take((size_t)L.parts_max * p.k * p.d * sizeof(float));
  L.off_part_m = take((size_t)L.parts_max * p.k * sizeof(float));
  if (bwd) {
    const size_t Rk = (size_t)p.num_users * p.k;
    // 8 waves (d = 128 only: one 16-byte load per thread and tile), else 4 or 2
    L.e_waves = (p.d == 128 && (p.k / kProtoPerWave) % 8 == 0) ? 8 : ((p.k / kProtoPerWave) % 4 == 0 ? 4 : 2);
    L.e_pblocks = p.k / (kProtoPerWave * L.e_waves);
    L.e_groups = std::max(1, (L.e_waves == 8 ? kBwdEWGs / 2 : kBwdEWGs) / L.e_pblocks);
    const int64_t rows = std::max<int64_t>((int64_t)Rk, p.k);
    L.o_chunks = (int32_t)((rows + kOuterRows - 1) / kOuterRows);
    L.off_bz32 = take(Rk * p.d * sizeof(float));
    L.off_bsbar = take(Rk * p.d * sizeof(float));
    L.off_bzmax = take((size_t)p.num_users * (p.k / 32) * sizeof(float));
    L.off_bz16 = take(Rk * p.d * 2);
    L.off_bcz = take(Rk * sizeof(float));
    L.off_bzs = take((size_t)p.num_users * sizeof(float));
    L.off_bbmax = take((size_t)p.num_users * sizeof(uint32_t));
    L.off_bdelta = take((size_t)tiles_max * kTile * sizeof(float));
    L.off_bepart = take(((size_t)L.e_groups + p.num_users) * p.k * p.d * sizeof(float));
    L.off_betot = take((size_t)p.k * p.d * sizeof(float));
    L.off_bopart = take((size_t)L.o_chunks * p.d * p.d * sizeof(float));
  }
  L.total = off;
  return L;
}

// Target attention: the candidate tiles' schedule only (total_tokens =
// total candidates); dtype f32 makes the schedule kernel skip the query
// norms, which this call has none of.
Layout make_layout_target(const sa_problem& p) {
  Layout L;
  memset(&L, 0, sizeof(L));
  L.N = p.total_tokens;
  L.R = (int32_t)p.num_users;
  L.d = p.d;
  L.k = p.k;
  L.dtype = SA_F32;
  const int64_t span = (int64_t)kTile * kUserTileAlign;
  L.tiles_max = (int32_t)((p.total_tokens + (span - 1) * p.num_users) / span * kUserTileAlign);
  L.tiles_per_chunk = kUserTileAlign;
  const size_t R1 = (size_t)p.num_users + 1;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align_up(off + bytes);
    return o;
  };
  L.off_hdr = take(64 * sizeof(int32_t));
  L.off_tile_base = take(R1 * sizeof(int32_t));
  L.off_chunk_base = take(R1 * sizeof(int32_t));
  L.total = off;
  return L;
}

sa_status check_problem_target(const sa_problem* p) {
  sa_status st = check_problem(p);
  if (st != SA_OK) return st;
  if (p->dtype != SA_BF16 || p->flags != 0) return SA_E_UNSUPPORTED;
  return SA_OK;
}

// Whether the one-pass cooperative grid fits `device`, asked once per device.
bool device_fits_fused(const Layout& L) {
  constexpr int kMaxDev = 64;
  static std::atomic<int> cache[kMaxDev][5];   // per P index: 0 unknown, 1 no, 2 yes
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return false;
  int pi = 0;
  for (int P = L.k / kFusedProtos; P > 1; P >>= 1) ++pi;
  if (pi > 4) return false;
  int v = cache[dev][pi].load(std::memory_order_relaxed);
  if (v == 0) {
    v = fused_fits_device(L, dev) ? 2 : 1;
    cache[dev][pi].store(v, std::memory_order_relaxed);
  }
  return v == 2;
}

// The one-pass kernel when the caller asks for it and the shape and device
// allow it; otherwise (and by default: it does not yet beat the two-pass
// kernels on MI355X) two passes.
bool use_fused(const sa_problem& p, const Layout& L) {
  if (L.groups == 0 || !(p.flags & SA_FLAG_ONE_PASS)) return false;
  return device_fits_fused(L);
}


// The forward: prep, passes 1 and 2 (or the one-pass kernel, or the fp32
// launcher), finalize.  Sbar (optional) receives the mass-normalised rows.
sa_status compress_impl(const sa_problem* problem, const void* H, const int64_t* offsets, const uint8_t* token_mask,
                        const void* Wk, const void* Wv, const void* P, float* S, float* mass, float* Sbar,
                        void* workspace, size_t workspace_bytes, void* stream, void* const* events) {
  try {
    sa_status st = sa::check_problem(problem);
    if (st != SA_OK) return st;
    const sa_problem& p = *problem;
    if (p.num_users == 0) return SA_OK;
    if (offsets == nullptr || Wk == nullptr || Wv == nullptr || P == nullptr || S == nullptr)
      return SA_E_INVALID;
    if (p.total_tokens > 0 && H == nullptr) return SA_E_INVALID;
    // the kernels read H, Wk, Wv and P in 16-byte vectors and offsets as int64
    if (!aligned16(H) || !aligned16(Wk) || !aligned16(Wv) || !aligned16(P) ||
        reinterpret_cast<uintptr_t>(offsets) % 8 != 0)
      return SA_E_INVALID;
    sa::Layout L = sa::make_layout(p);
    if (workspace == nullptr || workspace_bytes < L.total) return SA_E_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(workspace) % sa::kAlign != 0) return SA_E_INVALID;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    auto mark = [&](int i) {
      return events == nullptr || hipEventRecord(reinterpret_cast<hipEvent_t>(events[i]), s) == hipSuccess;
    };
    if (p.dtype == SA_BF16 && p.total_tokens > 0) L.fused = sa::use_fused(p, L) ? 1 : 0;
    if (!mark(0)) return SA_E_HIP;
    if (sa::launch_prep(L, P, Wk, offsets, workspace, s) != hipSuccess) return SA_E_HIP;
    if (!mark(1)) return SA_E_HIP;
    if (L.fused) {
      if (sa::launch_pack(L, H, offsets, token_mask, workspace, s) != hipSuccess) return SA_E_HIP;
      if (!mark(2)) return SA_E_HIP;
      if (sa::launch_fused(L, workspace, s) != hipSuccess) return SA_E_HIP;
    } else if (p.dtype == SA_BF16) {
      if (p.total_tokens > 0) {
        const hipError_t e = sa::pass1q_ok(L) ? sa::launch_pass1q(L, H, offsets, token_mask, workspace, s)
                                              : sa::launch_pass1(L, H, offsets, token_mask, workspace, s);
        if (e != hipSuccess) return SA_E_HIP;
      }
      if (!mark(2)) return SA_E_HIP;
      if (p.total_tokens > 0 && sa::launch_pass2(L, workspace, s) != hipSuccess) return SA_E_HIP;
    } else {
      // the fp32 path launches both passes from one launcher
      if (p.total_tokens > 0 && sa::launch_f32(L, H, offsets, token_mask, workspace, s) != hipSuccess)
        return SA_E_HIP;
      if (!mark(2)) return SA_E_HIP;
    }
    if (!mark(3)) return SA_E_HIP;
    if (sa::launch_finalize(L, Wv, workspace, S, mass, Sbar, s) != hipSuccess) return SA_E_HIP;
    if (!mark(4)) return SA_E_HIP;
    return SA_OK;
  } catch (...) {
    return SA_E_HIP;
  }
}


// The backward: forward passes 1 (and 2 unless Sbar_in and mass_in are
// given), then the per-user, per-token, E and parameter kernels.
sa_status backward_impl(const sa_problem* problem, const void* H, const int64_t* offsets, const uint8_t* token_mask,
                        const void* Wk, const void* Wv, const void* P, const float* Sbar_in, const float* mass_in,
                        const float* dS, float* dH, float* dP, float* dWk, float* dWv, void* workspace,
                        size_t workspace_bytes, void* stream, void* const* events) {
  try {
    sa_status st = sa::check_problem_bwd(problem);
    if (st != SA_OK) return st;
    const sa_problem& p = *problem;
    if (Wk == nullptr || Wv == nullptr || P == nullptr || dP == nullptr || dWk == nullptr || dWv == nullptr)
      return SA_E_INVALID;
    if (p.num_users > 0 && (offsets == nullptr || dS == nullptr)) return SA_E_INVALID;
    if (p.total_tokens > 0 && (H == nullptr || dH == nullptr)) return SA_E_INVALID;
    if (!aligned16(H) || !aligned16(Wk) || !aligned16(Wv) || !aligned16(P) ||
        reinterpret_cast<uintptr_t>(offsets) % 8 != 0)
      return SA_E_INVALID;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    auto mark = [&](int i) {
      return events == nullptr || hipEventRecord(reinterpret_cast<hipEvent_t>(events[i]), s) == hipSuccess;
    };
    const int64_t dd = (int64_t)p.d * p.d;
    if (p.num_users == 0) {   // no users: the parameter gradients are empty sums
      if (!mark(0)) return SA_E_HIP;
      if (sa::launch_fill_zero(dP, (int64_t)p.k * p.d, s) != hipSuccess ||
          sa::launch_fill_zero(dWk, dd, s) != hipSuccess || sa::launch_fill_zero(dWv, dd, s) != hipSuccess)
        return SA_E_HIP;
      for (int i = 1; i < SA_NUM_BWD_PHASE_EVENTS; ++i)
        if (!mark(i)) return SA_E_HIP;
      return SA_OK;
    }
    sa::Layout L = sa::make_layout(p, true);
    if (workspace == nullptr || workspace_bytes < L.total) return SA_E_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(workspace) % sa::kAlign != 0) return SA_E_INVALID;
    if (!mark(0)) return SA_E_HIP;
    // forward passes 1 and 2: fp16 token rows, logsumexps, partial sums;
    // pass 2 is not needed when the caller hands in the forward's Sbar and
    // masses
    if (sa::launch_prep(L, P, Wk, offsets, workspace, s) != hipSuccess) return SA_E_HIP;
    if (p.total_tokens > 0) {
      const hipError_t e = sa::pass1q_ok(L) ? sa::launch_pass1q(L, H, offsets, token_mask, workspace, s)
                                            : sa::launch_pass1(L, H, offsets, token_mask, workspace, s);
      if (e != hipSuccess) return SA_E_HIP;
      if (Sbar_in == nullptr && sa::launch_pass2(L, workspace, s) != hipSuccess) return SA_E_HIP;
    }
    if (!mark(1)) return SA_E_HIP;
    if (sa::launch_bwd_user(L, Wv, dS, Sbar_in, mass_in, workspace, s) != hipSuccess) return SA_E_HIP;
    if (!mark(2)) return SA_E_HIP;
    if (sa::launch_bwd_dh(L, offsets, workspace, dH, s) != hipSuccess) return SA_E_HIP;
    if (!mark(3)) return SA_E_HIP;
    if (sa::launch_bwd_e(L, workspace, s) != hipSuccess) return SA_E_HIP;
    if (!mark(4)) return SA_E_HIP;
    if (sa::launch_bwd_params(L, P, Wk, dS, workspace, dP, dWk, dWv, s) != hipSuccess) return SA_E_HIP;
    if (!mark(5)) return SA_E_HIP;
    return SA_OK;
  } catch (...) {
    return SA_E_HIP;
  }
}

// ------------------------------------------------ allocation-free entry point
// sa_compress_static's workspace: a file-scope device array, held by every
// GPU the library runs on until the process ends.  In host code `scratch`
// names a host-side stand-in, never device memory: its device address on a
// GPU comes from hipGetSymbolAddress, taken once per device (with that
// device current) and kept; kernels only ever receive that address.
constexpr int kScratchDevices = 64;
std::atomic<void*> g_scratch_ptr[kScratchDevices];
std::mutex g_scratch_mutex;

}  // namespace

__device__ __align__(256) unsigned char scratch[SA_STATIC_SCRATCH_BYTES];

namespace {

// The current device's scratch address, or nullptr if it cannot be had.
void* scratch_address() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kScratchDevices) return nullptr;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p != nullptr) return p;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
  if (p == nullptr) {
    void* q = nullptr;
    if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || q == nullptr) return nullptr;
    if (reinterpret_cast<uintptr_t>(q) % kAlign != 0) return nullptr;
    g_scratch_ptr[dev].store(q, std::memory_order_release);
    p = q;
  }
  return p;
}

}  // namespace
}  // namespace sa

extern "C" {

sa_status sa_compress_static(const sa_problem* problem, const void* H, const int64_t* offsets,
                             const uint8_t* token_mask, const void* Wk, const void* Wv, const void* P, float* S,
                             float* mass, int32_t* device_error, void* stream) {
  try {
    sa_status st = sa::check_problem(problem);
    if (st != SA_OK) return st;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (problem->num_users == 0) {
      // nothing to compress; the error word of a no-op is 0
      if (device_error != nullptr &&
          sa::launch_fill_zero(reinterpret_cast<float*>(device_error), 1, s) != hipSuccess)
        return SA_E_HIP;
      return SA_OK;
    }
    if (sa::make_layout(*problem).total > (size_t)SA_STATIC_SCRATCH_BYTES) return SA_E_WORKSPACE;
    void* ws = sa::scratch_address();
    if (ws == nullptr) return SA_E_HIP;
    st = sa::compress_impl(problem, H, offsets, token_mask, Wk, Wv, P, S, mass, nullptr, ws,
                           (size_t)SA_STATIC_SCRATCH_BYTES, stream, nullptr);
    if (st != SA_OK) return st;
    if (device_error != nullptr &&
        sa::launch_copy_error(sa::make_layout(*problem), ws, device_error, s) != hipSuccess)
      return SA_E_HIP;
    return SA_OK;
  } catch (...) {
    return SA_E_HIP;
  }
}

sa_status sa_workspace_size(const sa_problem* problem, size_t* bytes) {
  if (bytes == nullptr) return SA_E_INVALID;
  sa_status st = sa::check_problem(problem);
  if (st != SA_OK) return st;
  *bytes = sa::make_layout(*problem).total;
  return SA_OK;
}

size_t sa_workspace_bytes(const sa_problem* problem) {
  size_t bytes = 0;
  return sa_workspace_size(problem, &bytes) == SA_OK ? bytes : 0;
}

sa_status sa_compress(const sa_problem* problem, const void* H, const int64_t* offsets, const uint8_t* token_mask,
                      const void* Wk, const void* Wv, const void* P, float* S, float* mass, void* workspace,
                      size_t workspace_bytes, void* stream) {
  return sa_compress_with_events(problem, H, offsets, token_mask, Wk, Wv, P, S, mass, workspace, workspace_bytes,
                                 stream, nullptr);
}

sa_status sa_compress_with_events(const sa_problem* problem, const void* H, const int64_t* offsets,
                                  const uint8_t* token_mask, const void* Wk, const void* Wv, const void* P, float* S,
                                  float* mass, void* workspace, size_t workspace_bytes, void* stream,
                                  void* const* events) {
  return sa::compress_impl(problem, H, offsets, token_mask, Wk, Wv, P, S, mass, nullptr, workspace, workspace_bytes,
                           stream, events);
}

sa_status sa_compress_with_sbar(const sa_problem* problem, const void* H, const int64_t* offsets,
                                const uint8_t* token_mask, const void* Wk, const void* Wv, const void* P, float* S,
                                float* mass, float* Sbar, void* workspace, size_t workspace_bytes, void* stream,
                                void* const* events) {
  if (problem != nullptr && problem->num_users > 0 && (mass == nullptr || Sbar == nullptr)) return SA_E_INVALID;
  return sa::compress_impl(problem, H, offsets, token_mask, Wk, Wv, P, S, mass, Sbar, workspace, workspace_bytes,
                           stream, events);
}

sa_status sa_read_device_error(const void* workspace, void* stream, int32_t* flag) {
  if (workspace == nullptr || flag == nullptr) return SA_E_INVALID;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  int32_t v = 0;
  if (hipMemcpyAsync(&v, workspace, sizeof(v), hipMemcpyDeviceToHost, s) != hipSuccess) return SA_E_HIP;
  if (hipStreamSynchronize(s) != hipSuccess) return SA_E_HIP;
  *flag = v;
  return SA_OK;
}

sa_status sa_backward_workspace_size(const sa_problem* problem, size_t* bytes) {
  if (bytes == nullptr) return SA_E_INVALID;
  sa_status st = sa::check_problem_bwd(problem);
  if (st != SA_OK) return st;
  *bytes = sa::make_layout(*problem, true).total;
  return SA_OK;
}

sa_status sa_compress_backward(const sa_problem* problem, const void* H, const int64_t* offsets,
                               const uint8_t* token_mask, const void* Wk, const void* Wv, const void* P,
                               const float* dS, float* dH, float* dP, float* dWk, float* dWv, void* workspace,
                               size_t workspace_bytes, void* stream) {
  return sa_compress_backward_with_events(problem, H, offsets, token_mask, Wk, Wv, P, dS, dH, dP, dWk, dWv,
                                          workspace, workspace_bytes, stream, nullptr);
}

sa_status sa_compress_backward_with_events(const sa_problem* problem, const void* H, const int64_t* offsets,
                                           const uint8_t* token_mask, const void* Wk, const void* Wv, const void* P,
                                           const float* dS, float* dH, float* dP, float* dWk, float* dWv,
                                           void* workspace, size_t workspace_bytes, void* stream,
                                           void* const* events) {
  return sa::backward_impl(problem, H, offsets, token_mask, Wk, Wv, P, nullptr, nullptr, dS, dH, dP, dWk, dWv,
                           workspace, workspace_bytes, stream, events);
}

sa_status sa_compress_backward_with_sbar(const sa_problem* problem, const void* H, const int64_t* offsets,
                                         const uint8_t* token_mask, const void* Wk, const void* Wv, const void* P,
                                         const float* Sbar, const float* mass, const float* dS, float* dH, float* dP,
                                         float* dWk, float* dWv, void* workspace, size_t workspace_bytes,
                                         void* stream, void* const* events) {
  if (problem == nullptr) return SA_E_INVALID;
  if (problem->num_users > 0 && (Sbar == nullptr || mass == nullptr)) return SA_E_INVALID;
  return sa::backward_impl(problem, H, offsets, token_mask, Wk, Wv, P, Sbar, mass, dS, dH, dP, dWk, dWv, workspace,
                           workspace_bytes, stream, events);
}

sa_status sa_target_attention_workspace_size(const sa_problem* problem, size_t* bytes) {
  if (bytes == nullptr) return SA_E_INVALID;
  sa_status st = sa::check_problem_target(problem);
  if (st != SA_OK) return st;
  *bytes = sa::make_layout_target(*problem).total;
  return SA_OK;
}

sa_status sa_target_attention(const sa_problem* problem, const void* Q, const int64_t* cand_offsets, const float* S,
                              float* out, float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  if (problem == nullptr) return SA_E_INVALID;
  return sa_target_attention_rows(problem, Q, cand_offsets, S, nullptr, problem->num_users, out, lse, workspace,
                                  workspace_bytes, stream);
}

sa_status sa_target_attention_rows(const sa_problem* problem, const void* Q, const int64_t* cand_offsets,
                                   const float* S, const int32_t* sketch_rows, int64_t sketch_count, float* out,
                                   float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  try {
    sa_status st = sa::check_problem_target(problem);
    if (st != SA_OK) return st;
    const sa_problem& p = *problem;
    if (p.num_users == 0) return SA_OK;
    if (cand_offsets == nullptr || S == nullptr || sketch_count < 0) return SA_E_INVALID;
    if (p.total_tokens > 0 && (Q == nullptr || out == nullptr)) return SA_E_INVALID;
    if (reinterpret_cast<uintptr_t>(S) % 16 != 0 || reinterpret_cast<uintptr_t>(Q) % 16 != 0) return SA_E_INVALID;
    const sa::Layout L = sa::make_layout_target(p);
    if (workspace == nullptr || workspace_bytes < L.total) return SA_E_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(workspace) % sa::kAlign != 0) return SA_E_INVALID;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (sa::launch_target_attention(L, Q, cand_offsets, S, sketch_rows, sketch_count, workspace, out, lse, s) !=
        hipSuccess)
      return SA_E_HIP;
    return SA_OK;
  } catch (...) {
    return SA_E_HIP;
  }
}

const char* sa_status_string(sa_status status) {
  switch (status) {
    case SA_OK: return "SA_OK: success";
    case SA_E_INVALID: return "SA_E_INVALID: invalid argument";
    case SA_E_UNSUPPORTED: return "SA_E_UNSUPPORTED: problem shape or dtype not built (d in {64,128}, k % 64 == 0, k <= 4096)";
    case SA_E_WORKSPACE: return "SA_E_WORKSPACE: workspace missing or smaller than sa_workspace_size";
    case SA_E_HIP: return "SA_E_HIP: HIP runtime or launch error";
  }
  return "unknown sa_status";
}

const char* sa_version(void) { return "0.1.0"; }

}  // extern "C"
