// sa_slots.h — the partial-sum slots of one user, shared by the kernels that
// reduce them (finalize, the backward's per-user step, the pre-reduction).
//
// Pass 2 (or the one-pass kernel, or the fp32 launcher) leaves each user's
// sums U, m in a contiguous range of partial slots.  When one user owns many
// slots (few long users), presum_slots first folds each of kPreSplit equal
// sub-ranges into its first slot, in slot order, in parallel over the
// sub-ranges; the reducing kernels then add the sub-range heads in order.
// Every kernel takes the same decision from the same inputs, so the sums are
// the same to the bit wherever they are formed.
#ifndef SA_SLOTS_H_
#define SA_SLOTS_H_

#include <stdint.h>

#include "sa_layout.h"

namespace sa {

constexpr int kPreSplit = 8;   // sub-ranges of a pre-summed user's slots
constexpr int kPreMin = 16;    // a user's slots are pre-summed beyond this count
constexpr int kPreUsers = 16;  // launches with at most this many users run the pre-reduction

// slot range [c0, c1) of user u: chunks (fp32 path), or group + u for the
// groups whose equal tile ranges meet the user's tiles (bf16 paths)
__device__ __forceinline__ void user_slots(const Layout& L, const void* ws, int u, int& c0, int& c1) {
  const char* base = static_cast<const char*>(ws);
  if (L.dtype != 0) {
    const int32_t* chunk_base = reinterpret_cast<const int32_t*>(base + L.off_chunk_base);
    c0 = chunk_base[u];
    c1 = chunk_base[u + 1];
    return;
  }
  const int32_t* tile_base = reinterpret_cast<const int32_t*>(base + L.off_tile_base);
  const int32_t nt = reinterpret_cast<const int32_t*>(base + L.off_hdr)[kHdrTiles];
  const int G = L.fused ? L.groups : L.p2_groups;
  const int32_t Tg = (nt + 4 * G - 1) / (4 * G) * 4;
  const int32_t t0 = tile_base[u], t1 = tile_base[u + 1];
  c0 = c1 = 0;
  if (t1 > t0) {
    c0 = t0 / Tg + u;
    c1 = (t1 - 1) / Tg + 1 + u;
  }
}

// first slot of sub-range s of a range of n slots starting at c0
__device__ __forceinline__ int sub_head(int c0, int n, int s) {
  return c0 + (int)((int64_t)n * s / kPreSplit);
}

// whether a launch runs the pre-reduction (host side)
inline bool presum_launch(const Layout& L) { return L.R > 0 && L.R <= kPreUsers; }

}  // namespace sa

#endif  // SA_SLOTS_H_
