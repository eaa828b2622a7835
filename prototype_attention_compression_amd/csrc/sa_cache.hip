// sa_cache.hip — the user-keyed sketch cache and its cache-miss driver.
//
// The sketch is user-only and target-agnostic, so SequenceO1 caches it: a
// local cache in training reuses a user's sketch across repeated instances
// (3 h lifetime, hit rate about 0.5) and a serving cache across consecutive
// requests (1 h, about 0.6); a hit skips storing, moving and processing the
// raw history, and the computation of the misses overlaps other work
// ("pipeline lift") (blog "100,000 videos in your pocket", "How it works"
// item 3 and "The numbers"; review page, "Summary").
//
// Host side (sa_cache_lookup, pure host code): a map user -> slot of a
// caller-owned device slab [capacity, k, d] float32 (+ masses [capacity,
// k]).  An entry is fresh while now - t_computed < ttl.  For a batch of
// requests, in order: a fresh entry is a hit; the first request of any other
// user is a miss and gets a slot (a free one, else an expired entry, else
// the least recently used entry that no request of this batch uses); later
// requests of that user in the batch share the miss's slot and count as
// hits (their sketch comes from the same computation).  More distinct users
// in one batch than slots is SA_E_INVALID.
//
// Device side (sa_cache_fill): the miss users' history rows are gathered
// from the caller's packed history store into one ragged batch (the one
// transfer a miss costs), compressed by one sa_compress launch, and the
// sketches scattered into their slots -- all stream-ordered on the caller's
// stream, so a caller runs it on a side stream while other work proceeds.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <new>
#include <unordered_map>
#include <unordered_set>
#include <vector>

#include "sa.h"
#include "sa_device.h"
#include "sa_launch.h"

namespace sa {

// Row gather: miss user i = blockIdx.y copies its rows [src_start[i],
// src_start[i] + len_i) to [dst_off[i], dst_off[i+1]) -- one contiguous,
// coalesced 16-byte-per-lane copy per user (rows of row_vec 16-byte words)
__global__ __launch_bounds__(256) void gather_rows(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                   const int64_t* __restrict__ src_start,
                                                   const int64_t* __restrict__ dst_off, int32_t row_vec) {
  const int i = blockIdx.y;
  const int64_t d0 = dst_off[i], n = (dst_off[i + 1] - d0) * row_vec;
  const uint4* s = src + src_start[i] * row_vec;
  uint4* t = dst + d0 * row_vec;
  for (int64_t v = (int64_t)blockIdx.x * 256 + threadIdx.x; v < n; v += (int64_t)gridDim.x * 256) t[v] = s[v];
}

// same for one byte per row (the token mask)
__global__ __launch_bounds__(256) void gather_bytes(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst,
                                                    const int64_t* __restrict__ src_start,
                                                    const int64_t* __restrict__ dst_off) {
  const int i = blockIdx.y;
  const int64_t d0 = dst_off[i], n = dst_off[i + 1] - d0;
  const uint8_t* s = src + src_start[i];
  uint8_t* t = dst + d0;
  for (int64_t v = (int64_t)blockIdx.x * 256 + threadIdx.x; v < n; v += (int64_t)gridDim.x * 256) t[v] = s[v];
}

// slab[slot[i]] = S[i] (k d floats) and mass_slab[slot[i]] = mass[i]
__global__ __launch_bounds__(256) void scatter_slots(const float4* __restrict__ S, const float* __restrict__ mass,
                                                     const int32_t* __restrict__ slots, int32_t row_vec, int32_t k,
                                                     float4* __restrict__ slab, float* __restrict__ mass_slab) {
  const int i = blockIdx.y;
  const int64_t dst = (int64_t)slots[i];
  for (int v = blockIdx.x * 256 + threadIdx.x; v < row_vec; v += gridDim.x * 256)
    slab[dst * row_vec + v] = S[(int64_t)i * row_vec + v];
  if (mass_slab != nullptr && blockIdx.x == 0)
    for (int j = threadIdx.x; j < k; j += 256) mass_slab[dst * k + j] = mass[(int64_t)i * k + j];
}

namespace {

struct Entry {
  int32_t slot;
  double t_computed;
  double t_used;
  int64_t batch;   // last batch that used the entry
};

}  // namespace
}  // namespace sa

struct sa_cache {
  int32_t capacity = 0, k = 0, d = 0;
  double ttl = 0.0;
  float* slab = nullptr;
  float* mass_slab = nullptr;
  std::unordered_map<int64_t, sa::Entry> map;
  std::vector<int64_t> slot_user;   // user held by each slot, -1 if free
  int64_t batch = 0;
};

namespace sa {
namespace {

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct FillLayout {
  size_t off_src_start, off_dst_off, off_slots, off_H, off_mask, off_S, off_mass, off_sa, sa_bytes, total;
};

FillLayout fill_layout(const sa_problem& store, int64_t max_users, int64_t max_tokens) {
  FillLayout F;
  size_t off = 0;
  auto take = [&](size_t b) {
    size_t o = off;
    off = align_up(off + b);
    return o;
  };
  const size_t elem = store.dtype == SA_BF16 ? 2 : 4;
  F.off_src_start = take((size_t)max_users * 8);
  F.off_dst_off = take(((size_t)max_users + 1) * 8);
  F.off_slots = take((size_t)max_users * 4);
  F.off_H = take((size_t)max_tokens * store.d * elem);
  F.off_mask = take((size_t)max_tokens);
  F.off_S = take((size_t)max_users * store.k * store.d * 4);
  F.off_mass = take((size_t)max_users * store.k * 4);
  sa_problem mp = store;
  mp.num_users = max_users;
  mp.total_tokens = max_tokens;
  mp.flags = 0;
  size_t b = 0;
  if (sa_workspace_size(&mp, &b) != SA_OK) b = 0;
  F.sa_bytes = b;
  F.off_sa = take(b);
  F.total = off;
  return F;
}

}  // namespace
}  // namespace sa

extern "C" {

sa_status sa_cache_create(int32_t capacity, int32_t k, int32_t d, double ttl_seconds, float* slab, float* mass_slab,
                          sa_cache** cache) {
  if (cache == nullptr) return SA_E_INVALID;
  *cache = nullptr;
  if (capacity <= 0 || k <= 0 || d <= 0 || !(ttl_seconds > 0.0) || slab == nullptr) return SA_E_INVALID;
  if (reinterpret_cast<uintptr_t>(slab) % 16 != 0) return SA_E_INVALID;
  sa_cache* c = new (std::nothrow) sa_cache();
  if (c == nullptr) return SA_E_INVALID;
  c->capacity = capacity;
  c->k = k;
  c->d = d;
  c->ttl = ttl_seconds;
  c->slab = slab;
  c->mass_slab = mass_slab;
  try {
    c->slot_user.assign((size_t)capacity, -1);
    c->map.reserve((size_t)capacity * 2);
  } catch (...) {
    delete c;
    return SA_E_INVALID;
  }
  *cache = c;
  return SA_OK;
}

sa_status sa_cache_destroy(sa_cache* cache) {
  delete cache;
  return SA_OK;
}

sa_status sa_cache_lookup(sa_cache* c, const int64_t* users, int64_t n, double now, int32_t* slots,
                          int64_t* miss_users, int32_t* miss_slots, int64_t* n_miss, sa_cache_stats* stats) {
  if (c == nullptr || n < 0 || n_miss == nullptr || stats == nullptr) return SA_E_INVALID;
  if (n > 0 && (users == nullptr || slots == nullptr || miss_users == nullptr || miss_slots == nullptr))
    return SA_E_INVALID;
  try {
    // Every distinct user of the batch holds one slot for the rest of the
    // batch, so a slot can be found for each new user exactly when the batch
    // has no more distinct users than slots.  Checked before anything
    // changes: a refused batch leaves the cache as it was.
    {
      std::unordered_set<int64_t> distinct;
      distinct.reserve((size_t)std::min<int64_t>(n, (int64_t)c->capacity + 1) * 2);
      for (int64_t i = 0; i < n; ++i) {
        distinct.insert(users[i]);
        if ((int64_t)distinct.size() > c->capacity) return SA_E_INVALID;
      }
    }
    const int64_t batch = ++c->batch;
    sa_cache_stats st;
    memset(&st, 0, sizeof(st));
    int64_t nm = 0;
    int32_t next_free = 0;
    for (int64_t i = 0; i < n; ++i) {
      const int64_t user = users[i];
      auto it = c->map.find(user);
      if (it != c->map.end()) {
        sa::Entry& e = it->second;
        const bool fresh = now - e.t_computed < c->ttl;
        if (fresh || e.batch == batch) {   // cached, or computed by this batch's miss
          e.t_used = now;
          e.batch = batch;
          slots[i] = e.slot;
          ++st.hits;
          continue;
        }
        // stale: recompute into the same slot
        e.t_computed = now;
        e.t_used = now;
        e.batch = batch;
        slots[i] = e.slot;
        miss_users[nm] = user;
        miss_slots[nm] = e.slot;
        ++nm;
        ++st.misses;
        ++st.expired;
        continue;
      }
      // a new user: a free slot, else an expired entry, else the least
      // recently used entry no request of this batch holds
      int32_t slot = -1;
      while (next_free < c->capacity && c->slot_user[(size_t)next_free] >= 0) ++next_free;
      if (next_free < c->capacity) {
        slot = next_free;
      } else {
        int32_t best = -1;
        bool best_expired = false;
        double best_used = 0.0;
        for (int32_t s = 0; s < c->capacity; ++s) {
          const sa::Entry& e = c->map.at(c->slot_user[(size_t)s]);
          if (e.batch == batch) continue;
          const bool expired = now - e.t_computed >= c->ttl;
          if (best < 0 || (expired && !best_expired) ||
              (expired == best_expired && e.t_used < best_used)) {
            best = s;
            best_expired = expired;
            best_used = e.t_used;
          }
        }
        if (best < 0) return SA_E_INVALID;   // excluded by the distinct-user check above
        c->map.erase(c->slot_user[(size_t)best]);
        ++st.evictions;
        slot = best;
      }
      c->slot_user[(size_t)slot] = user;
      c->map.emplace(user, sa::Entry{slot, now, now, batch});
      slots[i] = slot;
      miss_users[nm] = user;
      miss_slots[nm] = slot;
      ++nm;
      ++st.misses;
    }
    *n_miss = nm;
    *stats = st;
    return SA_OK;
  } catch (...) {
    return SA_E_INVALID;
  }
}

sa_status sa_cache_fill_workspace_size(const sa_problem* store, int64_t max_miss_users, int64_t max_miss_tokens,
                                       size_t* bytes) {
  if (store == nullptr || bytes == nullptr || max_miss_users < 0 || max_miss_tokens < 0) return SA_E_INVALID;
  sa_problem mp = *store;
  mp.num_users = max_miss_users;
  mp.total_tokens = max_miss_tokens;
  mp.flags = 0;
  size_t b = 0;
  const sa_status st = sa_workspace_size(&mp, &b);
  if (st != SA_OK) return st;
  *bytes = sa::fill_layout(*store, max_miss_users, max_miss_tokens).total;
  return SA_OK;
}

sa_status sa_cache_fill(sa_cache* c, const sa_problem* store, const void* H_store, const int64_t* store_offsets,
                        const uint8_t* mask_store, const void* Wk, const void* Wv, const void* P,
                        const int64_t* miss_users, const int32_t* miss_slots, int64_t n_miss, void* workspace,
                        size_t workspace_bytes, void* stream) {
  try {
    if (c == nullptr || store == nullptr || n_miss < 0) return SA_E_INVALID;
    if (n_miss == 0) return SA_OK;
    if (miss_users == nullptr || miss_slots == nullptr || store_offsets == nullptr || H_store == nullptr)
      return SA_E_INVALID;
    if (store->k != c->k || store->d != c->d || store->num_users <= 0) return SA_E_INVALID;
    if (n_miss > 65535) return SA_E_UNSUPPORTED;   // one scatter grid row per miss
    if (reinterpret_cast<uintptr_t>(H_store) % 16 != 0) return SA_E_INVALID;
    if (Wk == nullptr || Wv == nullptr || P == nullptr) return SA_E_INVALID;
    if (reinterpret_cast<uintptr_t>(Wk) % 16 != 0 || reinterpret_cast<uintptr_t>(Wv) % 16 != 0 ||
        reinterpret_cast<uintptr_t>(P) % 16 != 0)
      return SA_E_INVALID;
    // host: the miss batch's layout from the store's (host) offsets
    std::vector<int64_t> src_start((size_t)n_miss), dst_off((size_t)n_miss + 1);
    dst_off[0] = 0;
    for (int64_t i = 0; i < n_miss; ++i) {
      const int64_t u = miss_users[i];
      if (u < 0 || u >= store->num_users) return SA_E_INVALID;
      if (miss_slots[i] < 0 || miss_slots[i] >= c->capacity) return SA_E_INVALID;
      const int64_t lo = store_offsets[u], hi = store_offsets[u + 1];
      if (lo < 0 || hi < lo || hi > store->total_tokens) return SA_E_INVALID;
      src_start[(size_t)i] = lo;
      dst_off[(size_t)i + 1] = dst_off[(size_t)i] + (hi - lo);
    }
    const int64_t tokens = dst_off[(size_t)n_miss];
    const sa::FillLayout F = sa::fill_layout(*store, n_miss, tokens);
    if (workspace == nullptr || workspace_bytes < F.total) return SA_E_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(workspace) % sa::kAlign != 0) return SA_E_INVALID;
    char* ws = static_cast<char*>(workspace);
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    // Small host arrays to the device.  From pageable host memory an
    // asynchronous host-to-device copy returns once the runtime has staged
    // the source, so these locals may go out of scope afterwards.
    if (hipMemcpyAsync(ws + F.off_src_start, src_start.data(), (size_t)n_miss * 8, hipMemcpyHostToDevice, s) !=
            hipSuccess ||
        hipMemcpyAsync(ws + F.off_dst_off, dst_off.data(), ((size_t)n_miss + 1) * 8, hipMemcpyHostToDevice, s) !=
            hipSuccess ||
        hipMemcpyAsync(ws + F.off_slots, miss_slots, (size_t)n_miss * 4, hipMemcpyHostToDevice, s) != hipSuccess)
      return SA_E_HIP;
    const int64_t* d_src = reinterpret_cast<const int64_t*>(ws + F.off_src_start);
    const int64_t* d_dst = reinterpret_cast<const int64_t*>(ws + F.off_dst_off);
    const size_t elem = store->dtype == SA_BF16 ? 2 : 4;
    const size_t row_bytes = (size_t)store->d * elem;
    if (tokens > 0) {
      const int32_t row_vec = (int32_t)(row_bytes / 16);
      // enough workgroups per user to spread the longest histories
      const dim3 grid(64, (unsigned)n_miss);
      hipLaunchKernelGGL(sa::gather_rows, grid, dim3(256), 0, s, static_cast<const uint4*>(H_store),
                         reinterpret_cast<uint4*>(ws + F.off_H), d_src, d_dst, row_vec);
      if (hipGetLastError() != hipSuccess) return SA_E_HIP;
      if (mask_store != nullptr) {
        hipLaunchKernelGGL(sa::gather_bytes, dim3(16, (unsigned)n_miss), dim3(256), 0, s, mask_store,
                           reinterpret_cast<uint8_t*>(ws + F.off_mask), d_src, d_dst);
        if (hipGetLastError() != hipSuccess) return SA_E_HIP;
      }
    }
    // one compression launch for every miss
    sa_problem mp = *store;
    mp.num_users = n_miss;
    mp.total_tokens = tokens;
    mp.flags = 0;
    float* S = reinterpret_cast<float*>(ws + F.off_S);
    float* mass = reinterpret_cast<float*>(ws + F.off_mass);
    const sa_status st = sa_compress(&mp, tokens > 0 ? ws + F.off_H : nullptr, d_dst,
                                     mask_store != nullptr ? reinterpret_cast<uint8_t*>(ws + F.off_mask) : nullptr,
                                     Wk, Wv, P, S, mass, ws + F.off_sa, F.sa_bytes, stream);
    if (st != SA_OK) return st;
    const int32_t row_vec = c->k * c->d / 4;
    dim3 grid((unsigned)std::max(1, std::min(64, (row_vec + 255) / 256)), (unsigned)n_miss);
    hipLaunchKernelGGL(sa::scatter_slots, grid, dim3(256), 0, s, reinterpret_cast<const float4*>(S), mass,
                       reinterpret_cast<const int32_t*>(ws + F.off_slots), row_vec, c->k,
                       reinterpret_cast<float4*>(c->slab), c->mass_slab);
    return hipGetLastError() == hipSuccess ? SA_OK : SA_E_HIP;
  } catch (...) {
    return SA_E_HIP;
  }
}

}  // extern "C"
