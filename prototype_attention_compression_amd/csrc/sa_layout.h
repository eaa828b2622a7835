// sa_layout.h — work decomposition and workspace layout shared by the host
// API and the kernels of libsa.
//
// Work units.  Every user's history is cut into TILEs of 32 tokens; the tile
// count of a user is rounded up to a multiple of kUserTileAlign (the trailing
// tiles hold padding rows, which carry zero allocation).  Pass 1 (per-token logsumexp over prototypes)
// runs over tiles; pass 2 (allocation + accumulation) runs over CHUNKs of up
// to `tiles_per_chunk` consecutive tiles of one user, times prototype blocks.
// Tiles and chunks are numbered user by user; tile_base[u] / chunk_base[u]
// (exclusive prefix sums, written on the device from `offsets`) map a global
// tile or chunk index back to its user by binary search.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace sa {

constexpr int kTile = 32;            // tokens per tile (one 32-wide MFMA block)
constexpr int kUserTileAlign = 4;    // tiles per user: multiple of this (pass-2 stage)
constexpr int kPass1Tiles = 8;       // tiles per pass-1 workgroup (4 waves x 2 tiles)
constexpr int kProtoPerWave = 32;    // prototypes owned by one pass-2 wave
constexpr int kQChunk = 64;          // prototypes per pass-1 LDS chunk
constexpr int kFinRows = 32;         // prototypes per finalize workgroup
constexpr float kAllocShift = 14.0f; // fp16 allocations carry a 2^14 scale
constexpr int kF32ChunkTiles = 8;    // tiles per chunk on the fp32 path

// Device error flags (workspace header word 0).
constexpr int32_t kErrBadOffsets = 1;

struct Layout {
  // problem
  int64_t N;
  int32_t R;
  int32_t d;
  int32_t k;
  int32_t dtype;           // sa_dtype
  int32_t waves;           // pass-2 waves per workgroup
  int32_t n_pblocks;       // k / (waves * kProtoPerWave)
  int32_t tiles_per_chunk;
  int32_t tiles_max;       // bound on sum_u tiles_u
  int32_t chunks_max;      // bound on sum_u ceil(tiles_u / tiles_per_chunk)
  // byte offsets into the workspace (all 256-aligned)
  size_t off_hdr;          // [64] int32: error flag, qmax (float), totals
  size_t off_tile_base;    // [R+1] int32
  size_t off_chunk_base;   // [R+1] int32
  size_t off_q16;          // [k, d] fp16    queries
  size_t off_qnorm;        // [k] float      |q_j| of the fp16 queries
  size_t off_h16;          // [tiles_max, 32, d] fp16    token rows
  size_t off_nl;           // [tiles_max, 32] fp16 pairs (-l_hi, -l_lo), l = lse_t - 14;
                           //   (-60000, 0) if the token is dropped
  size_t off_q32;          // [k, d] float   queries, fp32 path
  size_t off_lse32;        // [tiles_max*32] float, fp32 path
  size_t off_part_u;       // [chunks_max, k, d] float  per-chunk sums of A h
  size_t off_part_m;       // [chunks_max, k] float     per-chunk masses
  size_t total;
};

// Header words.
constexpr int kHdrErr = 0;
constexpr int kHdrQmax = 1;      // float bits
constexpr int kHdrTiles = 2;     // total tiles
constexpr int kHdrChunks = 3;    // total chunks

}  // namespace sa
