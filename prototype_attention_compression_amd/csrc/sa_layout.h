// sa_layout.h — work decomposition and workspace layout shared by the host
// API and the kernels of libsa.
//
// Work units.  Every user's history is cut into TILEs of 32 tokens; the tile
// count of a user is rounded up to a multiple of kUserTileAlign (the trailing
// tiles hold padding rows, which carry zero allocation).  Tiles are numbered
// user by user; tile_base[u] (exclusive prefix sums, written on the device
// from `offsets`) maps a global tile index back to its user by binary search.
//
// Two paths share the workspace:
//   * two-pass: pass 1 (per-token logsumexp over prototypes) runs over tiles;
//     pass 2 (allocation + accumulation, bf16) runs as p2_groups GROUPS of
//     n_pblocks workgroups (one per prototype block), each group walking an
//     equal contiguous tile range, with partial sums per (group, user) pair
//     at index group + user as below.  The fp32 path instead cuts every user
//     into CHUNKs of up to `tiles_per_chunk` tiles (chunk_base[u] numbers them
//     user by user), with partial sums per chunk.
//   * one-pass: a packing kernel writes the fp16 token rows; then GROUPS of
//     n_pblocks co-resident workgroups (one per 256-prototype block) each walk
//     an equal contiguous range of tiles, exchanging per-token partial
//     softmax denominators; partial sums per (group, user) pair, stored at
//     index group + user (unique for overlapping pairs: both ranges are
//     contiguous and increasing, so along the overlaps group + user rises).
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
constexpr int kFusedProtos = 256;    // prototypes per one-pass workgroup (8 waves x 32)
constexpr int kFusedWGs = 256;       // one-pass grid: groups x n_pblocks workgroups
constexpr int kP2WGs = 256;          // pass-2 grid (bf16): p2_groups x n_pblocks workgroups
constexpr int kXSlots = 8;           // ring slots of the one-pass exchange
constexpr int kBwdEWGs = 512;        // bwd_e grid: e_groups x e_pblocks workgroups
constexpr int kOuterRows = 256;      // rows per chunk of the outer-product reductions

// Device error flags (workspace header word 0, bitwise or).
constexpr int32_t kErrBadOffsets = 1;
constexpr int32_t kErrExchange = 2;  // a bounded wait between workgroups expired
constexpr int32_t kErrRange = 4;     // a kept bf16 input value outside fp16's finite range
constexpr int32_t kErrSketchRow = 8; // a sketch row index outside the given sketch array

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
  int32_t fused;           // 1: the one-pass path is built for this shape
  int32_t groups;          // one-pass groups (kFusedWGs / n_pblocks)
  int32_t parts_max;       // partial-sum slots: chunks_max (fp32), else max(groups, p2_groups) + R
  int32_t p2_groups;       // pass-2 groups (bf16): kP2WGs / n_pblocks
  // byte offsets into the workspace (all 256-aligned)
  size_t off_hdr;          // [64] int32: error flag, totals
  size_t off_tile_base;    // [R+1] int32
  size_t off_chunk_base;   // [R+1] int32
  size_t off_q16;          // [k, d] fp16    queries
  size_t off_qpart;        // [k / 32] float largest |q_j| of each 32-row block of the fp16 queries
  size_t off_zrow;         // [128] uint16 zeros: the row pass 1 loads for a tile slot without a token
  size_t off_h16;          // [tiles_max, 32, d] fp16    token rows
  size_t off_nl;           // [tiles_max, 32] uint32 per token (+ 4 words).  Two-pass: fp16 pairs
                           //   (-l_hi, -l_lo), l = lse_t - 14, (-60000, 0) if dropped.
                           //   One-pass: 1 if the token takes part, else 0.
  size_t off_xbuf;         // [groups, kXSlots, 32, n_pblocks] uint64 exchange words
  size_t off_q32;          // [k, d] float   queries, fp32 path
  size_t off_lse32;        // [tiles_max*32] float, fp32 path
  size_t off_part_u;       // [parts_max, k, d] float  partial sums of A h
  size_t off_part_m;       // [parts_max, k] float     partial masses
  // backward (bf16 only; laid out by the backward workspace query, else 0)
  int32_t e_waves;         // bwd_e waves per workgroup (4 or 2), 32 prototypes each
  int32_t e_pblocks;       // k / (32 e_waves)
  int32_t e_groups;        // bwd_e groups: max(1, kBwdEWGs / e_pblocks)
  int32_t o_chunks;        // row chunks of the outer-product reductions
  size_t off_bz32;         // [R, k, d] float   Z = (dS / m) Wv^T
  size_t off_bsbar;        // [R, k, d] float   U / m (the mass-normalised history rows)
  size_t off_bzmax;        // [R, k / 32] float largest |Z| of each 32-row block
  size_t off_bz16;         // [R, k, d] fp16    Z zs_u
  size_t off_bcz;          // [R, k] float      c zs_u
  size_t off_bzs;          // [R] float         zs_u, a power of two
  size_t off_bbmax;        // [R] uint32        bits of the user's largest |Y - c| (scaled, >= 0)
  size_t off_bdelta;       // [tiles_max, 32] float  delta_t zs_u
  size_t off_bepart;       // [e_groups + R, k, d] float partial E per (group, user) at group + user
  size_t off_betot;        // [k, d] float      E = sum_t dL[., t] h_t
  size_t off_bopart;       // [o_chunks, d, d] float partial outer products
  size_t total;
};

// Header words.
constexpr int kHdrErr = 0;
                                 // (word 1 unused)
constexpr int kHdrTiles = 2;     // total tiles
constexpr int kHdrChunks = 3;    // total chunks
constexpr int kHdrHmax = 4;      // float bits: largest |h_t| of a kept token (one-pass)

}  // namespace sa
