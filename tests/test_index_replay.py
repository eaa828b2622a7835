"""Host replay of the kernels' index arithmetic, with bounds checks (no GPU).

For a problem (ragged lengths, d, k) this restates, in plain Python, how the
forward and backward kernels of libsa pick their tiles, users, partial-sum
slots and rows, and checks every index against the size of the buffer it
addresses.  The buffer sizes come from a restatement of the library's
workspace layout, pinned to the library itself: its byte totals must equal
sa_workspace_size / sa_backward_workspace_size for every shape replayed.

It also pins a bug found this way: pass 1 with resident queries used to
read a padding tile's first slot, offsets[u] + 32 i, as its clamped row,
which for the last user lies up to 95 rows past the end of H (and 95 bytes
past the mask) whenever that user's length leaves a padding tile; the
fixed kernel reads the user's first row instead."""
import ctypes
import math

import numpy as np
import pytest

import prototype_attention_compression_amd as sa
from prototype_attention_compression_amd import _lib

TILE, ALIGN_T, PPW = 32, 4, 32
P2_WGS, FUSED_WGS, FUSED_PROTOS, XSLOTS, BWD_E_WGS, OUTER_ROWS = 256, 256, 256, 8, 512, 256
PRE_SPLIT, PRE_MIN, PRE_USERS = 8, 16, 16


def _align(x):
    return (x + 255) // 256 * 256


def layout(R, N, d, k, bwd):
    """The workspace layout of a bf16 problem: element counts of each buffer
    and the launch constants the kernels read."""
    L = dict(R=R, N=N, d=d, k=k)
    blocks = k // PPW
    waves = 8 if blocks % 8 == 0 else (4 if blocks % 4 == 0 else 2)
    L["n_pblocks"] = k // (waves * PPW)
    span = TILE * ALIGN_T
    L["tiles_max"] = (N + (span - 1) * R) // span * ALIGN_T
    L["p2_groups"] = max(1, P2_WGS // L["n_pblocks"])
    parts = L["p2_groups"] + R
    fused = k % FUSED_PROTOS == 0 and (k // FUSED_PROTOS) in (1, 2, 4, 8, 16)
    L["groups"] = FUSED_WGS // (k // FUSED_PROTOS) if fused else 0
    if fused:
        parts = max(parts, L["groups"] + R)
    L["parts_max"] = parts
    off = 0
    sizes = {}
    offs = {}

    def take(name, nbytes, elem):
        nonlocal off
        sizes[name] = nbytes // elem
        offs[name] = off
        off = _align(off + nbytes)

    take("hdr", 256, 4)
    take("tile_base", (R + 1) * 4, 4)
    take("chunk_base", (R + 1) * 4, 4)
    take("q16", k * d * 2, 2)
    take("qpart", (k // 32) * 4, 4)
    take("zrow", 256, 4)
    take("h16", L["tiles_max"] * TILE * d * 2, 2)
    take("nl", L["tiles_max"] * TILE * 4 + 16, 4)
    if L["groups"]:
        take("xbuf", L["groups"] * XSLOTS * TILE * (k // FUSED_PROTOS) * 8, 8)
    take("part_u", parts * k * d * 4, 4)
    take("part_m", parts * k * 4, 4)
    if bwd:
        Rk = R * k
        ew = 8 if (d == 128 and blocks % 8 == 0) else (4 if blocks % 4 == 0 else 2)
        L["e_waves"] = ew
        L["e_pblocks"] = k // (PPW * ew)
        L["e_groups"] = max(1, (BWD_E_WGS // 2 if ew == 8 else BWD_E_WGS) // L["e_pblocks"])
        L["o_chunks"] = (max(Rk, k) + OUTER_ROWS - 1) // OUTER_ROWS
        take("bz32", Rk * d * 4, 4)
        take("bsbar", Rk * d * 4, 4)
        take("bzmax", R * (k // 32) * 4, 4)
        take("bz16", Rk * d * 2, 2)
        take("bcz", Rk * 4, 4)
        take("bzs", R * 4, 4)
        take("bbmax", R * 4, 4)
        take("bdelta", L["tiles_max"] * TILE * 4, 4)
        take("bepart", (L["e_groups"] + R) * k * d * 4, 4)
        take("betot", k * d * 4, 4)
        take("bopart", L["o_chunks"] * d * d * 4, 4)
    L["total"] = off
    L["size"] = sizes
    L["off"] = offs   # byte offsets
    return L


def _lib_sizes(R, N, d, k):
    lib = _lib.load()
    pb = _lib.problem(R, N, d, k, sa.SA_BF16)
    fw, bw = ctypes.c_size_t(0), ctypes.c_size_t(0)
    assert lib.sa_workspace_size(ctypes.byref(pb), ctypes.byref(fw)) == sa.SA_OK
    st = lib.sa_backward_workspace_size(ctypes.byref(pb), ctypes.byref(bw))
    return fw.value, (bw.value if st == sa.SA_OK else None)


def schedule(lengths):
    lens = np.asarray(lengths, dtype=np.int64)
    offsets = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    tiles = (lens + TILE * ALIGN_T - 1) // (TILE * ALIGN_T) * ALIGN_T
    tile_base = np.concatenate([[0], np.cumsum(tiles)]).astype(np.int64)
    return offsets, tile_base, int(tile_base[-1])


def user_of(tile_base, t):
    """find_user: the largest u with tile_base[u] <= t (users without tiles
    skipped)."""
    return np.searchsorted(tile_base, t, side="right") - 1


def check(cond, what):
    assert bool(np.all(cond)), what


def group_grid(P, G):
    """pass 2 / bwd_e launch: 8 P ceil(G / 8) workgroups, XCD-aware order;
    every (group < G, block < P) pair appears exactly once."""
    x = np.arange(8 * P * ((G + 7) // 8))
    group = (x & 7) + 8 * ((x >> 3) // P)
    pb = (x >> 3) % P
    live = group < G
    pairs = group[live] * P + pb[live]
    check(np.sort(pairs) == np.arange(G * P), "every (group, block) pair once")


def segments(tile_base, T, G, R):
    """(group, user, first tile, end tile) of every segment of the equal tile
    ranges cut at user boundaries."""
    Tg = (T + 4 * G - 1) // (4 * G) * 4
    out = []
    for g in range(G):
        s0, s1 = g * Tg, min(T, g * Tg + Tg)
        if s0 >= s1:
            continue
        u = int(user_of(tile_base, s0))
        while True:
            ua, ub = int(tile_base[u]), int(tile_base[u + 1])
            t0, te = max(s0, ua), min(s1, ub)
            if te > t0:
                out.append((g, u, t0, te))
            if ub >= s1:
                break
            u += 1
    return Tg, out


def user_slots(tile_base, u, Tg):
    t0, t1 = int(tile_base[u]), int(tile_base[u + 1])
    if t1 <= t0:
        return 0, 0
    return t0 // Tg + u, (t1 - 1) // Tg + 1 + u


def replay(lengths, d, k, backward=True):
    offsets, tile_base, T = schedule(lengths)
    R, N = len(lengths), int(offsets[-1])
    L = layout(R, N, d, k, backward)
    fw, bw = _lib_sizes(R, N, d, k)
    assert layout(R, N, d, k, False)["total"] == fw, "forward layout restated wrongly"
    if backward and bw is not None:
        assert L["total"] == bw, "backward layout restated wrongly"
    # (a backward shape the library refuses, k = 256 at d = 128, is still
    # replayed: its layout follows the same rules as the pinned shapes)
    S = L["size"]
    check(T <= L["tiles_max"], "tile count within tiles_max")
    CPR = d // 8
    if T == 0:
        return L

    # ---- pass 1 with resident queries: the row loads of every tile slot
    t = np.arange(T)
    u = user_of(tile_base, t)
    first = offsets[u]
    check(offsets[u + 1] > first, "a user with tiles has a token")
    tok = first[:, None] + (t - tile_base[u])[:, None] * TILE + np.arange(TILE)[None, :]
    live = tok < offsets[u + 1][:, None]
    # slots with a token read their row of H; the others the workspace's zero
    # row (masked batches: their mask byte from the user's first token)
    check((tok[live] >= 0) & (tok[live] < N), "pass 1 row loads inside H")
    check(tok[live] * d + (CPR - 1) * 8 + 7 < N * d, "pass 1 chunk loads inside H")
    check((CPR - 1) * 8 + 7 < S["zrow"] * 2, "pass 1 zero-row chunk loads inside the zero row")
    tc = np.where(live, tok, first[:, None])
    check((tc >= 0) & (tc < N), "pass 1 mask byte loads inside the mask")
    check((t[:, None] * TILE + np.arange(TILE)) * d + d - 1 < S["h16"], "fp16 rows inside the workspace")
    check(t * TILE + TILE - 1 < S["nl"], "-l pairs inside the workspace")
    # the tile's token count from 32-bit tile arithmetic (user's tile count and
    # last-tile count) equals the count of live slots
    n_u = offsets[u + 1] - first
    nt = (n_u + TILE - 1) // TILE
    last = n_u - (nt - 1) * TILE
    trel = t - tile_base[u]
    cnt = np.where(trel < nt - 1, TILE, np.where(trel == nt - 1, last, 0))
    check(np.array_equal(cnt, live.sum(axis=1)), "pass 1 tile token counts")

    # ---- pass 2: groups, segments, slots and stage reads
    P, G = L["n_pblocks"], L["p2_groups"]
    group_grid(P, G)
    Tg, segs = segments(tile_base, T, G, R)
    for g, uu, t0, te in segs:
        check((te - t0) % 4 == 0, "segments hold whole 4-tile stages")
        check(te <= T, "stage reads inside the tiles")
        # -l pieces: token i's pair and the next three, 4 bytes each; past the
        # last tile only the 4 zeroed words that follow the pairs
        last = (te * TILE - 1) + 3
        check(last <= T * TILE + 3, "-l piece reads end at most 4 words past the last tile")
        check(last < S["nl"], "-l piece reads inside the workspace")
        check(g + uu < L["parts_max"], "pass-2 slot inside part_u")
    covered = sum(te - t0 for _, _, t0, te in segs)
    check(covered == T, "the segments cover every tile once")
    # finalize / presum / bwd_user read each user's slot range
    for uu in range(R):
        c0, c1 = user_slots(tile_base, uu, Tg)
        check(c1 <= L["parts_max"], "user slots inside part_u")
        if R <= PRE_USERS and c1 - c0 > PRE_MIN:
            n = c1 - c0
            heads = [c0 + n * s // PRE_SPLIT for s in range(PRE_SPLIT + 1)]
            check(heads[-1] == c1 and all(a < b for a, b in zip(heads, heads[1:])), "pre-sum sub-ranges")
    if not backward:
        return L

    # ---- per-user step and packing of Z
    nrb = k // 32
    check((R - 1) * k + (nrb - 1) * 32 + 31 < R * k, "per-user rows")
    check(R * nrb <= S["bzmax"], "block maxima")
    # ---- dH: one workgroup per 4 tiles of one user
    quads = np.arange(max(1, L["tiles_max"] // ALIGN_T))
    q = quads[4 * quads < T]
    uq = user_of(tile_base, 4 * q)
    check(user_of(tile_base, 4 * q + 3) == uq, "a quad's tiles belong to one user")
    for w in range(4):
        tile = 4 * q + w
        tok0 = offsets[uq] + (tile - tile_base[uq]) * TILE
        count = np.clip(offsets[uq + 1] - tok0, 0, TILE)
        check(np.where(count > 0, tok0 + count - 1, 0) < N, "dH rows inside dH")
        check(tile * TILE + TILE - 1 < S["bdelta"], "delta inside the workspace")
        check((tile * TILE + TILE - 1) * d + d - 1 < S["h16"], "dH reads of the fp16 rows")
    check((uq * k + k - 1) * d + d - 1 < S["bz16"], "Z rows of the tile's user")
    # ---- E: prototype-major groups
    EP, EG, EW = L["e_pblocks"], L["e_groups"], L["e_waves"]
    group_grid(EP, EG)
    check(EP * EW * 32 == k, "E blocks cover the prototypes")
    ETg, esegs = segments(tile_base, T, EG, R)
    for g, uu, t0, te in esegs:
        check(g + uu < EG + R, "E slot inside the partials")
        check(te <= T, "E tile reads")
    check(sum(te - t0 for _, _, t0, te in esegs) == T, "E segments cover every tile")
    # bwd_ereduce walks the same slots, users in order
    for uu in range(R):
        c0, c1 = user_slots(tile_base, uu, ETg)
        check(c1 <= EG + R, "E-reduce slots")
        check(max(c1 - 1, 0) * k * d + k * d - 1 < S["bepart"], "E-reduce reads")
    # ---- outer products
    per = (k + L["o_chunks"] - 1) // L["o_chunks"]
    rk = max(32, (per + 31) // 32 * 32)
    check((k + rk - 1) // rk <= L["o_chunks"], "dWk chunks inside the partials")
    check((R * k + OUTER_ROWS - 1) // OUTER_ROWS <= L["o_chunks"], "dWv chunks inside the partials")
    return L


SHAPES = [
    ([700, 0, 2049, 33], 128, 256),      # the smoke inputs
    ([700, 0, 2049, 33], 128, 1024),
    ([700, 0, 2049, 33], 64, 256),
    ([1], 128, 256), ([33], 128, 256), ([96], 128, 256), ([127], 128, 64), ([128], 128, 256),
    ([129], 64, 320), ([0, 0, 0], 128, 512), ([0, 1, 31, 33, 700, 2049, 4], 128, 320),
    ([100_000] * 40, 128, 1024),
    ([1500, 0, 33, 700], 128, 4096), ([60000, 5], 128, 1024), ([20000, 3, 0, 1500], 64, 128),
]


@pytest.mark.parametrize("lengths,d,k", SHAPES)
def test_replay_in_bounds(lengths, d, k):
    replay(lengths, d, k)


@pytest.mark.parametrize("seed", range(6))
def test_replay_random_ragged(seed):
    rng = np.random.default_rng(seed)
    R = int(rng.integers(1, 300))
    lens = rng.integers(0, 3000, size=R)
    lens[rng.random(R) < 0.1] = 0
    d = int(rng.choice([64, 128]))
    k = int(rng.choice([64, 128, 256, 320, 512, 1024, 2048]))
    replay(lens.tolist(), d, k)


def test_old_pass1_clamp_read_past_h():
    """The clamp pass 1 used before the fix (a tile's first slot) addressed
    rows past N for the smoke inputs, whose last user has 33 tokens: of its
    four tiles, the last two hold no token and start at rows N + 31 and
    N + 63."""
    offsets, tile_base, T = schedule([700, 0, 2049, 33])
    N = int(offsets[-1])
    t = np.arange(T)
    u = user_of(tile_base, t)
    t0 = offsets[u] + (t - tile_base[u]) * TILE
    old_max = int(t0.max())
    assert old_max == N + 63
    assert math.ceil(33 / 128) * 4 == 4
    # the fixed clamp stays inside H
    first = offsets[u]
    tok = t0[:, None] + np.arange(TILE)[None, :]
    tc = np.where(tok < offsets[u + 1][:, None], tok, first[:, None])
    assert int(tc.max()) == N - 1


# ------------------------------------------------------------- fp32 path
def replay_f32(lengths, d, k, masked=False):
    """The fp32 kernels' indices (pass1_f32: eight threads per token slot, 32
    slots per workgroup, queries staged 64 rows at a time; pass2_f32: one
    workgroup per (chunk, 64-prototype block), rows loaded from addresses
    clamped to the user's rows) against their buffers: H and the mask [N],
    the fp32 queries [k, d], lse32 [tiles_max * 32] and the chunk partials."""
    offsets, tile_base, T = schedule(lengths)
    R, N = len(lengths), int(offsets[-1])
    span = TILE * ALIGN_T
    tiles_max = (N + (span - 1) * R) // span * ALIGN_T
    check(T <= tiles_max, "tiles within tiles_max")
    n_lse = tiles_max * TILE
    # pass1_f32: grid ceil(tiles_max * 32 / 32) workgroups of 256 threads
    g1 = (tiles_max * TILE + 31) // 32
    tid = np.arange(256)
    part = tid % 8
    for b in range(g1):
        slot = b * 32 + tid // 8
        tile = slot // TILE
        row = slot % TILE
        live = tile < T
        if not live.any():
            continue
        u = user_of(tile_base, tile[live])
        tok0 = offsets[u] + (tile[live] - tile_base[u]) * TILE
        count = np.minimum(TILE, offsets[u + 1] - tok0)
        valid = row[live] < count
        tok = (tok0 + row[live])[valid]
        check((tok >= 0) & (tok < N), "pass1_f32: H row / mask byte in range")
        check(tok * d + d <= N * d, "pass1_f32: H row end in range")
        writes = slot[live & (part == 0)]
        check(writes < n_lse, "pass1_f32: lse32 index in range")
    for j0 in range(0, k, 64):
        e = np.arange(64 * (d // 4))
        r = e // (d // 4)
        check((j0 + r) * d + 4 * (e % (d // 4)) + 4 <= k * d, "pass1_f32: query staging in range")
    # pass2_f32: chunks of CT tiles per user, k / 64 prototype blocks
    nblk = k // 64
    want = (tiles_max * nblk + 255) // 256
    ct = min(max(want, 4), 64)
    CT = (ct + ALIGN_T - 1) // ALIGN_T * ALIGN_T
    chunks_max = (tiles_max + (CT - 1) * R) // CT
    tiles_u = np.diff(tile_base)
    chunks_u = (tiles_u + CT - 1) // CT
    check(chunks_u.sum() <= chunks_max, "pass2_f32: chunks within chunks_max")
    nv = TILE * d // 4 // 256
    for u in range(R):
        lo, hi = int(offsets[u]), int(offsets[u + 1])
        for ci in range(int(chunks_u[u])):
            nt = min(CT, int(tiles_u[u]) - ci * CT)
            check(nt > 0 and hi > lo, "pass2_f32: a chunk's user has a token")
            for it in range(nt):
                tok0 = lo + (ci * CT + it) * TILE
                e = tid[:, None] + 256 * np.arange(nv)[None, :]
                tok = tok0 + e // (d // 4)
                tc = np.minimum(tok, hi - 1)
                check((tc >= lo) & (tc < N), "pass2_f32: clamped row in the user's rows")
                check(tc * d + 4 * (e % (d // 4)) + 4 <= N * d, "pass2_f32: row piece in range")
                lse_idx = (int(tile_base[u]) + ci * CT + it) * TILE + np.arange(TILE)
                check(lse_idx < n_lse, "pass2_f32: lse32 read in range")


@pytest.mark.parametrize("lengths,d,k", [
    ([4096], 64, 64),                      # C1
    ([700, 0, 2049, 33], 128, 192),
    ([1, 0, 0, 31, 32, 33, 129], 64, 128),
    ([0, 0, 5], 128, 64),
    ([100000], 128, 1024),
])
def test_replay_f32_in_bounds(lengths, d, k):
    replay_f32(lengths, d, k)


@pytest.mark.parametrize("seed", range(4))
def test_replay_f32_random_ragged(seed):
    rng = np.random.default_rng(100 + seed)
    R = int(rng.integers(1, 120))
    lens = rng.integers(0, 2500, size=R)
    lens[rng.random(R) < 0.15] = 0
    replay_f32(lens.tolist(), int(rng.choice([64, 128])), int(rng.choice([64, 128, 192, 256, 1024])))
