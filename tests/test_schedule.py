"""Work decomposition on the CPU: the functions the kernels use to map a
workgroup (and a persistent workgroup's rounds) to work items, called through
libattn09_sched.so (host code compiled from the same attn_sched.h).  Each grid
must visit every work item exactly once, for the CU counts the host accepts.

The pages' decomposition is one workgroup per (query tile, head, batch),
located through the prefix sums for packed sequences (TileLang tutorial,
sections 3.0 and 5.3); off-by-one errors at the causal boundary and in the
varlen guard are where such grids go wrong (its sections 5.2 and 5.3).
"""

import ctypes
import os

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "exact_attention_09_amd", "libattn09_sched.so")

BM_FWD = 256     # query rows per forward workgroup (the ping-pong kernel)
TILE_BWD = 128   # rows per backward tile
CU_COUNTS = [256, 304, 80, 8]   # persistent grids of 8 x (CUs / 8) workgroups

I = ctypes.c_int
P = ctypes.POINTER(ctypes.c_int)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        from exact_attention_09_amd import build
        build.build_sched()
    L = ctypes.CDLL(LIB)
    L.sched_xcd_remap.restype = I
    L.sched_xcd_remap.argtypes = [I, I]
    L.sched_dense_item.argtypes = [I, I, I, I, P, P, P]
    L.sched_persist_dense_item.restype = I
    L.sched_persist_dense_item.argtypes = [I, I, I, I]
    L.sched_persist_listed_index.restype = ctypes.c_int64
    L.sched_persist_listed_index.argtypes = [I, I, I, ctypes.c_int64]
    L.sched_listed_locate.argtypes = [ctypes.c_void_p, I, I, ctypes.c_int64, I, P, P, P]
    L.sched_varlen_item.restype = I
    L.sched_varlen_item.argtypes = [ctypes.c_void_p, I, I, I, I, I, I, P, P, P]
    L.sched_varlen_tile.restype = I
    L.sched_varlen_tile.argtypes = [ctypes.c_void_p, I, I, I, I, P, P, P]
    L.sched_varlen_ranked.restype = I
    L.sched_varlen_ranked.argtypes = [ctypes.c_void_p, I, I, I, I, P, P, P]
    L.sched_bwd_dkdv_item.argtypes = [I, I, I, I, P, P]
    L.sched_bwd_dq_item.argtypes = [I, I, I, I, P, P]
    L.sched_ranked_max_seqs.restype = I
    return L


def outs(n):
    return [ctypes.c_int() for _ in range(n)]


def cu_of(lengths):
    return np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)


def tiles(lengths, rows):
    return [-(-int(L) // rows) for L in lengths]


LENGTH_SETS = {
    "workload-like": [2710, 2303, 3246, 2048, 3820, 3028, 3951, 1236],
    "edges": [0, 1, 2, 255, 256, 257, 511, 512, 513, 0],
    "one-empty": [0],
    "one-token": [1],
    "long": [300000, 1, 5000],      # more than 1024 tiles in one sequence
}


def random_lengths(seed, n, hi):
    rng = np.random.default_rng(seed)
    L = rng.integers(0, hi, n)
    L[rng.random(n) < 0.1] = 0
    return [int(x) for x in L]


# ------------------------------------------------------------------ forward

@pytest.mark.parametrize("n", [1, 7, 8, 9, 255, 256, 1000, 4097])
def test_xcd_remap_is_a_bijection_with_contiguous_xcd_ranges(lib, n):
    grid = 8 * -(-n // 8)
    got = {}
    for wg in range(grid):
        v = lib.sched_xcd_remap(wg, n)
        if v >= 0:
            assert v not in got, f"item {v} twice"
            got[v] = wg % 8
    assert sorted(got) == list(range(n))
    per = -(-n // 8)
    for v, x in got.items():
        assert x * per <= v < (x + 1) * per  # one contiguous range per XCD


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,H,tph", [(1, 32, 32), (4, 16, 8), (2, 3, 5)])
def test_dense_item_covers_every_tile(lib, B, H, tph, causal):
    b, h, t = outs(3)
    seen = set()
    for v in range(B * H * tph):
        lib.sched_dense_item(v, tph, H, int(causal), b, h, t)
        key = (b.value, h.value, t.value)
        assert 0 <= key[0] < B and 0 <= key[1] < H and 0 <= key[2] < tph
        assert key not in seen
        seen.add(key)
        if v % tph == 0:  # a head's first item is its heaviest tile under a causal mask
            assert t.value == (tph - 1 if causal else 0)
    assert len(seen) == B * H * tph


@pytest.mark.parametrize("cus", CU_COUNTS)
@pytest.mark.parametrize("mult", [1, 2, 4, 5])
def test_persistent_dense_visits_each_item_once(lib, cus, mult):
    C = cus // 8
    work = 8 * C * mult  # the host takes the persistent grid only for a multiple of 8 C
    per = work // 8
    seen = {}
    for blk in range(8 * C):
        r = 0
        while True:
            v = lib.sched_persist_dense_item(blk, r, C, work)
            if v < 0:
                break
            assert v not in seen, f"item {v} twice"
            x = blk % 8
            assert x * per <= v < (x + 1) * per, "an item left its XCD's range"
            seen[v] = blk
            r += 1
        assert r == mult
    assert sorted(seen) == list(range(work))


def test_persistent_causal_pairing_balances_the_headline(lib):
    """B=1, H=32, 8192 rows (32 tiles of 256) causal on 256 CUs: every
    workgroup gets the same number of key tiles (heavy and light paired)."""
    H, tph, C = 32, 32, 32
    work = H * tph
    b, h, t = outs(3)
    load = []
    for blk in range(8 * C):
        units, r = 0, 0
        while (v := lib.sched_persist_dense_item(blk, r, C, work)) >= 0:
            lib.sched_dense_item(v, tph, H, 1, b, h, t)
            units += t.value + 1  # tile t sees t + 1 tiles of 256 keys
            r += 1
        load.append(units)
    assert min(load) == max(load) == 66


def run_listed(lib, lengths, H, cus):
    """Enumerate the persistent varlen grid; return the visited (seq, tile,
    head) items in visiting order per workgroup."""
    C = cus // 8
    hpx = H // 8
    st = np.asarray(tiles(lengths, BM_FWD), np.int32)
    B = len(lengths)
    v_items = hpx * int(st.sum())
    seq, tile, head = outs(3)
    visits = []
    for blk in range(8 * C):
        r = 0
        while True:
            f = lib.sched_persist_listed_index(blk, r, C, v_items)
            if f == -1:
                break
            if f >= 0:
                lib.sched_listed_locate(st.ctypes.data, B, hpx, f, blk % 8, seq, tile, head)
                visits.append((blk, f, seq.value, tile.value, head.value))
            else:
                assert f == -2
            r += 1
        assert r == -(-v_items // C)  # every workgroup runs the same number of rounds
    return visits, st


@pytest.mark.parametrize("cus", CU_COUNTS)
@pytest.mark.parametrize("name", sorted(LENGTH_SETS))
def test_persistent_listed_visits_each_item_once(lib, name, cus):
    lengths = LENGTH_SETS[name]
    H = 16
    visits, st = run_listed(lib, lengths, H, cus)
    want = {(i, t, h) for i, n in enumerate(st) for t in range(n) for h in range(H)}
    got = [(s, t, h) for _, _, s, t, h in visits]
    assert len(got) == len(set(got)), "an item visited twice"
    assert set(got) == want
    hpx = H // 8
    for blk, f, s, t, h in visits:
        x = blk % 8
        assert x * hpx <= h < (x + 1) * hpx, "a head left its XCD"


@pytest.mark.parametrize("seed", [1, 2])
def test_persistent_listed_many_sequences(lib, seed):
    """1024 sequences (the most the listed order takes), mostly short, with
    empty and one-token ones."""
    lengths = random_lengths(seed, 1024, 700)
    lengths[:4] = [0, 1, 256, 257]
    H = 8
    visits, st = run_listed(lib, lengths, H, 256)
    want = {(i, t, h) for i, n in enumerate(st) for t in range(n) for h in range(H)}
    got = [(s, t, h) for _, _, s, t, h in visits]
    assert len(got) == len(set(got)) and set(got) == want


def test_listed_order_is_heaviest_first(lib):
    """Within an XCD's list, tile indices never increase with f."""
    lengths = LENGTH_SETS["workload-like"]
    visits, _ = run_listed(lib, lengths, 32, 256)
    for x in range(8):
        mine = sorted((f, t) for blk, f, s, t, h in visits if blk % 8 == x)
        ts = [t for _, t in mine]
        assert ts == sorted(ts, reverse=True)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("name", sorted(LENGTH_SETS))
def test_dispatched_varlen_visits_each_item_once(lib, name, causal):
    lengths = LENGTH_SETS[name]
    cu = cu_of(lengths)
    T, B, H = int(cu[-1]), len(lengths), 4
    tph = T // BM_FWD + B  # the host's upper bound of tiles per head
    h, s, t = outs(3)
    got = []
    for v in range(H * tph):
        if lib.sched_varlen_item(cu.ctypes.data, B, T, BM_FWD, tph, int(causal), v, h, s, t):
            got.append((s.value, t.value, h.value))
    want = {(i, tt, hh) for i, n in enumerate(tiles(lengths, BM_FWD)) for tt in range(n) for hh in range(H)}
    assert len(got) == len(set(got)) and set(got) == want


def test_malformed_prefix_sums_stay_in_range(lib):
    """Prefix sums outside [0, T] or decreasing are clamped: every located
    tile lies inside the tensors."""
    cu = np.array([0, 500, 300, 5000, -7, 900], np.int32)
    T, B, H = 900, 5, 2
    tph = T // BM_FWD + B
    h, s, t = outs(3)
    for v in range(H * tph):
        if lib.sched_varlen_item(cu.ctypes.data, B, T, BM_FWD, tph, 1, v, h, s, t):
            a = min(max(int(cu[s.value]), 0), T)
            e = min(max(int(cu[s.value + 1]), a), T)
            assert 0 <= a + BM_FWD * t.value < e <= T


# ------------------------------------------------------------------ backward

@pytest.mark.parametrize("name", sorted(LENGTH_SETS))
def test_backward_varlen_tiles(lib, name):
    lengths = LENGTH_SETS[name]
    cu = cu_of(lengths)
    T, B = int(cu[-1]), len(lengths)
    s0, ln, t = outs(3)
    got = []
    for vt in range(T // TILE_BWD + B):
        if lib.sched_varlen_tile(cu.ctypes.data, B, T, vt, TILE_BWD, s0, ln, t):
            got.append((s0.value, ln.value, t.value))
    want = {(int(cu[i]), L, tt) for i, L in enumerate(lengths) for tt in range(-(-L // TILE_BWD))}
    assert len(got) == len(set(got)) and set(got) == want


@pytest.mark.parametrize("name", ["workload-like", "edges", "one-token", "random"])
def test_backward_ranked_order(lib, name):
    """Causal varlen backward: items listed by level (work), heaviest first;
    every (sequence, level) pair once, so every key tile (dK/dV: tile n -
    level) and every query tile (dQ: tile level - 1) once."""
    lengths = random_lengths(9, 60, 3000) if name == "random" else LENGTH_SETS[name]
    assert len(lengths) <= lib.sched_ranked_max_seqs()
    cu = cu_of(lengths)
    T, B = int(cu[-1]), len(lengths)
    s0, ln, lev = outs(3)
    got, levels = [], []
    f = 0
    while lib.sched_varlen_ranked(cu.ctypes.data, B, T, f, TILE_BWD, s0, ln, lev):
        got.append((s0.value, ln.value, lev.value))
        levels.append(lev.value)
        f += 1
    assert levels == sorted(levels, reverse=True)
    want = {(int(cu[i]), L, r) for i, L in enumerate(lengths) for r in range(1, -(-L // TILE_BWD) + 1)}
    assert len(got) == len(set(got)) and set(got) == want


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("nb,ntiles", [(32, 64), (8, 1), (3, 7)])
def test_backward_dense_items(lib, nb, ntiles, causal):
    """dK/dV: (key tile, b * Hkv + kv head); dQ: (b * H + h, query tile).
    Non-causal grids go through xcd_remap (padded to a multiple of 8)."""
    n = nb * ntiles
    grid = n if causal else 8 * -(-n // 8)
    a, b = outs(2)
    for fn, order in ((lib.sched_bwd_dkdv_item, "kt first"), (lib.sched_bwd_dq_item, "bh first")):
        seen = set()
        for blk in range(grid):
            item = blk if causal else lib.sched_xcd_remap(blk, n)
            if item < 0:
                continue
            fn(item, nb, ntiles, int(causal), a, b)
            key = (a.value, b.value)
            seen.add(key)
        if order == "kt first":
            assert seen == {(kt, bk) for kt in range(ntiles) for bk in range(nb)}
        else:
            assert seen == {(bh, t) for bh in range(nb) for t in range(ntiles)}
        assert len(seen) == n
