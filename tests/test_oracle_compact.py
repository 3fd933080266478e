"""Pins of the oracle's route compaction (CPU only).

Source: b70-optimization-lab note "MTP1 M2 compact scheduler closure"
(2026-07-16), design paragraph (row count and remapped-row prefix of each
local expert from topk_ids plus expert_map, tile ownership by occurrence) and
correctness paragraph (the seven route patterns, a valid all-remote EP rank).
"""
import json
import os

import numpy as np
import pytest

import oracle
import synth

E_LOCAL = 40


def _contig_ids(pattern):
    """Pattern of local ids (None = remote) -> global ids under the contiguous
    map (local i <-> global 40 + i); remote slots use global id 200."""
    return np.array([[200 if l is None else 40 + l for l in row] for row in synth.DECODE_PATTERNS[pattern]],
                    dtype=np.int32)


def _offsets_from(counts_by_expert):
    counts = [0] * E_LOCAL
    for e, c in counts_by_expert.items():
        counts[e] = c
    offs = [0]
    for c in counts:
        offs.append(offs[-1] + c)
    return counts, offs


# Worked by hand: rows of one expert follow slot order s = t*6 + k, remote
# slots are -1, row_to_slot beyond R is -1.
HAND = {
    "same": ({3: 2, 17: 2, 29: 2},
             [0, -1, 2, -1, 4, -1, 1, -1, 3, -1, 5, -1],
             [0, 6, 2, 8, 4, 10] + [-1] * 6),
    "disjoint": ({1: 1, 5: 1, 12: 1, 18: 1, 22: 1, 35: 1},
                 [0, -1, 2, -1, 4, -1, 1, -1, 3, -1, 5, -1],
                 [0, 6, 2, 8, 4, 10] + [-1] * 6),
    "cross_row": ({2: 1, 10: 2, 20: 2, 30: 1},
                  [0, 1, 3, -1, -1, -1, 2, 4, 5, -1, -1, -1],
                  [0, 1, 6, 2, 7, 8] + [-1] * 6),
    "within_row_dup": ({4: 2, 6: 1, 8: 1, 15: 1, 25: 1},
                       [0, 1, 3, -1, -1, -1, 2, 4, 5, -1, -1, -1],
                       [0, 1, 6, 2, 7, 8] + [-1] * 6),
    "all_dup": ({7: 12}, list(range(12)), list(range(12))),
    "twelve_local": ({e: 1 for e in range(0, 34, 3)}, list(range(12)), list(range(12))),
    "all_remote": ({}, [-1] * 12, [-1] * 12),
}


@pytest.mark.parametrize("pattern", list(HAND))
def test_hand_patterns(pattern):
    emap = synth.contiguous_expert_map(256, E_LOCAL)
    counts, offsets, s2r, r2s = oracle.route_compact(_contig_ids(pattern), emap, E_LOCAL)
    hc, hs2r, hr2s = HAND[pattern]
    exp_counts, exp_offs = _offsets_from(hc)
    assert counts.tolist() == exp_counts
    assert offsets.tolist() == exp_offs
    assert s2r.tolist() == hs2r
    assert r2s.tolist() == hr2s


def test_page_worked_example_tile_owners(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "b70_all_duplicate_tiles.json")))
    ids = _contig_ids("all_dup")
    assert ids.shape == (g["T"], g["K"])
    emap = synth.contiguous_expert_map(256, E_LOCAL)
    counts, offsets, s2r, _ = oracle.route_compact(ids, emap, E_LOCAL)
    assert counts.max() == g["rows_on_expert"]
    owners = oracle.tile_owners(ids, emap, E_LOCAL, g["tile_rows"])
    occ = [r - int(offsets[l]) for (_, l, r) in owners]
    assert occ == g["owner_occurrences"]
    # more rows than two tiles: T=3, top-6 all duplicate, BM=16 -> occurrences 0 and 16
    ids3 = np.full((3, 6), 40 + 7, dtype=np.int32)
    owners3 = oracle.tile_owners(ids3, emap, E_LOCAL, 16)
    assert [s for (s, _, _) in owners3] == [0, 16]


def brute_force_compact(ids, emap, E_local):
    """Quadratic pure-Python version: occurrence = number of earlier slots with
    the same local id; row = (number of local slots with a smaller local id)
    + occurrence."""
    flat = [int(i) for i in np.asarray(ids).reshape(-1)]
    loc = [int(emap[i]) if emap is not None else i for i in flat]
    N = len(flat)
    counts = [sum(1 for l in loc if l == e) for e in range(E_local)]
    s2r = []
    for s in range(N):
        if loc[s] < 0:
            s2r.append(-1)
            continue
        before = sum(1 for l in loc if 0 <= l < loc[s])
        occ = sum(1 for s2 in range(s) if loc[s2] == loc[s])
        s2r.append(before + occ)
    r2s = [-1] * N
    for s, r in enumerate(s2r):
        if r >= 0:
            r2s[r] = s
    return counts, s2r, r2s


@pytest.mark.parametrize("seed", range(6))
def test_random_vs_brute_force(seed):
    rng = np.random.default_rng(100 + seed)
    Eg = int(rng.integers(2, 40))
    El = int(rng.integers(1, Eg + 1))
    T, K = int(rng.integers(1, 12)), int(rng.integers(1, 7))
    emap = synth.random_expert_map(Eg, El, seed) if seed % 2 else None
    if emap is None:
        El = Eg
    ids = rng.integers(0, Eg, size=(T, K)).astype(np.int32)
    counts, offsets, s2r, r2s = oracle.route_compact(ids, emap, El)
    bc, bs2r, br2s = brute_force_compact(ids, emap, El)
    assert counts.tolist() == bc
    assert s2r.tolist() == bs2r
    assert r2s.tolist() == br2s


def test_invariants_large():
    rng = np.random.default_rng(3)
    T, K, Eg, El = 4096, 8, 256, 32
    emap = synth.random_expert_map(Eg, El, 9)
    ids = rng.integers(0, Eg, size=(T, K)).astype(np.int32)
    counts, offsets, s2r, r2s = oracle.route_compact(ids, emap, El)
    loc = emap[ids.reshape(-1)]
    R = int((loc >= 0).sum())
    assert counts.sum() == R and offsets[-1] == R and offsets[0] == 0
    assert np.array_equal(np.diff(offsets), counts)
    assert np.array_equal(s2r[r2s[:R]], np.arange(R))
    assert np.all(r2s[R:] == -1)
    assert np.all(s2r[loc < 0] == -1)
    for e in range(El):
        block = r2s[offsets[e]:offsets[e + 1]]
        assert np.all(loc[block] == e)
        assert np.all(np.diff(block) > 0)  # slot order inside an expert
    # all-remote rank: nothing local
    ids_remote = np.flatnonzero(emap < 0)[rng.integers(0, Eg - El, size=(T, K))].astype(np.int32)
    counts, offsets, s2r, r2s = oracle.route_compact(ids_remote, emap, El)
    assert counts.sum() == 0 and np.all(offsets == 0) and np.all(s2r == -1) and np.all(r2s == -1)


def test_identity_map_equals_explicit_identity():
    rng = np.random.default_rng(4)
    ids = rng.integers(0, 16, size=(50, 4)).astype(np.int32)
    a = oracle.route_compact(ids, None, 16)
    b = oracle.route_compact(ids, np.arange(16, dtype=np.int32), 16)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


# ---------------------------------------------------------------------------
# block-aligned (padded) layout


def test_align_hand_example():
    # "same" pattern: local experts 3, 17, 29 with 2 rows each; blocks of 4
    emap = synth.contiguous_expert_map(256, 40)
    inv = np.flatnonzero(emap >= 0)
    rows = [[3, None, 17, None, 29, None]] * 2
    remote = np.flatnonzero(emap < 0)[0]
    ids = np.array([[inv[l] if l is not None else remote for l in r] for r in rows], np.int32)
    poff, sorted_slots, block_expert, s2r = oracle.route_align(ids, emap, 40, 4)
    want_poff = [0] * 4 + [4] * 14 + [8] * 12 + [12] * 11
    assert poff.tolist() == want_poff
    assert sorted_slots[:12].tolist() == [0, 6, -1, -1, 2, 8, -1, -1, 4, 10, -1, -1]
    assert np.all(sorted_slots[12:] == -1) and sorted_slots.size == 12 + 40 * 3
    assert block_expert[:3].tolist() == [3, 17, 29] and np.all(block_expert[3:] == -1)
    assert s2r.tolist() == [0, -1, 4, -1, 8, -1, 1, -1, 5, -1, 9, -1]


@pytest.mark.parametrize("seed", range(4))
def test_align_block_size_one_is_compaction(seed):
    rng = np.random.default_rng(seed)
    ids = rng.integers(0, 64, size=(37, 6)).astype(np.int32)
    emap = synth.random_expert_map(64, 20, seed=seed)
    counts, offsets, s2r_c, r2s_c = oracle.route_compact(ids, emap, 20)
    poff, sorted_slots, block_expert, s2r = oracle.route_align(ids, emap, 20, 1)
    R = int(offsets[-1])
    assert np.array_equal(poff, offsets) and np.array_equal(s2r, s2r_c)
    assert np.array_equal(sorted_slots[:R], r2s_c[:R]) and np.all(sorted_slots[R:] == -1)
    assert np.array_equal(block_expert[:R], np.repeat(np.arange(20), counts))


@pytest.mark.parametrize("bs", [2, 8, 16, 64])
def test_align_invariants(bs):
    rng = np.random.default_rng(bs)
    N_tok, K, Eg, El = 300, 8, 128, 48
    ids = rng.integers(0, Eg, size=(N_tok, K)).astype(np.int32)
    emap = synth.random_expert_map(Eg, El, seed=bs)
    poff, sorted_slots, block_expert, s2r = oracle.route_align(ids, emap, El, bs)
    loc = emap[ids.reshape(-1)]
    total = int(poff[-1])
    assert total % bs == 0 and np.all(np.diff(poff) % bs == 0)
    # every local slot exactly once, at the row slot_to_row names
    placed = sorted_slots[sorted_slots >= 0]
    assert np.array_equal(np.sort(placed), np.flatnonzero(loc >= 0))
    for s in np.flatnonzero(loc >= 0):
        assert sorted_slots[s2r[s]] == s
    assert np.all(s2r[loc < 0] == -1)
    # each block holds one expert's slots, padding only after them, slot order kept
    for b in range(total // bs):
        e = block_expert[b]
        seg = sorted_slots[b * bs:(b + 1) * bs]
        real = seg[seg >= 0]
        assert np.all(loc[real] == e)
        assert np.all(np.diff(real) > 0)
        k = real.size
        assert np.all(seg[:k] >= 0) and np.all(seg[k:] == -1)
    assert np.all(block_expert[total // bs:] == -1)


def test_align_capacity_closed_form_and_tight():
    # N slots over E_local experts padded to blocks of B: at most N + E_local*(B-1)
    # rows and ceil(N/B) + E_local blocks
    assert oracle.route_align_capacity(10, 3, 4) == (19, 6)
    assert oracle.route_align_capacity(0, 5, 8) == (35, 5)
    # reached exactly when every expert holds one route: E_local slots, each
    # padded to a full block
    El, B = 5, 4
    ids = np.arange(El, dtype=np.int32).reshape(1, El)
    poff, sorted_slots, block_expert, s2r = oracle.route_align(ids, None, El, B)
    assert poff[-1] == El * B == oracle.route_align_capacity(El, El, B)[0]
    assert len(sorted_slots) == oracle.route_align_capacity(El, El, B)[0]
