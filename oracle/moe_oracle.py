"""Plain, slow, fp64 CPU oracle of the MoE layer hot path.

TEST INFRASTRUCTURE ONLY: imported by the tests, by the package entry file's
smoke check and by the benchmark's CPU-baseline leg; never by the product path.
It shares no code, table or helper with the HIP path.

Sources ("the pages"):
  [UR]  project_6 "Upstream Reference: Deep-Spark xllm + vllm" page:
        section "Call Chain: MoE topk_softmax on BI-V100" (a fused softmax +
        top-k op returning routing weights, expert ids and a token-expert
        index map) and section "File Index" (the FusedMoE layer order
        gate -> topk -> expand -> gemm1 -> act -> gemm2 -> combine;
        silu_and_mul as the activation).
  [B70] b70-optimization-lab note "MTP1 M2 compact scheduler closure"
        (2026-07-16): the design paragraph (each local expert's row count and
        remapped-row prefix derived from topk_ids plus expert_map; occurrence
        0 and 8 own the two M=8 tiles in the all-duplicate case; expert-grouped
        activation layout with cross-row weight reuse), the correctness
        paragraph (route patterns, valid all-remote EP rank, an independent
        fixed-M1 arithmetic oracle and a direct slot-order gather).

Every function computes the plain definition of its step.  Grouping, tiling
and compaction in the method only reach the same per-route result faster, so
the FFN here is evaluated route by route (the fixed-M1 oracle of [B70]) and
the combine is a direct slot-order gather ([B70]).

Readings where the pages are silent (each is also listed in the design notes):
  * top-k ranks logits (softmax is strictly increasing, so this is the exact
    softmax order); equal values go to the lower expert index; the K ids of a
    row are listed best first.
  * token_expert_indices[t, k] = k*T + t (the slot's source row in a k-major
    expanded layout, the convention of the vLLM lineage named in [UR]).
  * renormalisation divides by the sum over all K chosen experts, remote ones
    included (it is a gate property, computed before any EP split).
  * rows of one local expert are ordered by slot index s = t*K + k; every slot
    gets its own row, duplicates included; rows beyond R in row_to_slot are -1.
  * W1[e] is [2F, H] with the gate half (through SiLU) in rows [0, F) and the
    up half in rows [F, 2F); W2[e] is [H, F].
  * the combine on an EP rank is a partial sum over local routes only, not
    renormalised; an all-remote token gets exact zeros.
  * MXFP4 follows the OCP Microscaling (MX) v1.0 definition: e2m1 elements
    (sign, 2 exponent bits with bias 1, 1 mantissa bit), two per byte with
    element 2i in the low nibble, one e8m0 scale 2^(e-127) per 32 consecutive
    elements along the reduction dimension.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "decode_bf16", "decode_mxfp4", "decode_weights", "topk_softmax", "topk_sigmoid", "route_compact", "route_align", "route_align_capacity",
    "tile_owners", "silu", "ffn_route", "ffn_rows", "grouped_ffn", "grouped_ffn_rows",
    "combine", "moe_layer", "E2M1_VALUES",
]

# ---------------------------------------------------------------------------
# storage formats


def decode_bf16(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64.  Exact: a bf16 is the upper half
    of a float32, and every float32 is a float64."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


# e2m1 magnitudes for the three low bits of a code (OCP MX v1.0, FP4 E2M1)
E2M1_VALUES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)


def decode_mxfp4(codes, scales) -> np.ndarray:
    """MXFP4 -> float64.  codes [..., n/2] uint8 with element 2i in the low
    nibble of byte i and element 2i+1 in the high nibble; scales [..., n/32]
    uint8 e8m0, value 2^(e-127).  Returns [..., n]."""
    c = np.asarray(codes, dtype=np.uint8)
    s = np.asarray(scales, dtype=np.uint8)
    n = c.shape[-1] * 2
    assert s.shape[-1] * 32 == n, "one e8m0 scale per 32 elements"
    nib = np.empty(c.shape[:-1] + (n,), dtype=np.uint8)
    nib[..., 0::2] = c & 0x0F
    nib[..., 1::2] = c >> 4
    mag = E2M1_VALUES[nib & 0x7]
    val = np.where(nib & 0x8, -mag, mag)
    assert not np.any(s == 0xFF), "e8m0 0xFF is NaN"
    scale = np.ldexp(1.0, s.astype(np.int64) - 127)
    return val * np.repeat(scale, 32, axis=-1)


def decode_weights(w, w_scale, w_dtype: str, e: int) -> np.ndarray:
    """Expert e's weight matrix as float64, from f32 / bf16-bits / MXFP4 storage."""
    if w_dtype == "f32":
        return np.asarray(w[e], dtype=np.float64)
    if w_dtype == "bf16":
        return decode_bf16(w[e])
    if w_dtype == "mxfp4":
        return decode_mxfp4(w[e], w_scale[e])
    raise ValueError(w_dtype)


def _as_f64(a, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.asarray(a, dtype=np.float64)
    if dtype == "bf16":
        return decode_bf16(a)
    raise ValueError(dtype)


# ---------------------------------------------------------------------------
# step 1: fused top-k softmax gate  ([UR] "Call Chain: MoE topk_softmax")


def topk_softmax(logits, K: int, renormalize: bool, logits_dtype: str = "f32"):
    """Softmax over each row's E logits, then the K best experts.

    Returns (weights float64 [T,K], ids int32 [T,K], token_expert_indices
    int32 [T,K]).  Order: larger logit first; equal logits -> lower index
    first.  weights[t,k] = softmax(row t)[ids[t,k]], divided by the sum of the
    row's K chosen probabilities when renormalize is set."""
    v = _as_f64(logits, logits_dtype)
    T, E = v.shape
    assert 1 <= K <= E
    assert np.all(np.isfinite(v)), "logits must be finite"
    m = v.max(axis=1, keepdims=True)
    ex = np.exp(v - m)
    p = ex / ex.sum(axis=1, keepdims=True)
    j = np.broadcast_to(np.arange(E), v.shape)
    # np.lexsort: last key is primary -> sort by -v ascending, then by j ascending
    order = np.lexsort((j, -v), axis=-1)
    ids = order[:, :K].astype(np.int32)
    w = np.take_along_axis(p, ids.astype(np.int64), axis=1)
    if renormalize:
        w = w / w.sum(axis=1, keepdims=True)
    tei = (np.arange(K, dtype=np.int64)[None, :] * T + np.arange(T, dtype=np.int64)[:, None]).astype(np.int32)
    return w, ids, tei


def topk_sigmoid(logits, K: int, renormalize: bool, logits_dtype: str = "f32"):
    """Sigmoid-scoring gate ([UR] "File Index": a sigmoid variant of the
    top-k kernel for DeepSeek-style routing, named but not defined there).

    Reading: each expert is scored on its own, s_j = 1 / (1 + exp(-v_j)); the
    K best scores (= the K largest logits, s being increasing; equal logits ->
    lower index first) are chosen in descending order; weights[t,k] =
    s[ids[t,k]], divided by the sum of the row's K chosen scores when
    renormalize is set.  Returns (weights float64, ids int32, token_expert_
    indices int32) like topk_softmax."""
    v = _as_f64(logits, logits_dtype)
    T, E = v.shape
    assert 1 <= K <= E
    assert np.all(np.isfinite(v)), "logits must be finite"
    with np.errstate(over="ignore"):
        s = 1.0 / (1.0 + np.exp(-v))
    j = np.broadcast_to(np.arange(E), v.shape)
    order = np.lexsort((j, -v), axis=-1)
    ids = order[:, :K].astype(np.int32)
    w = np.take_along_axis(s, ids.astype(np.int64), axis=1)
    if renormalize:
        w = w / w.sum(axis=1, keepdims=True)
    tei = (np.arange(K, dtype=np.int64)[None, :] * T + np.arange(T, dtype=np.int64)[:, None]).astype(np.int32)
    return w, ids, tei


# ---------------------------------------------------------------------------
# step 2: route compaction  ([B70] design paragraph)


def route_compact(topk_ids, expert_map, E_local: int):
    """Derive, for one EP rank, each local expert's row count, the exclusive
    row prefix and the slot <-> row permutation of the expert-grouped layout.

    Slot s = t*K + k carries global id topk_ids.flat[s]; its local id is
    l = expert_map[id] (identity when expert_map is None), -1 meaning remote.
    Rows of the grouped layout are ordered by (l, s): a stable counting sort.

    Returns counts [E_local], offsets [E_local+1] (offsets[E_local] = R, the
    number of local slots), slot_to_row [N] (-1 for remote slots) and
    row_to_slot [N] (-1 beyond R), all int32, N = T*K.
    """
    ids = np.asarray(topk_ids, dtype=np.int64).reshape(-1)
    N = ids.size
    if expert_map is None:
        assert np.all((ids >= 0) & (ids < E_local))
        loc = ids
    else:
        emap = np.asarray(expert_map, dtype=np.int64)
        assert np.all((ids >= 0) & (ids < emap.size)), "topk_ids out of range"
        assert np.all((emap >= -1) & (emap < E_local)), "expert_map out of range"
        loc = emap[ids]
    is_local = loc >= 0
    counts = np.bincount(loc[is_local], minlength=E_local).astype(np.int64)
    offsets = np.zeros(E_local + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    R = int(offsets[-1])
    local_slots = np.flatnonzero(is_local)
    # stable sort of the local slots by local id keeps slot order inside an expert
    grouped = local_slots[np.argsort(loc[local_slots], kind="stable")]
    row_to_slot = np.full(N, -1, dtype=np.int64)
    row_to_slot[:R] = grouped
    slot_to_row = np.full(N, -1, dtype=np.int64)
    slot_to_row[grouped] = np.arange(R)
    return (counts.astype(np.int32), offsets.astype(np.int32),
            slot_to_row.astype(np.int32), row_to_slot.astype(np.int32))


def route_align_capacity(N: int, E_local: int, block_size: int):
    """Sizes the block-aligned layout can reach: padded rows and blocks."""
    return N + E_local * (block_size - 1), -(-N // block_size) + E_local


def route_align(topk_ids, expert_map, E_local: int, block_size: int):
    """Block-aligned (padded) variant of the expert-grouped layout ([UR] "File
    Index": a block-alignment kernel for the scatter).  Reading: every local
    expert's rows, in the same slot order as route_compact, start on a
    multiple of block_size; the unused tail rows of an expert's last block
    are padding.

    Returns padded_offsets [E_local+1] (expert e owns padded rows
    [padded_offsets[e], padded_offsets[e+1]), a multiple of block_size
    apart), sorted_slots [cap_rows] (slot of each padded row, -1 for padding
    and past the end), block_expert [cap_blocks] (local expert of each
    block, -1 past the end) and slot_to_row [N] (padded row of each slot, -1
    for remote slots), all int32; the capacities come from
    route_align_capacity."""
    ids = np.asarray(topk_ids, dtype=np.int64).reshape(-1)
    N = ids.size
    counts, offsets, slot_to_row, row_to_slot = route_compact(ids, expert_map, E_local)
    bs = int(block_size)
    counts = counts.astype(np.int64)
    offsets = offsets.astype(np.int64)
    padded = -(-counts // bs) * bs
    poff = np.zeros(E_local + 1, dtype=np.int64)
    poff[1:] = np.cumsum(padded)
    cap_rows, cap_blocks = route_align_capacity(N, E_local, bs)
    sorted_slots = np.full(cap_rows, -1, dtype=np.int64)
    block_expert = np.full(cap_blocks, -1, dtype=np.int64)
    for e in range(E_local):
        sorted_slots[poff[e]:poff[e] + counts[e]] = row_to_slot[offsets[e]:offsets[e + 1]]
        block_expert[poff[e] // bs:poff[e + 1] // bs] = e
    s2r = slot_to_row.astype(np.int64)
    out_rows = np.full(N, -1, dtype=np.int64)
    local = np.flatnonzero(s2r >= 0)
    if local.size:
        e_of = np.searchsorted(offsets, s2r[local], side="right") - 1
        out_rows[local] = poff[e_of] + (s2r[local] - offsets[e_of])
    return (poff.astype(np.int32), sorted_slots.astype(np.int32), block_expert.astype(np.int32),
            out_rows.astype(np.int32))


def tile_owners(topk_ids, expert_map, E_local: int, BM: int):
    """Slots that own an M-tile of height BM: those whose occurrence index (the
    number of earlier slots routed to the same local expert) is a multiple of
    BM.  Returns a list of (slot, local expert, first row of the tile) in slot
    order.  [B70]: with M=2, top-6 and M=8 tiles, the all-duplicate case has
    tiles owned by occurrences 0 and 8."""
    ids = np.asarray(topk_ids, dtype=np.int64).reshape(-1)
    counts, offsets, slot_to_row, _ = route_compact(ids, expert_map, E_local)
    out = []
    for s in range(ids.size):
        r = int(slot_to_row[s])
        if r < 0:
            continue
        l = int(np.searchsorted(offsets, r, side="right") - 1)
        occ = r - int(offsets[l])
        if occ % BM == 0:
            out.append((s, l, r))
    return out


# ---------------------------------------------------------------------------
# steps 3-6: expand, GEMM1, silu_and_mul, GEMM2  ([UR] "File Index": FusedMoE)


def silu(g):
    """SiLU(g) = g / (1 + exp(-g)), evaluated without overflow for g << 0."""
    g = np.asarray(g, dtype=np.float64)
    out = np.empty_like(g)
    pos = g >= 0
    out[pos] = g[pos] / (1.0 + np.exp(-g[pos]))
    eg = np.exp(g[~pos])
    out[~pos] = g[~pos] * eg / (1.0 + eg)
    return out


def ffn_route(x_t, w1_e, w2_e):
    """One route (M=1): y = W2 (silu(W1_gate x) * (W1_up x)), all float64."""
    x_t = np.asarray(x_t, dtype=np.float64)
    F = w2_e.shape[1]
    assert w1_e.shape == (2 * F, x_t.size) and w2_e.shape[0] == x_t.size
    h = w1_e @ x_t
    act = silu(h[:F]) * h[F:]
    return w2_e @ act


def ffn_rows(x_rows, w1_e, w2_e):
    """ffn_route applied to each row of x_rows [m, H] (rows are independent;
    the matrix product only evaluates the m dot products of each output in
    one library call)."""
    x_rows = np.asarray(x_rows, dtype=np.float64)
    F = w2_e.shape[1]
    h = x_rows @ w1_e.T
    act = silu(h[:, :F]) * h[:, F:]
    return act @ w2_e.T


def grouped_ffn(x, x_dtype: str, K: int, w1, w2, w_dtype: str, counts, offsets, row_to_slot,
                w1_scale=None, w2_scale=None):
    """The expert FFN of every local route, written into the expert-grouped
    layout: y[r] = FFN_{expert of row r}(x[row_to_slot[r] // K]) for r < R.
    Returns float64 [R, H]."""
    xf = _as_f64(x, x_dtype)
    counts = np.asarray(counts)
    offsets = np.asarray(offsets)
    R = int(offsets[-1])
    H = xf.shape[1]
    y = np.zeros((R, H), dtype=np.float64)
    for e in range(counts.size):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        w1_e = decode_weights(w1, w1_scale, w_dtype, e)
        w2_e = decode_weights(w2, w2_scale, w_dtype, e)
        tokens = np.asarray(row_to_slot[lo:hi], dtype=np.int64) // K
        y[lo:hi] = ffn_rows(xf[tokens], w1_e, w2_e)
    return y


def grouped_ffn_rows(rows, x, x_dtype: str, K: int, w1, w2, w_dtype: str, offsets, row_to_slot,
                     w1_scale=None, w2_scale=None):
    """y at a sample of grouped rows only (for full-size checks): returns
    float64 [len(rows), H], computed one route at a time."""
    xf = _as_f64(x, x_dtype)
    offsets = np.asarray(offsets, dtype=np.int64)
    rows = np.asarray(rows, dtype=np.int64)
    out = np.zeros((rows.size, xf.shape[1]), dtype=np.float64)
    experts = np.searchsorted(offsets, rows, side="right") - 1
    for e in np.unique(experts):
        w1_e = decode_weights(w1, w1_scale, w_dtype, int(e))
        w2_e = decode_weights(w2, w2_scale, w_dtype, int(e))
        for i in np.flatnonzero(experts == e):
            out[i] = ffn_route(xf[int(row_to_slot[rows[i]]) // K], w1_e, w2_e)
    return out


# ---------------------------------------------------------------------------
# step 7: top-k weighted combine  ([B70] direct slot-order gather)


def combine(y, topk_weights, slot_to_row, T: int, K: int):
    """out[t] = sum over k ascending of w[t,k] * y[slot_to_row[t*K+k]], local
    slots only (remote slots, slot_to_row = -1, contribute nothing)."""
    y = np.asarray(y, dtype=np.float64)
    w = np.asarray(topk_weights, dtype=np.float64).reshape(T, K)
    s2r = np.asarray(slot_to_row).reshape(T, K)
    H = y.shape[1]
    out = np.zeros((T, H), dtype=np.float64)
    for t in range(T):
        for k in range(K):
            r = int(s2r[t, k])
            if r >= 0:
                out[t] += w[t, k] * y[r]
    return out


# ---------------------------------------------------------------------------
# the whole layer


def moe_layer(case):
    """Run every step on a synth.MoECase.  Returns a dict with the gate
    outputs (or the forced routes), the compaction arrays, y (grouped, f64)
    and out (f64 [T, H])."""
    if case.topk_ids is None:
        w, ids, tei = topk_softmax(case.logits, case.K, case.renormalize, case.logits_dtype)
    else:
        w = np.asarray(case.topk_weights, dtype=np.float64)
        ids = np.asarray(case.topk_ids, dtype=np.int32)
        tei = None
    counts, offsets, s2r, r2s = route_compact(ids, case.expert_map, case.E_local)
    y = grouped_ffn(case.x, case.x_dtype, case.K, case.w1, case.w2, case.w_dtype, counts, offsets, r2s,
                    case.w1_scale, case.w2_scale)
    # the combine uses the gate weights as the GPU receives them: float32
    w32 = w.astype(np.float32)
    out = combine(y, w32, s2r, case.T, case.K)
    return dict(topk_weights=w, topk_ids=ids, token_expert_indices=tei, counts=counts, offsets=offsets,
                slot_to_row=s2r, row_to_slot=r2s, y=y, out=out)
