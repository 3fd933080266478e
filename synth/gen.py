"""Seeded synthetic workloads for the MoE gate -> route compaction -> grouped
SwiGLU FFN -> weighted combine path.

Every tensor is drawn from its own PCG64 stream, ``default_rng([seed, tensor,
expert...])``, so any subset of experts can be regenerated bit-identically and
the draw order never couples two tensors.  Normals are drawn in float32 and
scaled in float32; bf16 tensors are then rounded to nearest-even and stored as
their raw uint16 bit patterns (numpy has no bf16 type).  MXFP4 tensors are
uniform random e2m1 nibbles (two per byte) plus e8m0 scale bytes.

This module holds no step of the method: no softmax, no selection, no
compaction, no GEMM.  The oracle and the HIP path both consume the host arrays
returned here.
"""
from __future__ import annotations

import dataclasses
from concurrent.futures import ThreadPoolExecutor
from typing import Optional

import numpy as np

__all__ = [
    "MoECase", "round_to_bf16_bits", "decode_patterns", "DECODE_PATTERNS",
    "tiny_layer", "decode_case", "gate_case", "prefill_layer", "mxfp4_case",
    "contiguous_expert_map", "random_expert_map", "bf16_normal", "f32_normal",
    "gate_logits_bf16", "forced_routes", "decode_weights", "mxfp4_weights",
]

# stream ids, one per tensor role
_LOGITS, _X, _W1, _W2, _W1S, _W2S, _ROUTES, _TOPKW, _MAP, _TIES, _REMOTE = range(1, 12)

_THREADS = 8


def _rng(*key: int) -> np.random.Generator:
    return np.random.default_rng([int(k) for k in key])


def round_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest, ties to even.

    Only finite inputs are generated, so NaN handling is not needed here.
    """
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def f32_normal(shape, sigma: float, *key: int) -> np.ndarray:
    z = _rng(*key).standard_normal(size=shape, dtype=np.float32)
    return z * np.float32(sigma)


def bf16_normal(shape, sigma: float, *key: int) -> np.ndarray:
    return round_to_bf16_bits(f32_normal(shape, sigma, *key))


def _per_expert(fill, E: int, threads: int = _THREADS):
    with ThreadPoolExecutor(max_workers=max(1, min(threads, E))) as pool:
        list(pool.map(fill, range(E)))


def _bf16_expert_weights(E: int, rows: int, cols: int, sigma: float, seed: int, tid: int) -> np.ndarray:
    out = np.empty((E, rows, cols), dtype=np.uint16)

    def fill(e):
        out[e] = bf16_normal((rows, cols), sigma, seed, tid, e)

    _per_expert(fill, E)
    return out


def _f32_expert_weights(E: int, rows: int, cols: int, sigma: float, seed: int, tid: int) -> np.ndarray:
    out = np.empty((E, rows, cols), dtype=np.float32)

    def fill(e):
        out[e] = f32_normal((rows, cols), sigma, seed, tid, e)

    _per_expert(fill, E)
    return out


def _mxfp4_expert_weights(E: int, rows: int, cols: int, seed: int, tid: int, tid_s: int):
    """Uniform e2m1 codes (both nibbles of every byte uniform over 0..15, so +0
    and -0 both occur) and e8m0 scales uniform over exponents 119..127, i.e.
    block scales 2^-8 .. 2^0.  Layout: codes [E, rows, cols/2] with element 2i
    in the low nibble of byte i; scales [E, rows, cols/32]."""
    assert cols % 32 == 0
    codes = np.empty((E, rows, cols // 2), dtype=np.uint8)
    scales = np.empty((E, rows, cols // 32), dtype=np.uint8)

    def fill(e):
        codes[e] = _rng(seed, tid, e).integers(0, 256, size=(rows, cols // 2), dtype=np.uint8)
        scales[e] = _rng(seed, tid_s, e).integers(119, 128, size=(rows, cols // 32), dtype=np.uint8)

    _per_expert(fill, E)
    return codes, scales


@dataclasses.dataclass
class MoECase:
    """One synthetic workload.  Array conventions (all row-major, contiguous):

    logits   [T, E_global]   float32, or bf16 bits (uint16) when logits_dtype == "bf16"
    topk_ids [T, K] int32 and topk_weights [T, K] float32 when routes are forced
    expert_map [E_global] int32 global -> local id, -1 = remote; None = identity
    x        [T, H]          float32 or bf16 bits
    w1       [E_local, 2F, H] gate rows [0, F) then up rows [F, 2F)
    w2       [E_local, H, F]
    MXFP4: w1 = codes [E_local, 2F, H/2] uint8, w1_scale [E_local, 2F, H/32] uint8,
           w2 = codes [E_local, H, F/2],        w2_scale [E_local, H, F/32].
    """
    name: str
    T: int
    E_global: int
    E_local: int
    K: int
    H: int
    F: int
    renormalize: bool
    x_dtype: str
    w_dtype: str
    out_dtype: str
    x: np.ndarray
    w1: Optional[np.ndarray]
    w2: Optional[np.ndarray]
    w1_scale: Optional[np.ndarray] = None
    w2_scale: Optional[np.ndarray] = None
    logits: Optional[np.ndarray] = None
    logits_dtype: Optional[str] = None
    topk_ids: Optional[np.ndarray] = None
    topk_weights: Optional[np.ndarray] = None
    expert_map: Optional[np.ndarray] = None
    meta: dict = dataclasses.field(default_factory=dict)


# ---------------------------------------------------------------------------
# expert maps (one EP rank's view of the global expert set)


def contiguous_expert_map(E_global: int, E_local: int, rank: int = 1) -> np.ndarray:
    """Global experts [rank*E_local, (rank+1)*E_local) are local ids 0..E_local-1."""
    m = np.full(E_global, -1, dtype=np.int32)
    lo = rank * E_local
    assert lo + E_local <= E_global
    m[lo:lo + E_local] = np.arange(E_local, dtype=np.int32)
    return m


def random_expert_map(E_global: int, E_local: int, seed: int) -> np.ndarray:
    """A seeded random injective partial map: E_local distinct global ids, in
    random order, become local ids 0..E_local-1."""
    g = _rng(seed, _MAP).choice(E_global, size=E_local, replace=False)
    m = np.full(E_global, -1, dtype=np.int32)
    m[g] = np.arange(E_local, dtype=np.int32)
    return m


def _local_to_global(expert_map: np.ndarray) -> np.ndarray:
    E_local = int(expert_map.max()) + 1 if (expert_map >= 0).any() else 0
    inv = np.full(E_local, -1, dtype=np.int64)
    for g, l in enumerate(expert_map):
        if l >= 0:
            inv[l] = g
    return inv


# ---------------------------------------------------------------------------
# config 1: tiny full layer


def tiny_layer(seed: int = 0) -> MoECase:
    """T=16, E=8 (all local), K=2, H=64, F=128; everything float32.
    logits N(0,1), x N(0,1), W1/W2 N(0, 0.05); softmax then top-k, no renorm."""
    T, E, K, H, F = 16, 8, 2, 64, 128
    return MoECase(
        name="tiny_layer", T=T, E_global=E, E_local=E, K=K, H=H, F=F, renormalize=False,
        x_dtype="f32", w_dtype="f32", out_dtype="f32",
        logits=f32_normal((T, E), 1.0, seed, _LOGITS), logits_dtype="f32",
        x=f32_normal((T, H), 1.0, seed, _X),
        w1=_f32_expert_weights(E, 2 * F, H, 0.05, seed, _W1),
        w2=_f32_expert_weights(E, H, F, 0.05, seed, _W2),
    )


# ---------------------------------------------------------------------------
# config 2: decode (M=2, top-6, 40 of 256 experts local), forced route patterns

# Local expert ids per token row; None marks a remote route (a global id that
# the expert map sends to -1).  One entry per route pattern of the decode
# scheduler note: same, disjoint, cross-row overlap, within-row duplicate, all
# duplicate, twelve distinct local, all remote.
DECODE_PATTERNS = {
    "same": [[3, None, 17, None, 29, None], [3, None, 17, None, 29, None]],
    "disjoint": [[1, None, 12, None, 22, None], [5, None, 18, None, 35, None]],
    "cross_row": [[2, 10, 20, None, None, None], [10, 20, 30, None, None, None]],
    "within_row_dup": [[4, 4, 8, None, None, None], [6, 15, 25, None, None, None]],
    "all_dup": [[7] * 6, [7] * 6],
    "twelve_local": [[0, 3, 6, 9, 12, 15], [18, 21, 24, 27, 30, 33]],
    "all_remote": [[None] * 6, [None] * 6],
}


def decode_patterns():
    return list(DECODE_PATTERNS)


_decode_weight_cache: dict = {}


def decode_weights(seed: int = 0, E_local: int = 40, H: int = 4096, F: int = 2048):
    """bf16 W1 [E_local, 2F, H] and W2 [E_local, H, F], N(0, 0.02).  Cached:
    the 40-expert set is 2.0 GB of bf16."""
    key = (seed, E_local, H, F)
    if key not in _decode_weight_cache:
        _decode_weight_cache.clear()
        _decode_weight_cache[key] = (
            _bf16_expert_weights(E_local, 2 * F, H, 0.02, seed, _W1),
            _bf16_expert_weights(E_local, H, F, 0.02, seed, _W2),
        )
    return _decode_weight_cache[key]


def forced_routes(pattern_rows, expert_map: np.ndarray, seed: int) -> np.ndarray:
    """Turn a pattern of local ids (None = remote) into global topk_ids.
    Remote routes draw a global id uniformly from the ids the map sends to -1."""
    inv = _local_to_global(expert_map)
    remote_pool = np.flatnonzero(expert_map < 0)
    rr = _rng(seed, _REMOTE)
    ids = np.empty((len(pattern_rows), len(pattern_rows[0])), dtype=np.int32)
    for t, row in enumerate(pattern_rows):
        for k, l in enumerate(row):
            ids[t, k] = int(rr.choice(remote_pool)) if l is None else int(inv[l])
    return ids


def decode_case(pattern: str, map_kind: str = "contiguous", seed: int = 0, weight_seed: int = 0,
                with_weights: bool = True) -> MoECase:
    """M=T=2 tokens, E_global=256, 40 local experts, top-6, H=4096, F=2048,
    bf16 weights N(0,0.02) and x N(0,1).  topk_ids are forced by the pattern;
    topk_weights are Dirichlet(1) over the 6 routes of each token."""
    T, K, Eg, El, H, F = 2, 6, 256, 40, 4096, 2048
    emap = contiguous_expert_map(Eg, El) if map_kind == "contiguous" else random_expert_map(Eg, El, seed)
    ids = forced_routes(DECODE_PATTERNS[pattern], emap, seed)
    w = _rng(seed, _TOPKW).dirichlet(np.ones(K), size=T).astype(np.float32)
    w1 = w2 = None
    if with_weights:
        w1, w2 = decode_weights(weight_seed, El, H, F)
    return MoECase(
        name=f"decode_{pattern}_{map_kind}_s{seed}", T=T, E_global=Eg, E_local=El, K=K, H=H, F=F,
        renormalize=False, x_dtype="bf16", w_dtype="bf16", out_dtype="bf16",
        x=bf16_normal((T, H), 1.0, seed, _X), w1=w1, w2=w2,
        topk_ids=ids, topk_weights=w, expert_map=emap,
        meta={"pattern": pattern, "map_kind": map_kind, "seed": seed},
    )


# ---------------------------------------------------------------------------
# config 3: gate throughput


def gate_logits_bf16(T: int, E: int, seed: int, tie_fraction: float = 0.01, K: int = 8) -> np.ndarray:
    """bf16 logits 2*N(0,1) [T, E] with exact ties injected into ~1% of rows.

    Half of the chosen rows get a boundary tie: the value ranked K-th in the
    row (order: value descending, index ascending) is copied onto a random
    expert ranked below K, so the K-th place is decided by the lower-index
    rule.  The other half copy the row's largest value onto another random
    expert.  (With E <= K every chosen row gets the second kind.)  Ties
    between distinct bf16 draws also occur naturally (bf16 has an 8-bit
    significand)."""
    bits = bf16_normal((T, E), 2.0, seed, _LOGITS)
    n_ties = int(round(T * tie_fraction))
    if n_ties and E > 1:
        r = _rng(seed, _TIES)
        rows = r.choice(T, size=n_ties, replace=False)
        for i, t in enumerate(rows):
            # bf16 bit patterns are sign-magnitude; decode to float32 to rank
            f = (bits[t].astype(np.uint32) << np.uint32(16)).view(np.float32)
            if i % 2 == 0 and E > K:
                order = np.lexsort((np.arange(E), -f.astype(np.float64)))
                src = int(order[K - 1])
                dst = int(order[K + int(r.integers(E - K))])
            else:
                src = int(np.argmax(f))
                dst = int(r.integers(E - 1))
                dst = dst + 1 if dst >= src else dst
            bits[t, dst] = bits[t, src]
    return bits


def gate_case(E: int, T: int = 65536, K: int = 8, seed: int = 0, renormalize: bool = False) -> MoECase:
    """Gate-only workload: T rows of E bf16 logits, top-K; no FFN tensors."""
    return MoECase(
        name=f"gate_T{T}_E{E}_K{K}", T=T, E_global=E, E_local=E, K=K, H=0, F=0,
        renormalize=renormalize, x_dtype="bf16", w_dtype="bf16", out_dtype="bf16",
        x=np.zeros((T, 0), np.uint16), w1=None, w2=None,
        logits=gate_logits_bf16(T, E, seed, K=K), logits_dtype="bf16",
    )


# ---------------------------------------------------------------------------
# config 4: prefill layer


def prefill_layer(seed: int = 0, T: int = 4096, E: int = 128, K: int = 8, H: int = 2048, F: int = 768,
                  with_weights: bool = True) -> MoECase:
    """T=4096 tokens, E=128 all local, top-8 renormalised, H=2048, F=768.
    logits bf16 2*N(0,1), x bf16 N(0,1), W1/W2 bf16 N(0,0.02); bf16 output."""
    return MoECase(
        name=f"prefill_T{T}_E{E}_K{K}_H{H}_F{F}", T=T, E_global=E, E_local=E, K=K, H=H, F=F,
        renormalize=True, x_dtype="bf16", w_dtype="bf16", out_dtype="bf16",
        logits=bf16_normal((T, E), 2.0, seed, _LOGITS), logits_dtype="bf16",
        x=bf16_normal((T, H), 1.0, seed, _X),
        w1=_bf16_expert_weights(E, 2 * F, H, 0.02, seed, _W1) if with_weights else None,
        w2=_bf16_expert_weights(E, H, F, 0.02, seed, _W2) if with_weights else None,
    )


# ---------------------------------------------------------------------------
# config 5: MXFP4 expert weights, decode-sized T

_mxfp4_weight_cache: dict = {}


def mxfp4_weights(seed: int = 0, E_local: int = 32, H: int = 4096, F: int = 2048):
    key = (seed, E_local, H, F)
    if key not in _mxfp4_weight_cache:
        _mxfp4_weight_cache.clear()
        w1, w1s = _mxfp4_expert_weights(E_local, 2 * F, H, seed, _W1, _W1S)
        w2, w2s = _mxfp4_expert_weights(E_local, H, F, seed, _W2, _W2S)
        _mxfp4_weight_cache[key] = (w1, w1s, w2, w2s)
    return _mxfp4_weight_cache[key]


def mxfp4_case(T: int, routes: str = "uniform", seed: int = 0, weight_seed: int = 0,
               E_global: int = 256, E_local: int = 32, K: int = 8, H: int = 4096, F: int = 2048,
               with_weights: bool = True) -> MoECase:
    """MXFP4 experts: E_global=256, 32 local (global [32,64)), top-8, H=4096,
    F=2048, bf16 x N(0,1).  routes="uniform": each token picks 8 distinct
    global experts uniformly (the law of top-8 over iid logits); "all_local":
    8 distinct experts among the 32 local ones.  topk_weights are Dirichlet(1),
    which sum to 1 like renormalised gate weights."""
    emap = contiguous_expert_map(E_global, E_local)
    rr = _rng(seed, _ROUTES)
    ids = np.empty((T, K), dtype=np.int32)
    local_globals = np.flatnonzero(emap >= 0)
    for t in range(T):
        pool = E_global if routes == "uniform" else local_globals
        ids[t] = rr.choice(pool, size=K, replace=False)
    w = _rng(seed, _TOPKW).dirichlet(np.ones(K), size=T).astype(np.float32)
    w1 = w1s = w2 = w2s = None
    if with_weights:
        w1, w1s, w2, w2s = mxfp4_weights(weight_seed, E_local, H, F)
    return MoECase(
        name=f"mxfp4_T{T}_{routes}_s{seed}", T=T, E_global=E_global, E_local=E_local, K=K, H=H, F=F,
        renormalize=True, x_dtype="bf16", w_dtype="mxfp4", out_dtype="bf16",
        x=bf16_normal((T, H), 1.0, seed, _X), w1=w1, w2=w2, w1_scale=w1s, w2_scale=w2s,
        topk_ids=ids, topk_weights=w, expert_map=emap, meta={"routes": routes, "seed": seed},
    )
