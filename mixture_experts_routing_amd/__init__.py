"""MI355X-native MoE routing + expert-FFN hot path.

Thin Python binding over the C ABI of libmoe_routing.so (include/moe_routing.h).
The functions below only marshal torch tensors (device memory) and the
current HIP stream into the C calls; every step of the path runs in the HIP
kernels of the library.  Importing this package fails if the library has not
been built: there is no fallback implementation.
"""
from __future__ import annotations

from typing import Optional, Tuple

import torch

from . import _lib
from ._lib import MOE_BF16, MOE_BF16_TILED, MOE_F32, MOE_MXFP4, MOE_MXFP4_MMA_BF16, MOE_MXFP4_MMA_F8F6F4

_LIB = _lib.load()

__all__ = [
    "moe_topk_softmax", "moe_topk_sigmoid", "moe_route_compact", "moe_route_align", "moe_grouped_ffn",
    "moe_grouped_ffn_noalloc", "moe_grouped_ffn_control", "moe_fused_experts", "moe_topk_compact", "moe_combine", "moe_pack_ffn_weights", "moe_layer",
    "moe_probe_read", "moe_probe_copy", "moe_probe_mfma", "moe_probe_mfma_clock", "moe_probe_gate_loads", "moe_set_mxfp4_mma",
    "moe_get_mxfp4_mma", "mxfp4_mma",
    "MOE_F32", "MOE_BF16", "MOE_MXFP4", "MOE_BF16_TILED", "MOE_MXFP4_MMA_BF16", "MOE_MXFP4_MMA_F8F6F4", "MoeError",
    "library_path",
]


class MoeError(RuntimeError):
    pass


def library_path() -> str:
    return _lib.LIB_PATH


def _check(code: int, what: str):
    if code != 0:
        msg = _lib.status_string(code)
        if code == _lib.MOE_ERR_HIP:
            msg += f" (hipError {_LIB.moe_last_hip_error()})"
        raise MoeError(f"{what}: {msg}")


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return MOE_F32
    if t.dtype == torch.bfloat16:
        return MOE_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _dev(*ts):
    dev = None
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("tensors must live in GPU memory")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
        dev = t.device if dev is None else dev
        if t.device != dev:
            raise ValueError("tensors on different devices")
    return dev


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


_I32, _F32, _BF16, _U8 = torch.int32, torch.float32, torch.bfloat16, torch.uint8


def _req(t: Optional[torch.Tensor], name: str, dtypes=None, min_numel: Optional[int] = None, shape=None,
         ndim: Optional[int] = None):
    """Checks what the C call will read or write through t -- dtype, rank,
    shape, size -- and raises MoeError before anything reaches the library
    (the C side sees only pointers: a wrong dtype or a short buffer would be
    read or written out of bounds on the device)."""
    if t is None:
        return
    if dtypes is not None:
        dts = dtypes if isinstance(dtypes, tuple) else (dtypes,)
        if t.dtype not in dts:
            raise MoeError(f"{name}: dtype {t.dtype}, expected {' or '.join(str(d) for d in dts)}")
    if ndim is not None and t.dim() != ndim:
        raise MoeError(f"{name}: {t.dim()}-d tensor, expected {ndim}-d")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise MoeError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if min_numel is not None and t.numel() < min_numel:
        raise MoeError(f"{name}: {t.numel()} elements, the call needs {min_numel}")


def _nbytes(t: Optional[torch.Tensor]) -> int:
    return 0 if t is None else t.numel() * t.element_size()


def _ffn_weights(x: torch.Tensor, w1: torch.Tensor, w2: torch.Tensor, w1_scale, w2_scale):
    """(T, H, E_local, F, w_dtype) of a grouped-FFN call, after checking that
    x [T, H], w1 [E, 2F, H] and w2 [E, H, F] agree (MXFP4: uint8 codes
    [E, 2F, H/2], [E, H, F/2] with scales [E, 2F, H/32], [E, H, F/32])."""
    _req(x, "x", (_F32, _BF16), ndim=2)
    _req(w1, "w1", ndim=3)
    _req(w2, "w2", ndim=3)
    T, H = x.shape
    E_local = w1.shape[0]
    if w1.dtype == _U8:
        _req(w2, "w2", _U8)
        F = w2.shape[2] * 2
        _req(w1, "w1", shape=(E_local, 2 * F, H // 2))
        _req(w2, "w2", shape=(E_local, H, F // 2))
        if w1_scale is None or w2_scale is None:
            raise MoeError("MXFP4 weights need w1_scale and w2_scale")
        _req(w1_scale, "w1_scale", _U8, shape=(E_local, 2 * F, H // 32))
        _req(w2_scale, "w2_scale", _U8, shape=(E_local, H, F // 32))
        return T, H, E_local, F, MOE_MXFP4
    _req(w1, "w1", (_F32, _BF16))
    _req(w2, "w2", w1.dtype)
    F = w2.shape[2]
    _req(w1, "w1", shape=(E_local, 2 * F, H))
    _req(w2, "w2", shape=(E_local, H, F))
    return T, H, E_local, F, _dt(w1)


def _route_arrays(T: int, K: int, E_local: int, counts, offsets, s2r=None, r2s=None):
    _req(counts, "counts", _I32, E_local)
    _req(offsets, "offsets", _I32, E_local + 1)
    _req(s2r, "slot_to_row", _I32, T * K)
    _req(r2s, "row_to_slot", _I32, T * K)


def _stream(stream, device) -> int:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream


def _gate(fn_name, logits, K, renormalize, topk_weights, topk_ids, token_expert_indices, with_indices, stream):
    _req(logits, "logits", (_F32, _BF16), ndim=2)
    T, E = logits.shape
    _req(topk_weights, "topk_weights", _F32, T * K)
    _req(topk_ids, "topk_ids", _I32, T * K)
    _req(token_expert_indices, "token_expert_indices", _I32, T * K)
    dev = _dev(logits)
    if topk_weights is None:
        topk_weights = torch.empty((T, K), dtype=torch.float32, device=dev)
    if topk_ids is None:
        topk_ids = torch.empty((T, K), dtype=torch.int32, device=dev)
    if token_expert_indices is None and with_indices:
        token_expert_indices = torch.empty((T, K), dtype=torch.int32, device=dev)
    _dev(topk_weights, topk_ids, token_expert_indices)
    _check(getattr(_LIB, fn_name)(_ptr(logits), _dt(logits), T, E, K, int(bool(renormalize)), _ptr(topk_weights),
                                  _ptr(topk_ids), _ptr(token_expert_indices), _stream(stream, dev)), fn_name)
    return topk_weights, topk_ids, token_expert_indices


def moe_topk_softmax(logits: torch.Tensor, K: int, renormalize: bool = False,
                     topk_weights: Optional[torch.Tensor] = None, topk_ids: Optional[torch.Tensor] = None,
                     token_expert_indices: Optional[torch.Tensor] = None, with_indices: bool = True,
                     stream=None) -> Tuple[torch.Tensor, torch.Tensor, Optional[torch.Tensor]]:
    """logits [T, E] (f32 or bf16) -> (weights f32 [T,K], ids i32 [T,K], token_expert_indices i32 [T,K])."""
    return _gate("moe_topk_softmax", logits, K, renormalize, topk_weights, topk_ids, token_expert_indices,
                 with_indices, stream)


def moe_topk_sigmoid(logits: torch.Tensor, K: int, renormalize: bool = False,
                     topk_weights: Optional[torch.Tensor] = None, topk_ids: Optional[torch.Tensor] = None,
                     token_expert_indices: Optional[torch.Tensor] = None, with_indices: bool = True,
                     stream=None) -> Tuple[torch.Tensor, torch.Tensor, Optional[torch.Tensor]]:
    """Sigmoid-scoring gate: same arguments and outputs as moe_topk_softmax,
    weight = sigmoid(logit) of each chosen expert (optionally renormalised)."""
    return _gate("moe_topk_sigmoid", logits, K, renormalize, topk_weights, topk_ids, token_expert_indices,
                 with_indices, stream)


def route_compact_workspace_bytes(T: int, K: int, E_local: int) -> int:
    return int(_LIB.moe_route_compact_workspace_bytes(T, K, E_local))


def moe_route_compact(topk_ids: torch.Tensor, expert_map: Optional[torch.Tensor], E_local: int,
                      E_global: Optional[int] = None, out=None, workspace: Optional[torch.Tensor] = None,
                      stream=None):
    """topk_ids [T, K] int32 (global ids), expert_map [E_global] int32 or None
    -> (counts [E_local], offsets [E_local+1], slot_to_row [T*K], row_to_slot [T*K]), all int32."""
    _req(topk_ids, "topk_ids", _I32, ndim=2)
    T, K = topk_ids.shape
    if E_global is None:
        E_global = expert_map.numel() if expert_map is not None else E_local
    _req(expert_map, "expert_map", _I32, E_global)
    if out is not None:
        _route_arrays(T, K, E_local, *out)
    dev = _dev(topk_ids, expert_map)
    if out is None:
        counts = torch.empty(E_local, dtype=torch.int32, device=dev)
        offsets = torch.empty(E_local + 1, dtype=torch.int32, device=dev)
        s2r = torch.empty(T * K, dtype=torch.int32, device=dev)
        r2s = torch.empty(T * K, dtype=torch.int32, device=dev)
    else:
        counts, offsets, s2r, r2s = out
    need = route_compact_workspace_bytes(T, K, E_local)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = _nbytes(workspace)
    _check(_LIB.moe_route_compact(_ptr(topk_ids), T, K, _ptr(expert_map), E_global, E_local, _ptr(counts),
                                  _ptr(offsets), _ptr(s2r), _ptr(r2s), _ptr(workspace), ws_bytes,
                                  _stream(stream, dev)), "moe_route_compact")
    return counts, offsets, s2r, r2s


def moe_topk_compact(logits: torch.Tensor, K: int, renormalize: bool = False, scoring: str = "softmax",
                     expert_map: Optional[torch.Tensor] = None, E_local: Optional[int] = None, gate_out=None,
                     route_out=None, with_indices: bool = True, workspace: Optional[torch.Tensor] = None,
                     stream=None):
    """Gate and route compaction in one call (the compaction's count pass runs
    inside the gate kernel where the shape allows).  logits [T, E]; scoring
    "softmax" or "sigmoid".  Returns ((topk_weights, topk_ids,
    token_expert_indices or None), (counts, offsets, slot_to_row, row_to_slot))."""
    _req(logits, "logits", (_F32, _BF16), ndim=2)
    T, E = logits.shape
    if E_local is None:
        E_local = E
    _req(expert_map, "expert_map", _I32, E)
    if gate_out is not None:
        _req(gate_out[0], "topk_weights", _F32, T * K)
        _req(gate_out[1], "topk_ids", _I32, T * K)
        _req(gate_out[2], "token_expert_indices", _I32, T * K)
    if route_out is not None:
        _route_arrays(T, K, E_local, *route_out)
    dev = _dev(logits, expert_map)
    if scoring not in ("softmax", "sigmoid"):
        raise MoeError(f"unknown scoring {scoring!r}")
    if gate_out is None:
        gate_out = (torch.empty((T, K), dtype=torch.float32, device=dev),
                    torch.empty((T, K), dtype=torch.int32, device=dev),
                    torch.empty((T, K), dtype=torch.int32, device=dev) if with_indices else None)
    tw, tid, tei = gate_out
    if route_out is None:
        route_out = (torch.empty(E_local, dtype=torch.int32, device=dev),
                     torch.empty(E_local + 1, dtype=torch.int32, device=dev),
                     torch.empty(T * K, dtype=torch.int32, device=dev),
                     torch.empty(T * K, dtype=torch.int32, device=dev))
    counts, offsets, s2r, r2s = route_out
    need = route_compact_workspace_bytes(T, K, E_local)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = _nbytes(workspace)
    _check(_LIB.moe_topk_compact(_ptr(logits), _dt(logits), T, E, K, int(renormalize),
                                 0 if scoring == "softmax" else 1, _ptr(tw), _ptr(tid), _ptr(tei), _ptr(expert_map),
                                 E_local, _ptr(counts), _ptr(offsets), _ptr(s2r), _ptr(r2s), _ptr(workspace),
                                 ws_bytes, _stream(stream, dev)), "moe_topk_compact")
    return gate_out, route_out


def route_align_workspace_bytes(T: int, K: int, E_local: int) -> int:
    return int(_LIB.moe_route_align_workspace_bytes(T, K, E_local))


def moe_route_align(topk_ids: torch.Tensor, expert_map: Optional[torch.Tensor], E_local: int, block_size: int,
                    E_global: Optional[int] = None, out=None, workspace: Optional[torch.Tensor] = None, stream=None):
    """Block-aligned layout: -> (padded_offsets [E_local+1], sorted_slots [cap_rows],
    block_expert [cap_blocks], slot_to_row [T*K]), all int32 (see moe_route_align)."""
    _req(topk_ids, "topk_ids", _I32, ndim=2)
    T, K = topk_ids.shape
    N = T * K
    if E_global is None:
        E_global = expert_map.numel() if expert_map is not None else E_local
    _req(expert_map, "expert_map", _I32, E_global)
    cap_rows = N + E_local * (block_size - 1)
    cap_blocks = -(-N // block_size) + E_local
    if out is not None:
        _req(out[0], "padded_offsets", _I32, E_local + 1)
        _req(out[1], "sorted_slots", _I32, cap_rows)
        _req(out[2], "block_expert", _I32, cap_blocks)
        _req(out[3], "slot_to_row", _I32, N)
    dev = _dev(topk_ids, expert_map)
    if out is None:
        out = (torch.empty(E_local + 1, dtype=torch.int32, device=dev),
               torch.empty(cap_rows, dtype=torch.int32, device=dev),
               torch.empty(cap_blocks, dtype=torch.int32, device=dev),
               torch.empty(N, dtype=torch.int32, device=dev))
    poff, sorted_slots, block_expert, s2r = out
    need = route_align_workspace_bytes(T, K, E_local)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    _check(_LIB.moe_route_align(_ptr(topk_ids), T, K, _ptr(expert_map), E_global, E_local, block_size, _ptr(poff),
                                _ptr(sorted_slots), _ptr(block_expert), _ptr(s2r), _ptr(workspace),
                                _nbytes(workspace), _stream(stream, dev)), "moe_route_align")
    return poff, sorted_slots, block_expert, s2r


def grouped_ffn_workspace_bytes(T: int, K: int, H: int, F: int, E_local: int, w_dtype: int) -> int:
    return int(_LIB.moe_grouped_ffn_workspace_bytes(T, K, H, F, E_local, w_dtype))


def moe_set_mxfp4_mma(mode: int) -> None:
    """MOE_MXFP4_MMA_BF16 or MOE_MXFP4_MMA_F8F6F4: the arithmetic of MXFP4
    expert GEMMs in the decode kernels, for calls launched from now on."""
    _check(_LIB.moe_set_mxfp4_mma(int(mode)), "moe_set_mxfp4_mma")


def moe_get_mxfp4_mma() -> int:
    return int(_LIB.moe_get_mxfp4_mma())


class mxfp4_mma:
    """Context manager: `with mxfp4_mma(MOE_MXFP4_MMA_F8F6F4): ...` sets the
    MXFP4 decode arithmetic and restores the previous one on exit."""

    def __init__(self, mode: int):
        self.mode = int(mode)

    def __enter__(self):
        self.prev = moe_get_mxfp4_mma()
        moe_set_mxfp4_mma(self.mode)
        return self

    def __exit__(self, *exc):
        moe_set_mxfp4_mma(self.prev)
        return False


def moe_pack_ffn_weights(w1: torch.Tensor, w2: torch.Tensor, w1_tiled: Optional[torch.Tensor] = None,
                         w2_tiled: Optional[torch.Tensor] = None, stream=None):
    """bf16 w1 [E_local, 2F, H], w2 [E_local, H, F] -> the same weights in the
    tile-packed layout (tensors of the same shapes and dtype, whose memory
    order is the packed one); pass them to moe_grouped_ffn with tiled=True."""
    _req(w2, "w2", _BF16, ndim=3)
    E_local, H, F = w2.shape
    _req(w1, "w1", _BF16, shape=(E_local, 2 * F, H))
    _req(w1_tiled, "w1_tiled", _BF16, shape=(E_local, 2 * F, H))
    _req(w2_tiled, "w2_tiled", _BF16, shape=(E_local, H, F))
    dev = _dev(w1, w2, w1_tiled, w2_tiled)
    if w1_tiled is None:
        w1_tiled = torch.empty_like(w1)
    if w2_tiled is None:
        w2_tiled = torch.empty_like(w2)
    _check(_LIB.moe_pack_ffn_weights(_ptr(w1), _ptr(w2), E_local, H, F, _ptr(w1_tiled), _ptr(w2_tiled),
                                     _stream(stream, dev)), "moe_pack_ffn_weights")
    return w1_tiled, w2_tiled


def moe_grouped_ffn(x: torch.Tensor, K: int, w1: torch.Tensor, w2: torch.Tensor, counts: torch.Tensor,
                    offsets: torch.Tensor, row_to_slot: torch.Tensor, w1_scale: Optional[torch.Tensor] = None,
                    w2_scale: Optional[torch.Tensor] = None, y_dtype: Optional[torch.dtype] = None,
                    y: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None, stream=None,
                    tiled: bool = False):
    """x [T, H]; w1 [E_local, 2F, H] and w2 [E_local, H, F] (f32 / bf16), or
    uint8 MXFP4 codes [E_local, 2F, H/2], [E_local, H, F/2] with e8m0 scales,
    or (tiled=True) bf16 weights from moe_pack_ffn_weights.
    Returns y [T*K, H] in the expert-grouped row order (rows >= R unwritten)."""
    T, H, E_local, F, w_dt = _ffn_weights(x, w1, w2, w1_scale, w2_scale)
    _route_arrays(T, K, E_local, counts, offsets, None, row_to_slot)
    _req(y, "y", (_F32, _BF16), T * K * H)
    dev = _dev(x, w1, w2, counts, offsets, row_to_slot, w1_scale, w2_scale, y)
    if tiled:
        if w_dt != MOE_BF16:
            raise MoeError("tiled weights must be bfloat16")
        w_dt = MOE_BF16_TILED
    if y is None:
        y = torch.empty((T * K, H), dtype=y_dtype or x.dtype, device=dev)
    need = grouped_ffn_workspace_bytes(T, K, H, F, E_local, w_dt)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    _check(_LIB.moe_grouped_ffn(_ptr(x), _dt(x), T, K, H, F, E_local, _ptr(w1), _ptr(w1_scale), _ptr(w2),
                                _ptr(w2_scale), w_dt, _ptr(counts), _ptr(offsets), _ptr(row_to_slot), _ptr(y),
                                _dt(y), _ptr(workspace), _nbytes(workspace), _stream(stream, dev)),
           "moe_grouped_ffn")
    return y


def moe_grouped_ffn_noalloc(x: torch.Tensor, K: int, w1: torch.Tensor, w2: torch.Tensor, counts: torch.Tensor,
                            offsets: torch.Tensor, row_to_slot: torch.Tensor, w1_scale: Optional[torch.Tensor] = None,
                            w2_scale: Optional[torch.Tensor] = None, y_dtype: Optional[torch.dtype] = None,
                            y: Optional[torch.Tensor] = None, stream=None, tiled: bool = False):
    """moe_grouped_ffn with the act rows in the library's fixed per-GPU scratch
    (64 MiB) instead of a workspace: the library allocates nothing.  Same
    arguments (no workspace) and result; raises MoeError
    (MOE_ERR_SCRATCH_LIMIT) when the act rows exceed the scratch.  y must be
    given by callers that cannot allocate."""
    T, H, E_local, F, w_dt = _ffn_weights(x, w1, w2, w1_scale, w2_scale)
    _route_arrays(T, K, E_local, counts, offsets, None, row_to_slot)
    _req(y, "y", (_F32, _BF16), T * K * H)
    dev = _dev(x, w1, w2, counts, offsets, row_to_slot, w1_scale, w2_scale, y)
    if tiled:
        if w_dt != MOE_BF16:
            raise MoeError("tiled weights must be bfloat16")
        w_dt = MOE_BF16_TILED
    if y is None:
        y = torch.empty((T * K, H), dtype=y_dtype or x.dtype, device=dev)
    _check(_LIB.moe_grouped_ffn_noalloc(_ptr(x), _dt(x), T, K, H, F, E_local, _ptr(w1), _ptr(w1_scale), _ptr(w2),
                                        _ptr(w2_scale), w_dt, _ptr(counts), _ptr(offsets), _ptr(row_to_slot),
                                        _ptr(y), _dt(y), _stream(stream, dev)), "moe_grouped_ffn_noalloc")
    return y


def grouped_ffn_control_workspace_bytes(T: int, K: int, H: int, F: int, E_local: int, w_dtype: int) -> int:
    return int(_LIB.moe_grouped_ffn_control_workspace_bytes(T, K, H, F, E_local, w_dtype))


def moe_grouped_ffn_control(x: torch.Tensor, K: int, w1: torch.Tensor, w2: torch.Tensor, counts: torch.Tensor,
                            offsets: torch.Tensor, row_to_slot: torch.Tensor, w1_scale=None, w2_scale=None,
                            y_dtype: Optional[torch.dtype] = None, y: Optional[torch.Tensor] = None,
                            workspace: Optional[torch.Tensor] = None, stream=None):
    """moe_grouped_ffn run by the generic atomic-counter scheduler (the A/B
    control); same arguments and result layout."""
    T, H, E_local, F, w_dt = _ffn_weights(x, w1, w2, w1_scale, w2_scale)
    _route_arrays(T, K, E_local, counts, offsets, None, row_to_slot)
    _req(y, "y", (_F32, _BF16), T * K * H)
    dev = _dev(x, w1, w2, counts, offsets, row_to_slot, w1_scale, w2_scale, y)
    if y is None:
        y = torch.empty((T * K, H), dtype=y_dtype or x.dtype, device=dev)
    need = grouped_ffn_control_workspace_bytes(T, K, H, F, E_local, w_dt)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    _check(_LIB.moe_grouped_ffn_control(_ptr(x), _dt(x), T, K, H, F, E_local, _ptr(w1), _ptr(w1_scale), _ptr(w2),
                                        _ptr(w2_scale), w_dt, _ptr(counts), _ptr(offsets), _ptr(row_to_slot),
                                        _ptr(y), _dt(y), _ptr(workspace), _nbytes(workspace), _stream(stream, dev)),
           "moe_grouped_ffn_control")
    return y


def moe_combine(y: torch.Tensor, topk_weights: torch.Tensor, slot_to_row: torch.Tensor,
                out_dtype: Optional[torch.dtype] = None, out: Optional[torch.Tensor] = None, stream=None):
    """y [R', H] grouped rows, topk_weights [T, K] f32, slot_to_row [T*K] -> out [T, H]."""
    _req(y, "y", (_F32, _BF16), ndim=2)
    _req(topk_weights, "topk_weights", _F32, ndim=2)
    T, K = topk_weights.shape
    H = y.shape[1]
    _req(slot_to_row, "slot_to_row", _I32, T * K)
    _req(out, "out", (_F32, _BF16), T * H)
    dev = _dev(y, topk_weights, slot_to_row, out)
    if out is None:
        out = torch.empty((T, H), dtype=out_dtype or y.dtype, device=dev)
    _check(_LIB.moe_combine(_ptr(y), _dt(y), _ptr(topk_weights), _ptr(slot_to_row), T, K, H, _ptr(out), _dt(out),
                            _stream(stream, dev)), "moe_combine")
    return out


def fused_experts_workspace_bytes(T: int, K: int, H: int, F: int, E_local: int, w_dtype: int) -> int:
    return int(_LIB.moe_fused_experts_workspace_bytes(T, K, H, F, E_local, w_dtype))


def moe_fused_experts(x: torch.Tensor, topk_ids: torch.Tensor, topk_weights: torch.Tensor, w1: torch.Tensor,
                      w2: torch.Tensor, expert_map: Optional[torch.Tensor] = None, E_global: Optional[int] = None,
                      w1_scale: Optional[torch.Tensor] = None, w2_scale: Optional[torch.Tensor] = None,
                      out_dtype: Optional[torch.dtype] = None, out: Optional[torch.Tensor] = None, routes=None,
                      workspace: Optional[torch.Tensor] = None, stream=None):
    """Decode batches (T*K <= 64, E_local <= 64): compaction, grouped FFN and
    combine in two launches.  x [T, H] bf16, topk_ids / topk_weights [T, K],
    weights as for moe_grouped_ffn (bf16 or MXFP4).
    Returns (out [T, H], (counts, offsets, slot_to_row, row_to_slot))."""
    T, H, E_local, F, w_dt = _ffn_weights(x, w1, w2, w1_scale, w2_scale)
    _req(topk_ids, "topk_ids", _I32, ndim=2)
    K = topk_ids.shape[1]
    _req(topk_ids, "topk_ids", shape=(T, K))
    _req(topk_weights, "topk_weights", _F32, shape=(T, K))
    if E_global is None:
        E_global = expert_map.numel() if expert_map is not None else E_local
    _req(expert_map, "expert_map", _I32, E_global)
    if routes is not None:
        _route_arrays(T, K, E_local, *routes)
    _req(out, "out", (_F32, _BF16), T * H)
    dev = _dev(x, topk_ids, topk_weights, w1, w2, expert_map, w1_scale, w2_scale, out)
    if out is None:
        out = torch.empty((T, H), dtype=out_dtype or x.dtype, device=dev)
    if routes is None:
        routes = (torch.empty(E_local, dtype=torch.int32, device=dev),
                  torch.empty(E_local + 1, dtype=torch.int32, device=dev),
                  torch.empty(T * K, dtype=torch.int32, device=dev),
                  torch.empty(T * K, dtype=torch.int32, device=dev))
    counts, offsets, s2r, r2s = routes
    need = fused_experts_workspace_bytes(T, K, H, F, E_local, w_dt)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    _check(_LIB.moe_fused_experts(_ptr(x), _dt(x), T, K, H, F, _ptr(topk_ids), _ptr(topk_weights),
                                  _ptr(expert_map), E_global, E_local, _ptr(w1), _ptr(w1_scale), _ptr(w2),
                                  _ptr(w2_scale), w_dt, _ptr(counts), _ptr(offsets), _ptr(s2r), _ptr(r2s),
                                  _ptr(out), _dt(out), _ptr(workspace), _nbytes(workspace), _stream(stream, dev)),
           "moe_fused_experts")
    return out, routes


def moe_layer(x: torch.Tensor, w1: torch.Tensor, w2: torch.Tensor, K: int, logits: Optional[torch.Tensor] = None,
              renormalize: bool = False, topk_ids: Optional[torch.Tensor] = None,
              topk_weights: Optional[torch.Tensor] = None, expert_map: Optional[torch.Tensor] = None,
              E_global: Optional[int] = None, w1_scale=None, w2_scale=None, out_dtype=None, y_dtype=None,
              stream=None, tiled: bool = False) -> dict:
    """The whole path: gate (if logits are given) -> compaction -> grouped FFN -> combine."""
    tei = None
    if logits is not None:
        topk_weights, topk_ids, tei = moe_topk_softmax(logits, K, renormalize, stream=stream)
    E_local = w1.shape[0]
    counts, offsets, s2r, r2s = moe_route_compact(topk_ids, expert_map, E_local, E_global=E_global, stream=stream)
    y = moe_grouped_ffn(x, K, w1, w2, counts, offsets, r2s, w1_scale, w2_scale, y_dtype=y_dtype or x.dtype,
                        stream=stream, tiled=tiled)
    out = moe_combine(y, topk_weights, s2r, out_dtype=out_dtype or x.dtype, stream=stream)
    return dict(topk_weights=topk_weights, topk_ids=topk_ids, token_expert_indices=tei, counts=counts,
                offsets=offsets, slot_to_row=s2r, row_to_slot=r2s, y=y, out=out)


# ---------------------------------------------------------------------------
# measurement probes (not steps of the layer): see include/moe_routing.h


def moe_probe_read(src: torch.Tensor, out: torch.Tensor, stream=None) -> None:
    """Read every byte of src once (streaming read); out: uint32 [4096*256]."""
    _req(out, "out", torch.int32, 4096 * 256)
    dev = _dev(src, out)
    _check(_LIB.moe_probe_read(_ptr(src), _nbytes(src), _ptr(out), out.numel(), _stream(stream, dev)),
           "moe_probe_read")


def moe_probe_copy(src: torch.Tensor, dst: torch.Tensor, stream=None) -> None:
    """Copy src into dst (same byte size)."""
    if _nbytes(dst) < _nbytes(src):
        raise MoeError("dst smaller than src")
    dev = _dev(src, dst)
    _check(_LIB.moe_probe_copy(_ptr(src), _ptr(dst), _nbytes(src), _stream(stream, dev)), "moe_probe_copy")


def moe_probe_mfma(iters: int, blocks: int, out: torch.Tensor, stream=None) -> None:
    """blocks x 256 threads, each wave iters rounds of 4 bf16 32x32x16 MFMAs; out: f32 [blocks*256]."""
    _req(out, "out", _F32, blocks * 256)
    dev = _dev(out)
    _check(_LIB.moe_probe_mfma(iters, blocks, _ptr(out), _stream(stream, dev)), "moe_probe_mfma")


def moe_probe_mfma_clock(iters: int, blocks: int, toggle: bool, out: torch.Tensor,
                         clocks: Optional[torch.Tensor] = None, stream=None) -> None:
    """The MFMA loop of moe_probe_mfma; toggle: operands change every round as
    real data does.  clocks: int64 [blocks*4*2] (per wave: shader cycles, then
    100 MHz ticks of the loop) or None."""
    _req(out, "out", _F32, blocks * 256)
    if clocks is not None:
        _req(clocks, "clocks", torch.int64, blocks * 4 * 2)
    dev = _dev(out, clocks)
    _check(_LIB.moe_probe_mfma_clock(iters, blocks, 1 if toggle else 0, _ptr(out), _ptr(clocks), _stream(stream, dev)),
           "moe_probe_mfma_clock")


def moe_probe_gate_loads(logits: torch.Tensor, K: int, topk_weights: torch.Tensor, topk_ids: torch.Tensor,
                         token_expert_indices: Optional[torch.Tensor] = None, stream=None) -> None:
    """The bf16 gate's loads and stores without its selection (load-only ceiling)."""
    _req(logits, "logits", _BF16, ndim=2)
    T, E = logits.shape
    _req(topk_weights, "topk_weights", _F32, T * K)
    _req(topk_ids, "topk_ids", _I32, T * K)
    _req(token_expert_indices, "token_expert_indices", _I32, T * K)
    dev = _dev(logits, topk_weights, topk_ids, token_expert_indices)
    _check(_LIB.moe_probe_gate_loads(_ptr(logits), T, E, K, _ptr(topk_weights), _ptr(topk_ids),
                                     _ptr(token_expert_indices), _stream(stream, dev)), "moe_probe_gate_loads")
