"""moe_grouped_ffn_noalloc (the allocation-free variant of moe_grouped_ffn,
act rows in the library's fixed per-GPU scratch) against moe_grouped_ffn on
the same inputs, through the C ABI: two calls in a row, the second on a
smaller batch (the scratch keeps the first call's contents), bit-identical
y rows (same kernels, same sums) and within the oracle's bound."""
import numpy as np
import pytest
import torch

import mixture_experts_routing_amd as moe
import oracle
import synth
from gpu_util import case_to_device, host_f64, rel_max_err

pytestmark = pytest.mark.gpu


def routes(c, d):
    if c.topk_ids is None:
        tw, tid, _ = moe.moe_topk_softmax(d["logits"], c.K, c.renormalize)
    else:
        tw, tid = d["topk_weights"], d["topk_ids"]
    counts, offsets, s2r, r2s = moe.moe_route_compact(tid, d["expert_map"], c.E_local, E_global=c.E_global)
    return counts, offsets, r2s


def both(c, d, tiled=False):
    counts, offsets, r2s = routes(c, d)
    w1, w2 = d["w1"], d["w2"]
    if tiled:
        w1, w2 = moe.moe_pack_ffn_weights(w1, w2)
    kw = dict(w1_scale=d["w1_scale"], w2_scale=d["w2_scale"], tiled=tiled)
    y_ref = moe.moe_grouped_ffn(d["x"], c.K, w1, w2, counts, offsets, r2s, **kw)
    y = torch.full_like(y_ref, float("nan"))
    moe.moe_grouped_ffn_noalloc(d["x"], c.K, w1, w2, counts, offsets, r2s, y=y, **kw)
    torch.cuda.synchronize()
    return y, y_ref, int(offsets[-1].item())


def check(c, y, y_ref, R):
    assert torch.equal(y[:R], y_ref[:R]), c.name
    ref = oracle.moe_layer(c)
    assert int(ref["offsets"][-1]) == R
    tol = 3e-2 if c.w_dtype == "mxfp4" else 1e-2
    err = rel_max_err(host_f64(y[:R]), ref["y"])
    print(f"[noalloc] {c.name}: R={R} y err vs oracle {err:.3e} (bound {tol})", flush=True)
    assert err <= tol


def test_noalloc_prefill_then_decode():
    # a full prefill batch (act rows 48 MiB of the 64 MiB scratch, packed
    # weights), then a two-token decode batch that reuses the same scratch
    big = synth.prefill_layer(0)
    print("[noalloc] prefill T=4096 E=128 K=8 H=2048 F=768 (tile-packed)", flush=True)
    db = case_to_device(big)
    y, y_ref, R = both(big, db, tiled=True)
    check(big, y, y_ref, R)
    del db
    small = synth.decode_case("within_row_dup", "random", seed=3)
    print("[noalloc] decode within_row_dup T=2 K=6 E_local=40 H=4096 F=2048", flush=True)
    ds = case_to_device(small)
    y, y_ref, R = both(small, ds)
    check(small, y, y_ref, R)


def test_noalloc_mxfp4_twice_shrinking():
    for T in (64, 16):
        c = synth.mxfp4_case(T, "all_local", seed=T)
        print(f"[noalloc] mxfp4 T={T} all_local", flush=True)
        d = case_to_device(c)
        y, y_ref, R = both(c, d)
        check(c, y, y_ref, R)


def test_noalloc_rejects_oversize():
    # act rows beyond 64 MiB: MOE_ERR_SCRATCH_LIMIT before anything runs
    c = synth.decode_case("same", "contiguous", seed=0)
    d = case_to_device(c)
    counts, offsets, r2s = routes(c, d)
    T = (64 << 20) // (c.K * c.F * 2) + 1
    x = torch.zeros((T, c.H), dtype=torch.bfloat16, device=d["x"].device)
    r2s_big = torch.full((T * c.K,), -1, dtype=torch.int32, device=x.device)
    y = torch.empty((T * c.K, c.H), dtype=torch.bfloat16, device=x.device)  # sized as the call needs
    with pytest.raises(moe.MoeError, match="MOE_ERR_SCRATCH_LIMIT"):
        moe.moe_grouped_ffn_noalloc(x, c.K, d["w1"], d["w2"], counts, offsets, r2s_big, y=y)
