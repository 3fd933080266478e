"""The timed path of the benchmark, call for call: moe_topk_compact (gate +
route compaction), moe_pack_ffn_weights once, moe_grouped_ffn on the packed
weights, moe_combine -- at the full prefill size (T=4096, E=128 all local,
top-8 renormalised, H=2048, F=768, bf16), checked against the oracle: ids and
the compaction arrays bit for bit, gate weights within 1e-6 relative, the
layer output within 1e-2 of max|ref|."""
import numpy as np
import pytest
import torch

import mixture_experts_routing_amd as moe
import oracle
import synth
from gpu_util import case_to_device, host_f64, host_i, rel_max_err

pytestmark = pytest.mark.gpu


def test_bench_prefill_path_matches_oracle():
    c = synth.prefill_layer(0)
    d = case_to_device(c)
    T, E, K, H, F = c.T, c.E_local, c.K, c.H, c.F
    print(f"[bench path] prefill T={T} E={E} K={K} H={H} F={F}", flush=True)
    w1, w2 = moe.moe_pack_ffn_weights(d["w1"], d["w2"])
    (tw, tid, tei), (counts, offsets, s2r, r2s) = moe.moe_topk_compact(d["logits"], K, True, "softmax", None, E)
    y = moe.moe_grouped_ffn(d["x"], K, w1, w2, counts, offsets, r2s, tiled=True)
    out = moe.moe_combine(y, tw, s2r)
    torch.cuda.synchronize()
    ref = oracle.moe_layer(c)
    assert np.array_equal(host_i(tid), ref["topk_ids"])
    w = tw.cpu().numpy().astype(np.float64)
    assert np.max(np.maximum(np.abs(w - ref["topk_weights"]) - 2.0 ** -126, 0.0) / ref["topk_weights"]) <= 1e-6
    for name, got in zip(("counts", "offsets", "slot_to_row", "row_to_slot"), (counts, offsets, s2r, r2s)):
        assert np.array_equal(host_i(got), ref[name]), name
    R = int(ref["offsets"][-1])
    ey = rel_max_err(host_f64(y[:R]), ref["y"])
    eo = rel_max_err(host_f64(out), ref["out"])
    print(f"[bench path] y err {ey:.3e} out err {eo:.3e}", flush=True)
    assert ey <= 1e-2 and eo <= 1e-2
