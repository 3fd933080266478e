"""The generic persistent scheduler (moe_grouped_ffn_control, the A/B control
of the compact path) computes the same FFN: checked against the oracle on
every decode route pattern, MXFP4 and ragged shapes, and repeatable."""
import numpy as np
import pytest
import torch

import mixture_experts_routing_amd as moe
import oracle
import synth
from gpu_util import case_to_device, dev_bf16, host_f64, rel_max_err

pytestmark = pytest.mark.gpu

TOL = {"bf16": 1e-2, "mxfp4": 3e-2}


def run_control(c, d):
    counts, offsets, s2r, r2s = moe.moe_route_compact(d["topk_ids"], d["expert_map"], c.E_local, E_global=c.E_global)
    y = moe.moe_grouped_ffn_control(d["x"], c.K, d["w1"], d["w2"], counts, offsets, r2s, d["w1_scale"],
                                    d["w2_scale"])
    out = moe.moe_combine(y, d["topk_weights"], s2r)
    torch.cuda.synchronize()
    return y, out


def check(c, d, tag):
    print(f"[control] {tag} {c.name}", flush=True)
    ref = oracle.moe_layer(c)
    y, out = run_control(c, d)
    R = int(ref["offsets"][-1])
    ey = rel_max_err(host_f64(y[:R]), ref["y"])
    eo = rel_max_err(host_f64(out), ref["out"])
    print(f"[control] {tag}: y err {ey:.3e} out err {eo:.3e}", flush=True)
    assert ey <= TOL[c.w_dtype] and eo <= TOL[c.w_dtype]
    y2, out2 = run_control(c, d)
    assert torch.equal(y2[:R], y[:R]) and torch.equal(out2, out)


@pytest.fixture(scope="module")
def decode_weights_dev():
    w1, w2 = synth.decode_weights(0)
    return dev_bf16(w1), dev_bf16(w2)


@pytest.mark.parametrize("pattern", synth.decode_patterns())
def test_control_decode_patterns(pattern, decode_weights_dev):
    c = synth.decode_case(pattern, "random", seed=2)
    d = case_to_device(synth.decode_case(pattern, "random", seed=2, with_weights=False))
    d["w1"], d["w2"] = decode_weights_dev
    d["w1_scale"] = d["w2_scale"] = None
    check(c, d, "decode")


@pytest.mark.parametrize("T", [2, 16])
def test_control_mxfp4(T):
    c = synth.mxfp4_case(T, "all_local", seed=4)
    check(c, case_to_device(c), "mxfp4")


def test_control_many_rows_one_expert():
    # one expert with 40 rows: three 16-row blocks per work item
    c = synth.decode_case("all_dup", "contiguous", seed=0, with_weights=False)
    T, K = 10, 4
    ids = np.full((T, K), c.topk_ids[0, 0], np.int32)
    w = np.full((T, K), 0.25, np.float32)
    x = synth.bf16_normal((T, c.H), 1.0, 3, 1)
    w1, w2 = synth.decode_weights(0)
    c2 = synth.MoECase(name="one_expert_40_rows", T=T, E_global=c.E_global, E_local=c.E_local, K=K, H=c.H, F=c.F,
                       renormalize=False, x_dtype="bf16", w_dtype="bf16", out_dtype="bf16", x=x, w1=w1, w2=w2,
                       topk_ids=ids, topk_weights=w, expert_map=c.expert_map)
    check(c2, case_to_device(c2), "rows40")
