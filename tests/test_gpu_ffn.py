"""GPU parity of moe_grouped_ffn and moe_combine (and the whole layer) against
the oracle.  Bound: max|err| / max|ref| <= 1e-2 for bf16 weights, <= 3e-2 for
MXFP4 weights (fp32 accumulation on the GPU, fp64 oracle); fp32 weights are
held to the bf16 bound and their measured error is printed."""
import numpy as np
import pytest
import torch

import mixture_experts_routing_amd as moe
import oracle
import synth
from gpu_util import DEV, TORCH_DT, case_to_device, dev_bf16, dev_f32, dev_i32, host_f64, host_i, rel_max_err

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-2, "bf16": 1e-2, "mxfp4": 3e-2}


def run_layer(c, d=None):
    d = d or case_to_device(c)
    print(f"[layer] {c.name}", flush=True)
    res = moe.moe_layer(d["x"], d["w1"], d["w2"], c.K, logits=d.get("logits"), renormalize=c.renormalize,
                        topk_ids=d.get("topk_ids"), topk_weights=d.get("topk_weights"), expert_map=d["expert_map"],
                        E_global=c.E_global, w1_scale=d["w1_scale"], w2_scale=d["w2_scale"],
                        out_dtype=TORCH_DT[c.out_dtype], y_dtype=TORCH_DT[c.out_dtype])
    torch.cuda.synchronize()
    return res


def compare_layer(c, res, ref, tag=""):
    tol = TOL[c.w_dtype]
    if c.topk_ids is None:
        assert np.array_equal(host_i(res["topk_ids"]), ref["topk_ids"])
    for k in ("counts", "offsets", "slot_to_row", "row_to_slot"):
        assert np.array_equal(host_i(res[k]), ref[k]), k
    R = int(ref["offsets"][-1])
    ey = rel_max_err(host_f64(res["y"][:R]), ref["y"])
    eo = rel_max_err(host_f64(res["out"]), ref["out"])
    print(f"[layer] {tag} {c.name}: R={R} y err {ey:.3e}  out err {eo:.3e}  (bound {tol})", flush=True)
    assert ey <= tol and eo <= tol
    if R < c.T * c.K or c.topk_ids is not None:
        # tokens with only remote routes are exact zeros
        s2r = ref["slot_to_row"].reshape(c.T, c.K)
        remote_only = np.all(s2r < 0, axis=1)
        if remote_only.any():
            assert np.all(host_f64(res["out"])[remote_only] == 0.0)
    return ey, eo


def test_tiny_layer_f32():
    c = synth.tiny_layer(0)
    res = run_layer(c)
    ref = oracle.moe_layer(c)
    ey, eo = compare_layer(c, res, ref, "tiny")
    # fp32 end to end: far inside the bound
    assert ey < 1e-5 and eo < 1e-5


@pytest.mark.parametrize("T,Eg,El,K,H,F,renorm", [(37, 12, 8, 3, 96, 40, False),   # odd sizes, remote routes
                                                    (200, 8, 8, 4, 64, 128, True),     # renormalised, all local
                                                    (1, 5, 3, 5, 32, 16, True)])       # one token, every expert
def test_f32_layer_shapes(T, Eg, El, K, H, F, renorm):
    """The fp32 path (every step in fp32) at shapes other than the tiny
    layer's: fp32 end to end stays far inside the bound of the fp64 oracle."""
    c = synth.tiny_layer(T)
    c.name = f"f32_T{T}_Eg{Eg}_El{El}_K{K}_H{H}_F{F}"
    c.T, c.E_global, c.E_local, c.K, c.H, c.F, c.renormalize = T, Eg, El, K, H, F, renorm
    c.logits = synth.f32_normal((T, Eg), 1.0, T, 71)
    c.x = synth.f32_normal((T, H), 1.0, T, 72)
    c.w1 = synth.f32_normal((El, 2 * F, H), 0.05, T, 73)
    c.w2 = synth.f32_normal((El, H, F), 0.05, T, 74)
    c.expert_map = synth.random_expert_map(Eg, El, T) if El < Eg else None
    res = run_layer(c)
    ref = oracle.moe_layer(c)
    ey, eo = compare_layer(c, res, ref, "f32 shapes")
    assert ey < 1e-5 and eo < 1e-5


@pytest.fixture(scope="module")
def decode_weights_dev():
    w1, w2 = synth.decode_weights(0)
    return dev_bf16(w1), dev_bf16(w2)


@pytest.mark.parametrize("pattern", synth.decode_patterns())
@pytest.mark.parametrize("map_kind", ["contiguous", "random"])
def test_decode_layer_patterns(pattern, map_kind, decode_weights_dev):
    c = synth.decode_case(pattern, map_kind, seed=1)
    d = case_to_device(synth.decode_case(pattern, map_kind, seed=1, with_weights=False))
    d["w1"], d["w2"] = decode_weights_dev
    d["w1_scale"] = d["w2_scale"] = None
    res = run_layer(c, d)
    ref = oracle.moe_layer(c)
    compare_layer(c, res, ref, "decode")
    if pattern == "all_remote":
        assert torch.count_nonzero(res["out"]) == 0


def test_prefill_layer_full():
    c = synth.prefill_layer(0)
    res = run_layer(c)
    ref = oracle.moe_layer(c)
    compare_layer(c, res, ref, "prefill")
    # deterministic: a second run is bit-identical
    again = run_layer(c)
    assert torch.equal(again["out"], res["out"]) and torch.equal(again["y"], res["y"])


@pytest.mark.parametrize("T", [2, 16, 64])
@pytest.mark.parametrize("routes", ["uniform", "all_local"])
def test_mxfp4_layer(T, routes):
    c = synth.mxfp4_case(T, routes, seed=0)
    res = run_layer(c)
    ref = oracle.moe_layer(c)
    compare_layer(c, res, ref, "mxfp4")


@pytest.mark.parametrize("w_dtype", ["bf16", "mxfp4"])
@pytest.mark.parametrize("H,F", [(256, 160), (128, 128), (96, 64), (512, 384)])
def test_small_shapes_many_tiles_ragged(w_dtype, H, F):
    # several M-tiles per expert, ragged last tiles, K step 32 and 128 paths
    rng = np.random.default_rng(H * 7 + F)
    T, K, Eg, El = 301, 4, 12, 5
    emap = synth.random_expert_map(Eg, El, seed=H)
    ids = np.stack([rng.choice(Eg, size=K, replace=False) for _ in range(T)]).astype(np.int32)
    ids[:40] = np.flatnonzero(emap >= 0)[0]  # a hot expert with > 64 rows
    w = rng.dirichlet(np.ones(K), size=T).astype(np.float32)
    x = synth.bf16_normal((T, H), 1.0, 7, 1)
    if w_dtype == "bf16":
        w1 = synth.bf16_normal((El, 2 * F, H), 0.05, 7, 2)
        w2 = synth.bf16_normal((El, H, F), 0.05, 7, 3)
        w1s = w2s = None
    else:
        w1 = rng.integers(0, 256, size=(El, 2 * F, H // 2), dtype=np.uint8)
        w2 = rng.integers(0, 256, size=(El, H, F // 2), dtype=np.uint8)
        w1s = rng.integers(119, 128, size=(El, 2 * F, H // 32), dtype=np.uint8)
        w2s = rng.integers(119, 128, size=(El, H, F // 32), dtype=np.uint8)
    c = synth.MoECase(name=f"small_{w_dtype}_{H}_{F}", T=T, E_global=Eg, E_local=El, K=K, H=H, F=F,
                      renormalize=False, x_dtype="bf16", w_dtype=w_dtype, out_dtype="bf16", x=x, w1=w1, w2=w2,
                      w1_scale=w1s, w2_scale=w2s, topk_ids=ids, topk_weights=w, expert_map=emap)
    res = run_layer(c)
    ref = oracle.moe_layer(c)
    compare_layer(c, res, ref, "small")


def small_case(w_dtype, T, K, Eg, El, H, F, hot, seed, out_dtype="bf16"):
    rng = np.random.default_rng(seed)
    emap = synth.random_expert_map(Eg, El, seed=seed)
    ids = np.stack([rng.choice(Eg, size=K, replace=False) for _ in range(T)]).astype(np.int32)
    if hot:
        ids[:, 0] = np.flatnonzero(emap >= 0)[0]
    w = rng.dirichlet(np.ones(K), size=T).astype(np.float32)
    x = synth.bf16_normal((T, H), 1.0, seed, 1)
    if w_dtype == "bf16":
        w1 = synth.bf16_normal((El, 2 * F, H), 0.05, seed, 2)
        w2 = synth.bf16_normal((El, H, F), 0.05, seed, 3)
        w1s = w2s = None
    else:
        w1 = rng.integers(0, 256, size=(El, 2 * F, H // 2), dtype=np.uint8)
        w2 = rng.integers(0, 256, size=(El, H, F // 2), dtype=np.uint8)
        w1s = rng.integers(119, 128, size=(El, 2 * F, H // 32), dtype=np.uint8)
        w2s = rng.integers(119, 128, size=(El, H, F // 32), dtype=np.uint8)
    return synth.MoECase(name=f"small_{w_dtype}_T{T}_{H}_{F}", T=T, E_global=Eg, E_local=El, K=K, H=H, F=F,
                         renormalize=False, x_dtype="bf16", w_dtype=w_dtype, out_dtype=out_dtype, x=x, w1=w1,
                         w2=w2, w1_scale=w1s, w2_scale=w2s, topk_ids=ids, topk_weights=w, expert_map=emap)


@pytest.mark.parametrize("w_dtype", ["bf16", "mxfp4"])
@pytest.mark.parametrize("H,F", [(96, 64), (256, 160), (512, 384), (1024, 4096), (1120, 160), (2080, 1056),
                                 (4128, 96)])
@pytest.mark.parametrize("T", [1, 3, 9])
@pytest.mark.parametrize("out_dtype", ["bf16", "f32"])
def test_decode_split_k_shapes(w_dtype, H, F, T, out_dtype):
    # few rows per expert: the K dimension is split over the waves of a block
    # and reduced in a fixed order; with 35, 65 or 33 K units (the 1120 and
    # 2080 shapes) the chosen splits leave uneven and empty K chunks; H = 4128
    # is past the longest MXFP4 A row staged in LDS (GEMM1 reads it directly)
    c = small_case(w_dtype, T, 4, 12, 6, H, F, hot=(T == 9), seed=H + F + T, out_dtype=out_dtype)
    res = run_layer(c)
    ref = oracle.moe_layer(c)
    compare_layer(c, res, ref, "split")
    again = run_layer(c)
    R = int(ref["offsets"][-1])  # rows >= R of y are never written
    assert torch.equal(again["y"][:R], res["y"][:R]) and torch.equal(again["out"], res["out"])


@pytest.mark.parametrize("w_dtype,H,F", [("mxfp4", 4096, 512), ("mxfp4", 4128, 96), ("mxfp4", 256, 2080),
                                         ("mxfp4", 512, 384), ("bf16", 512, 384), ("bf16", 1120, 160),
                                         ("bf16", 256, 2080)])
@pytest.mark.parametrize("hot", [(40, 20), (32, 17)])
def test_decode_tiles_past_16_rows(w_dtype, H, F, hot):
    # Decode regime (fewer than 24 slots per local expert) with experts past
    # 16 rows: one 32-row tile per expert up to 32 rows, both 16-row halves
    # fed by each weight byte; 40 rows = a full 32-row tile and an 8-row one.
    # MXFP4 A rows go through LDS in chunks of whole K units where 32 rows of
    # the reduction do not fit (H = 4096, 4128 for GEMM1; F = 2080 for GEMM2,
    # whose last chunk holds one unit).
    T, K, Eg, El = 40, 4, 16, 8
    rng = np.random.default_rng(H + F + hot[0])
    emap = synth.random_expert_map(Eg, El, seed=H + F)
    loc = np.flatnonzero(emap >= 0)
    others = np.setdiff1d(np.arange(Eg), loc[:2])
    rows = []
    for t in range(T):  # distinct ids per row: the forced hot experts, then others
        fixed = ([loc[0]] if t < hot[0] else []) + ([loc[1]] if t < hot[1] else [])
        rest = rng.choice(others, size=K - len(fixed), replace=False)
        rows.append(np.concatenate([np.array(fixed, dtype=np.int64), rest]))
    ids = np.stack(rows)
    ids = ids.astype(np.int32)
    c0 = small_case(w_dtype, T, K, Eg, El, H, F, hot=False, seed=H + F + hot[1])
    c = synth.MoECase(**{**c0.__dict__, "name": f"rows32_{w_dtype}_{H}_{F}_{hot}", "topk_ids": ids,
                         "expert_map": emap})
    ref = oracle.moe_layer(c)
    counts = ref["counts"]
    assert counts.max() == hot[0] and np.sort(counts)[-2] >= hot[1] and T * K / El < 24
    res = run_layer(c)
    compare_layer(c, res, ref, "rows32")
    again = run_layer(c)
    R = int(ref["offsets"][-1])
    assert torch.equal(again["y"][:R], res["y"][:R]) and torch.equal(again["out"], res["out"])


@pytest.mark.parametrize("w_dtype", ["bf16", "mxfp4"])
def test_decode_many_experts_past_16_rows(w_dtype):
    # more than 64 local experts: the decode kernels find tiles through a
    # scan of counts instead of the one-wave expert table; a few experts hold
    # 17-40 rows (32-row tiles, a second tile past 32)
    T, K, Eg, El, H, F = 48, 4, 160, 96, 256, 160
    rng = np.random.default_rng(96)
    emap = synth.random_expert_map(Eg, El, seed=96)
    loc = np.flatnonzero(emap >= 0)
    hot = loc[[0, 50, 95]]
    rows = []
    for t in range(T):
        fixed = [hot[0]] + ([hot[1]] if t < 20 else []) + ([hot[2]] if t % 2 == 0 else [])
        pool = np.setdiff1d(np.arange(Eg), hot)
        rows.append(np.concatenate([np.array(fixed), rng.choice(pool, size=K - len(fixed), replace=False)]))
    c0 = small_case(w_dtype, T, K, Eg, El, H, F, hot=False, seed=96)
    c = synth.MoECase(**{**c0.__dict__, "name": f"many_experts_{w_dtype}", "topk_ids": np.stack(rows).astype(np.int32),
                         "expert_map": emap})
    ref = oracle.moe_layer(c)
    assert ref["counts"].max() == T and T * K / El < 24
    res = run_layer(c)
    compare_layer(c, res, ref, "many-experts")
    if w_dtype == "mxfp4":
        with moe.mxfp4_mma(moe.MOE_MXFP4_MMA_F8F6F4):
            res4 = run_layer(c)
        compare_layer(c, res4, ref, "many-experts f8f6f4")


@pytest.mark.parametrize("pattern", ["same", "all_dup", "twelve_local"])
def test_decode_deterministic(pattern, decode_weights_dev):
    c = synth.decode_case(pattern, "random", seed=5, with_weights=False)
    d = case_to_device(c)
    d["w1"], d["w2"] = decode_weights_dev
    d["w1_scale"] = d["w2_scale"] = None
    a = run_layer(c, d)
    b = run_layer(c, d)
    R = int(a["offsets"][-1])
    assert torch.equal(a["y"][:R], b["y"][:R]) and torch.equal(a["out"], b["out"])


@pytest.mark.parametrize("ydt,odt", [("bf16", "bf16"), ("bf16", "f32"), ("f32", "f32"), ("f32", "bf16")])
@pytest.mark.parametrize("H", [4096, 2048, 136, 7])
def test_combine(ydt, odt, H):
    rng = np.random.default_rng(H)
    T, K = 37, 6
    N = T * K
    s2r = rng.permutation(N).astype(np.int32)
    s2r[rng.random(N) < 0.3] = -1
    s2r[:K] = -1  # token 0 all remote
    R = N
    y = rng.standard_normal((R, H)).astype(np.float32)
    if ydt == "bf16":
        yb = synth.round_to_bf16_bits(y)
        y_dev = dev_bf16(yb)
        y_ref = oracle.decode_bf16(yb)
    else:
        y_dev = dev_f32(y)
        y_ref = y.astype(np.float64)
    w = rng.random((T, K)).astype(np.float32)
    print(f"[combine] y={ydt} out={odt} H={H}", flush=True)
    out = moe.moe_combine(y_dev, dev_f32(w), dev_i32(s2r), out_dtype=TORCH_DT[odt])
    torch.cuda.synchronize()
    ref = oracle.combine(y_ref, w, s2r, T, K)
    got = host_f64(out)
    assert np.all(got[0] == 0.0)
    # fp32 accumulation (~1e-7 of the summed magnitudes); a bf16 output adds
    # one rounding to nearest, at most half an ulp = 2^-8 of each value
    scale = np.max(np.abs(ref))
    slack = 2.0 ** -8 * np.abs(ref) if odt == "bf16" else 0.0
    assert np.all(np.abs(got - ref) <= slack + 1e-6 * scale), np.max(np.abs(got - ref) - slack)
