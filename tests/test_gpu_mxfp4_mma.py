"""MXFP4 expert GEMMs on the CDNA4 block-scaled matrix cores
(MOE_MXFP4_MMA_F8F6F4): the e2m1 codes and e8m0 scales go to
v_mfma_scale_f32_16x16x128_f8f6f4 as stored, the bf16 activations as two e4m3
terms per 32 elements.  Every case is held to the MXFP4 bound of the oracle
comparison (max|err| / max|ref| <= 3e-2, the fp64 oracle on the unquantised
bf16 activations) and run twice for bit-identical results; the measured
error is printed beside that of the bf16-widening arithmetic."""
import numpy as np
import pytest
import torch

import mixture_experts_routing_amd as moe
import oracle
import synth
from gpu_util import case_to_device, host_f64, rel_max_err
from test_gpu_ffn import compare_layer, run_layer, small_case

pytestmark = pytest.mark.gpu

F4 = moe.MOE_MXFP4_MMA_F8F6F4


def f32_y(c, d, res):
    """y in f32 for the routes of a layer run (no bf16 rounding of the output)."""
    y = moe.moe_grouped_ffn(d["x"], c.K, d["w1"], d["w2"], res["counts"], res["offsets"], res["row_to_slot"],
                            d["w1_scale"], d["w2_scale"], y_dtype=torch.float32)
    torch.cuda.synchronize()
    return y


def both_modes(c, tag):
    ref = oracle.moe_layer(c)
    d = case_to_device(c)
    base = run_layer(c, d)
    R = int(ref["offsets"][-1])
    eb = rel_max_err(host_f64(base["out"]), ref["out"])
    yb = f32_y(c, d, base)[:R]
    with moe.mxfp4_mma(F4):
        res = run_layer(c, d)
        ey, eo = compare_layer(c, res, ref, f"f8f6f4 {tag}")
        again = run_layer(c, d)
        yf = f32_y(c, d, res)[:R]
    assert torch.equal(again["y"][:R], res["y"][:R]) and torch.equal(again["out"], res["out"])
    # the f32 y of both arithmetics against the oracle's fp64 y (the GPU still rounds act to bf16 between
    # the GEMMs), and against each other
    efy = rel_max_err(host_f64(yf), ref["y"])
    eby = rel_max_err(host_f64(yb), ref["y"])
    dfb = rel_max_err(host_f64(yf), host_f64(yb))
    print(f"[f8f6f4] {tag} {c.name}: out err {eo:.3e} (bf16 widening {eb:.3e}); f32 y err {efy:.3e} "
          f"(bf16 widening {eby:.3e}); f32 y between the two {dfb:.3e}", flush=True)
    assert efy <= 3e-2
    return ey, eo


@pytest.mark.parametrize("T", [2, 16, 64])
@pytest.mark.parametrize("routes", ["uniform", "all_local"])
def test_f8f6f4_mxfp4_layer(T, routes):
    both_modes(synth.mxfp4_case(T, routes, seed=0), "cfg")


@pytest.mark.parametrize("H,F", [(96, 64), (256, 160), (1120, 160), (2080, 1056), (4128, 96), (256, 2080)])
@pytest.mark.parametrize("T", [1, 9])
def test_f8f6f4_ragged_units(H, F, T):
    # 3, 35, 65 and 129 K units: MFMA steps of 4 units with a partial last
    # step (zero codes past the end), uneven split shares, chunked staging
    both_modes(small_case("mxfp4", T, 4, 12, 6, H, F, hot=(T == 9), seed=H + F + T), "ragged")


@pytest.mark.parametrize("H,F", [(4096, 512), (512, 384)])
def test_f8f6f4_tiles_past_16_rows(H, F):
    # 40 rows on one expert (a 32-row tile and an 8-row tile), 20 on another
    T, K, Eg, El = 40, 4, 16, 8
    rng = np.random.default_rng(H + F)
    emap = synth.random_expert_map(Eg, El, seed=H)
    loc = np.flatnonzero(emap >= 0)
    others = np.setdiff1d(np.arange(Eg), loc[:2])
    rows = []
    for t in range(T):
        fixed = [loc[0]] + ([loc[1]] if t < 20 else [])
        rows.append(np.concatenate([np.array(fixed), rng.choice(others, size=K - len(fixed), replace=False)]))
    c0 = small_case("mxfp4", T, K, Eg, El, H, F, hot=False, seed=H + F)
    c = synth.MoECase(**{**c0.__dict__, "name": f"f4_rows32_{H}_{F}", "topk_ids": np.stack(rows).astype(np.int32),
                         "expert_map": emap})
    both_modes(c, "rows32")


def test_f8f6f4_activation_magnitudes():
    # units of zeros, of equal values, of magnitudes spread over 2^-20..2^20,
    # and maxima just under and just over 1.75 * 2^k (the boundary of the
    # exponent choice that keeps every element at or below 448 * 2^e)
    T, H, F = 8, 256, 128
    c = small_case("mxfp4", T, 4, 12, 6, H, F, hot=True, seed=5)
    x = np.frombuffer(c.x.tobytes(), dtype=np.uint16).reshape(T, H).copy()
    f = synth.bf16_normal((T, H), 1.0, 5, 9)
    vals = np.frombuffer(f.tobytes(), dtype=np.uint16).reshape(T, H).astype(np.uint32) << 16
    fv = vals.view(np.float32).reshape(T, H)
    fv[0, :] = 0.0
    fv[1, :] = 3.0
    fv[2, :] *= np.exp2(np.linspace(-20, 20, H)).astype(np.float32)
    fv[3, ::32] = 1.75 * 64.0       # every unit's largest element has significand 1.75 exactly
    fv[4, ::32] = 1.7578125 * 64.0  # the next bf16 above it
    fv[5, :] = -fv[5, :] * 1e3
    xb = (fv.view(np.uint32) >> 16).astype(np.uint16)
    c = synth.MoECase(**{**c.__dict__, "name": "f4_magnitudes", "x": xb})
    both_modes(c, "magnitudes")


@pytest.mark.parametrize("T,routes", [(2, "uniform"), (2, "all_local")])
def test_f8f6f4_fused_path(T, routes):
    c = synth.mxfp4_case(T, routes, seed=6)
    d = case_to_device(c)
    ref = oracle.moe_layer(c)
    with moe.mxfp4_mma(F4):
        out, routes_ = moe.moe_fused_experts(d["x"], d["topk_ids"], d["topk_weights"], d["w1"], d["w2"],
                                             d["expert_map"], c.E_global, d["w1_scale"], d["w2_scale"])
        torch.cuda.synchronize()
    eo = rel_max_err(host_f64(out), ref["out"])
    print(f"[f8f6f4] fused {c.name}: out err {eo:.3e}", flush=True)
    assert eo <= 3e-2


def test_mode_switch_restores():
    assert moe.moe_get_mxfp4_mma() == moe.MOE_MXFP4_MMA_BF16
    with moe.mxfp4_mma(F4):
        assert moe.moe_get_mxfp4_mma() == F4
    assert moe.moe_get_mxfp4_mma() == moe.MOE_MXFP4_MMA_BF16
    with pytest.raises(moe.MoeError):
        moe.moe_set_mxfp4_mma(7)


@pytest.mark.parametrize("T", [1, 9])
def test_scale_range_both_arithmetics(T):
    # e8m0 scales far from 2^0 (2^-27 .. 2^23 for W1, 2^-37 .. 2^13 for W2,
    # with some blocks at byte 0 = 2^-127), so the scale reaches the matrix
    # cores (f8f6f4) or the widening (bf16) over a wide range; outputs stay
    # finite and within the MXFP4 bound of the oracle in both arithmetics
    H, F = 512, 256
    c = small_case("mxfp4", T, 4, 12, 6, H, F, hot=True, seed=77 + T)  # a local expert in every row
    rng = np.random.default_rng(5 + T)
    w1s = rng.integers(100, 151, size=c.w1_scale.shape, dtype=np.uint8)
    w2s = rng.integers(90, 141, size=c.w2_scale.shape, dtype=np.uint8)
    w1s[rng.random(w1s.shape) < 0.05] = 0
    w2s[rng.random(w2s.shape) < 0.05] = 0
    c = synth.MoECase(**{**c.__dict__, "name": f"mx_scales_T{T}", "w1_scale": w1s, "w2_scale": w2s})
    ey, eo = both_modes(c, "scales")
    assert np.isfinite(ey) and np.isfinite(eo)
    assert oracle.moe_layer(c)["offsets"][-1] > 0  # not an all-remote batch
