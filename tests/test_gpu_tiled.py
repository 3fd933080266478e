"""Tile-packed bf16 weights (MOE_BF16_TILED): moe_pack_ffn_weights writes
exactly the layout the header defines (checked against a numpy restatement
of that definition, bit for bit), and moe_grouped_ffn on packed weights
gives the same y as on row-major weights (bit for bit where both take the
tiled kernels) and matches the oracle everywhere."""
import numpy as np
import pytest
import torch

import mixture_experts_routing_amd as moe
import oracle
import synth
from gpu_util import DEV, case_to_device, dev_bf16, host_f64, rel_max_err

pytestmark = pytest.mark.gpu


def pack_reference(w: np.ndarray, gated: bool, F: int) -> np.ndarray:
    """The header's layout, restated: [E, rows, K] bf16 bits -> flat packed."""
    E, rows, K = w.shape
    out = np.empty((E, rows // 256, K // 32, 256, 4, 8), np.uint16)
    R = np.arange(256)
    swz = ((R >> 1) ^ (R >> 2)) & 3
    for nt in range(rows // 256):
        if gated:
            src = np.where((R >> 5) & 1, F, 0) + nt * 128 + (R >> 6) * 32 + (R & 31)
        else:
            src = nt * 256 + R
        blk = w[:, src, :].reshape(E, 256, K // 32, 4, 8)  # [E, R, kt, logical piece, 8]
        for r in range(256):
            for p in range(4):
                out[:, nt, :, r, p, :] = blk[:, r, :, p ^ swz[r], :]
    return out.reshape(-1)


@pytest.mark.parametrize("E,H,F", [(2, 256, 128), (3, 512, 384), (1, 2048, 768)])
def test_pack_layout_bit_exact(E, H, F):
    print(f"[tiled] pack E={E} H={H} F={F}", flush=True)
    w1 = synth.bf16_normal((E, 2 * F, H), 1.0, 11, 1)
    w2 = synth.bf16_normal((E, H, F), 1.0, 11, 2)
    t1, t2 = moe.moe_pack_ffn_weights(dev_bf16(w1), dev_bf16(w2))
    torch.cuda.synchronize()
    g1 = t1.view(torch.int16).cpu().numpy().view(np.uint16).reshape(-1)
    g2 = t2.view(torch.int16).cpu().numpy().view(np.uint16).reshape(-1)
    assert np.array_equal(g1, pack_reference(w1, True, F))
    assert np.array_equal(g2, pack_reference(w2, False, F))


def run(c, d, tiled):
    res = moe.moe_layer(d["x"], d["w1"], d["w2"], c.K, logits=d.get("logits"), renormalize=c.renormalize,
                        topk_ids=d.get("topk_ids"), topk_weights=d.get("topk_weights"),
                        expert_map=d.get("expert_map"), E_global=c.E_global, tiled=tiled)
    torch.cuda.synchronize()
    return res


CASES = {
    # name: (T, E, K, H, F) of a prefill-style layer (gate included)
    "prefill_small": (1024, 16, 4, 256, 128),   # ~256 rows per expert: 320-row tiles
    "mid_rows": (300, 8, 4, 512, 384),          # ~150 rows per expert: 128-row tiles
    "few_rows": (24, 16, 2, 256, 256),          # ~3 rows per expert: tiled kernels anyway
}


@pytest.mark.parametrize("name", list(CASES))
def test_tiled_layer_matches_rowmajor_and_oracle(name):
    T, E, K, H, F = CASES[name]
    c = synth.prefill_layer(seed=7, T=T, E=E, K=K, H=H, F=F)
    d = case_to_device(c)
    print(f"[tiled] layer {name} T={T} E={E} K={K} H={H} F={F}", flush=True)
    ref = oracle.moe_layer(c)
    row = run(c, d, False)
    t1, t2 = moe.moe_pack_ffn_weights(d["w1"], d["w2"])
    d_t = dict(d)
    d_t["w1"], d_t["w2"] = t1, t2
    til = run(c, d_t, True)
    R = int(ref["offsets"][-1])
    ey = rel_max_err(host_f64(til["y"][:R]), ref["y"])
    eo = rel_max_err(host_f64(til["out"]), ref["out"])
    print(f"[tiled] {name}: y err {ey:.3e} out err {eo:.3e}", flush=True)
    assert ey <= 1e-2 and eo <= 1e-2
    if (T * K) // E >= 96:  # both runs take the tiled kernels: identical sums
        assert torch.equal(til["y"][:R], row["y"][:R])
        assert torch.equal(til["out"], row["out"])


def skewed_case(T, Eg, El, K, H, F, seed):
    """A prefill layer whose router favours a few experts: local expert 0 takes
    about every token (several 320-row M-tiles and a partial last one),
    experts 1 and 2 many, the last four (almost surely) none; with
    E_global > E_local some routes are remote."""
    bias = np.zeros(Eg, np.float32)
    bias[0], bias[1], bias[2] = 7.0, 3.5, 1.5
    bias[El - 4:El] = -40.0
    logits = synth.round_to_bf16_bits(synth.f32_normal((T, Eg), 2.0, seed, 91) + bias)
    c = synth.prefill_layer(seed=seed, T=T, E=El, K=K, H=H, F=F)
    c.name = f"skewed_T{T}_Eg{Eg}_El{El}_K{K}"
    c.E_global = Eg
    c.logits = logits
    c.expert_map = synth.contiguous_expert_map(Eg, El, 0) if El < Eg else None
    return c


@pytest.mark.parametrize("T,Eg,El,K,H,F", [(2048, 16, 16, 4, 256, 128),    # 320-row tiles, up to 7 per expert
                                           (1536, 24, 16, 6, 512, 256),    # and remote routes
                                           (1024, 16, 16, 2, 256, 256)])   # 128-row tiles
def test_tiled_skewed_routes(T, Eg, El, K, H, F):
    c = skewed_case(T, Eg, El, K, H, F, seed=3)
    d = case_to_device(c)
    ref = oracle.moe_layer(c)
    counts = np.diff(ref["offsets"])
    R = int(ref["offsets"][-1])
    print(f"[tiled] skewed T={T} Eg={Eg} El={El} K={K}: rows per expert {counts.tolist()}", flush=True)
    assert counts.max() > 2 * 320 and (counts == 0).sum() >= 1  # the shapes this case is for
    row = run(c, d, False)
    t1, t2 = moe.moe_pack_ffn_weights(d["w1"], d["w2"])
    d_t = dict(d)
    d_t["w1"], d_t["w2"] = t1, t2
    til = run(c, d_t, True)
    ey = rel_max_err(host_f64(til["y"][:R]), ref["y"])
    eo = rel_max_err(host_f64(til["out"]), ref["out"])
    print(f"[tiled] skewed: y err {ey:.3e} out err {eo:.3e}", flush=True)
    assert ey <= 1e-2 and eo <= 1e-2
    assert torch.equal(til["y"][:R], row["y"][:R]) and torch.equal(til["out"], row["out"])


def test_tiled_full_prefill_bit_equal_to_rowmajor():
    c = synth.prefill_layer(0)
    d = case_to_device(c)
    print("[tiled] full prefill", flush=True)
    row = run(c, d, False)
    t1, t2 = moe.moe_pack_ffn_weights(d["w1"], d["w2"])
    d["w1"], d["w2"] = t1, t2
    til = run(c, d, True)
    assert torch.equal(til["y"], row["y"]) and torch.equal(til["out"], row["out"])


def test_tiled_rejects_unsupported_shapes():
    x = torch.zeros((4, 384), dtype=torch.bfloat16, device=DEV)
    w1 = torch.zeros((2, 256, 384), dtype=torch.bfloat16, device=DEV)
    w2 = torch.zeros((2, 384, 128), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(moe.MoeError):
        moe.moe_pack_ffn_weights(w1, w2)  # H = 384 is not a multiple of 256
    counts = torch.zeros(2, dtype=torch.int32, device=DEV)
    offsets = torch.zeros(3, dtype=torch.int32, device=DEV)
    r2s = torch.full((8,), -1, dtype=torch.int32, device=DEV)
    with pytest.raises(moe.MoeError):
        moe.moe_grouped_ffn(x, 2, w1, w2, counts, offsets, r2s, tiled=True)


@pytest.mark.parametrize("T,E,K", [(1024, 16, 4), (1000, 8, 4)])
def test_tiled_f32_y_rounds_to_the_bf16_y(T, E, K):
    # The tiled epilogue stores f32 y straight from the accumulators and bf16
    # y through the per-wave LDS block: the f32 result rounded to bf16 must
    # equal the bf16 result bit for bit, and both match the oracle.  T=1000
    # leaves experts with row counts off the 32-row MFMA blocks (ragged
    # last blocks, rows masked in the store).
    H, F = 256, 128
    c = synth.prefill_layer(seed=T + E, T=T, E=E, K=K, H=H, F=F)
    d = case_to_device(c)
    print(f"[tiled] f32 y T={T} E={E} K={K}", flush=True)
    (tw, tid, tei), (counts, offsets, s2r, r2s) = moe.moe_topk_compact(d["logits"], K, c.renormalize, "softmax",
                                                                       None, E)
    t1, t2 = moe.moe_pack_ffn_weights(d["w1"], d["w2"])
    yb = moe.moe_grouped_ffn(d["x"], K, t1, t2, counts, offsets, r2s, tiled=True)
    yf = moe.moe_grouped_ffn(d["x"], K, t1, t2, counts, offsets, r2s, tiled=True, y_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = oracle.moe_layer(c)
    R = int(ref["offsets"][-1])
    assert int(offsets[-1].item()) == R
    assert np.any(ref["counts"] % 32 != 0)
    assert torch.equal(yf[:R].to(torch.bfloat16), yb[:R])
    assert rel_max_err(host_f64(yf[:R]), ref["y"]) <= 1e-2
