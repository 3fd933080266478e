"""Pins of the oracle's expert FFN (GEMM1 -> silu_and_mul -> GEMM2), combine and
MXFP4 decoding (CPU only).

Sources: the FusedMoE order gate -> topk -> expand -> gemm1 -> act -> gemm2 ->
combine and the silu_and_mul activation ("Upstream Reference: Deep-Spark xllm
+ vllm", section "File Index"); the fixed-M1 oracle and direct slot-order
gather (b70 lab note "MTP1 M2 compact scheduler closure", correctness
paragraph); MXFP4 per the OCP Microscaling (MX) v1.0 format definition.
"""
import itertools
import math

import numpy as np
import pytest

import oracle
import synth


def test_silu_values_and_identity():
    assert oracle.silu(np.array([0.0]))[0] == 0.0
    # sigma(2) = 0.8807970779778823 -> silu(2) = 1.7615941559557646
    assert oracle.silu(np.array([2.0]))[0] == pytest.approx(1.7615941559557646, rel=1e-15)
    g = np.linspace(-30, 30, 601)
    # silu(g) - silu(-g) = g for every g
    np.testing.assert_allclose(oracle.silu(g) - oracle.silu(-g), g, rtol=1e-14, atol=1e-14)
    assert np.all(np.isfinite(oracle.silu(np.array([-1e4, 1e4]))))
    assert oracle.silu(np.array([-800.0]))[0] == pytest.approx(0.0, abs=1e-300)


def test_scalar_route_pins_gate_up_halves():
    # H = F = 1, x = 2, gate row 1, up row 3, W2 = 0.5:
    # y = 0.5 * silu(2) * 6 = 5.284782467867294
    # (a gate/up swap would give 0.5 * silu(6) * 2 = 5.985)
    y = oracle.ffn_route(np.array([2.0]), np.array([[1.0], [3.0]]), np.array([[0.5]]))
    assert y.shape == (1,)
    assert y[0] == pytest.approx(5.284782467867294, rel=1e-15)


def test_permutation_structure_pins_operand_orientation():
    # W1 gate = a * P1, up = b * P2, W2 = P3 (permutation matrices):
    # y[i] = silu(a * x[p1[p3[i]]]) * b * x[p2[p3[i]]] elementwise.
    rng = np.random.default_rng(0)
    H = F = 7
    p1, p2, p3 = (rng.permutation(H) for _ in range(3))
    P = lambda p: np.eye(H)[p]  # (P @ v)[i] = v[p[i]]
    a, b = 0.7, -1.3
    w1 = np.vstack([a * P(p1), b * P(p2)])
    w2 = P(p3)
    x = rng.standard_normal(H)
    y = oracle.ffn_route(x, w1, w2)
    for i in range(H):
        j = p3[i]
        g = a * x[p1[j]]
        u = b * x[p2[j]]
        assert y[i] == pytest.approx(g / (1 + math.exp(-g)) * u, rel=1e-13)
    # non-square shapes: W1 is [2F, H], W2 is [H, F]
    H, F = 5, 3
    w1 = rng.standard_normal((2 * F, H))
    w2 = rng.standard_normal((H, F))
    assert oracle.ffn_route(rng.standard_normal(H), w1, w2).shape == (H,)
    with pytest.raises(AssertionError):
        oracle.ffn_route(rng.standard_normal(H), w1.T.copy(), w2)


def test_grouped_equals_per_route_and_dense_reduction():
    c = synth.tiny_layer(0)
    res = oracle.moe_layer(c)
    xf = np.asarray(c.x, np.float64)
    # each grouped row is the M=1 evaluation of its route
    for r in range(int(res["offsets"][-1])):
        s = int(res["row_to_slot"][r])
        e = int(c.expert_map[c.topk_ids.flat[s]]) if c.expert_map is not None else int(res["topk_ids"].flat[s])
        y = oracle.ffn_route(xf[s // c.K], c.w1[e].astype(np.float64), c.w2[e].astype(np.float64))
        np.testing.assert_allclose(res["y"][r], y, rtol=1e-12, atol=1e-14)
    # duplicates of one (token, expert) give identical rows
    ids = np.array([[3, 3], [5, 3]], dtype=np.int32)
    counts, offsets, s2r, r2s = oracle.route_compact(ids, None, 8)
    y = oracle.grouped_ffn(c.x[:2], "f32", 2, c.w1, c.w2, "f32", counts, offsets, r2s)
    assert np.array_equal(y[s2r[0]], y[s2r[1]])


def test_combine_hand_example_and_remote():
    y = np.array([[1.0, 2.0], [3.0, 4.0]])
    out = oracle.combine(y, np.array([[0.25, 0.75]], np.float32), np.array([1, 0]), 1, 2)
    assert out.tolist() == [[0.25 * 3 + 0.75 * 1, 0.25 * 4 + 0.75 * 2]]
    # remote slot contributes nothing; an all-remote token is exactly zero
    out = oracle.combine(y, np.array([[0.5, 0.5], [0.3, 0.7]], np.float32), np.array([-1, 1, -1, -1]), 2, 2)
    assert out[0].tolist() == [1.5, 2.0]
    assert out[1].tolist() == [0.0, 0.0]


def test_combine_linear_in_weights_and_k1_reduction():
    rng = np.random.default_rng(2)
    T, K, H = 6, 3, 5
    y = rng.standard_normal((T * K, H))
    s2r = rng.permutation(T * K)
    w = rng.random((T, K))
    a = oracle.combine(y, w, s2r, T, K)
    b = oracle.combine(y, 2 * w, s2r, T, K)
    np.testing.assert_allclose(b, 2 * a, rtol=1e-15)
    # K = 1 with weight 1: the combine is a plain gather of rows
    s2r1 = rng.permutation(T)
    out = oracle.combine(y[:T], np.ones((T, 1)), s2r1, T, 1)
    assert np.array_equal(out, y[:T][s2r1])


def _e2m1_bitfield(code):
    """OCP MX v1.0 FP4 E2M1: sign bit 3, exponent bits 2..1 (bias 1), mantissa
    bit 0; exponent 0 is subnormal: (-1)^s * 2^0 * (m/2)."""
    s, e, m = (code >> 3) & 1, (code >> 1) & 3, code & 1
    mag = (m / 2.0) if e == 0 else 2.0 ** (e - 1) * (1 + m / 2.0)
    return -mag if s else mag


def test_mxfp4_decode_matches_bitfield_definition():
    # every byte value (both nibbles) with every legal scale
    codes = np.arange(256, dtype=np.uint8).reshape(1, 256)
    for e8 in (0, 1, 100, 119, 127, 128, 200, 254):
        scales = np.full((1, 512 // 32), e8, dtype=np.uint8)
        val = oracle.decode_mxfp4(codes, scales)[0]
        for i in range(256):
            lo, hi = i & 0xF, i >> 4
            assert val[2 * i] == _e2m1_bitfield(lo) * 2.0 ** (e8 - 127)
            assert val[2 * i + 1] == _e2m1_bitfield(hi) * 2.0 ** (e8 - 127)
    # the scale is per block of 32 elements along the row
    codes = np.full((2, 32), 0x22, dtype=np.uint8)  # every element = 1.0
    scales = np.array([[127, 126], [120, 130]], dtype=np.uint8)
    v = oracle.decode_mxfp4(codes, scales)
    assert np.all(v[0, :32] == 1.0) and np.all(v[0, 32:] == 0.5)
    assert np.all(v[1, :32] == 2.0 ** -7) and np.all(v[1, 32:] == 8.0)


def test_mxfp4_values_are_exact_in_bf16_and_oracle_agrees_with_dequantised_bf16():
    # every e2m1 value times 2^[-8, 0] is a bf16 value, so the MXFP4 oracle on
    # codes must equal the bf16 oracle on the pre-dequantised weights exactly
    vals = np.array([_e2m1_bitfield(c) * 2.0 ** s for c in range(16) for s in range(-8, 1)], np.float64)
    assert np.array_equal(oracle.decode_bf16(synth.round_to_bf16_bits(vals.astype(np.float32))), vals)
    c = synth.mxfp4_case(T=4, routes="all_local", seed=1, E_local=4, E_global=16, K=2, H=64, F=32,
                         with_weights=False)
    rng = np.random.default_rng(5)
    E, H, F = 4, 64, 32
    w1 = rng.integers(0, 256, size=(E, 2 * F, H // 2), dtype=np.uint8)
    w1s = rng.integers(119, 128, size=(E, 2 * F, H // 32), dtype=np.uint8)
    w2 = rng.integers(0, 256, size=(E, H, F // 2), dtype=np.uint8)
    w2s = rng.integers(119, 128, size=(E, H, F // 32), dtype=np.uint8)
    emap = np.full(16, -1, np.int32)
    emap[4:8] = np.arange(4)
    ids = np.array([[4, 5], [6, 7], [4, 4], [7, 5]], dtype=np.int32)
    counts, offsets, s2r, r2s = oracle.route_compact(ids, emap, E)
    y4 = oracle.grouped_ffn(c.x, "bf16", 2, w1, w2, "mxfp4", counts, offsets, r2s, w1s, w2s)
    w1b = np.stack([synth.round_to_bf16_bits(oracle.decode_mxfp4(w1[e], w1s[e]).astype(np.float32)) for e in range(E)])
    w2b = np.stack([synth.round_to_bf16_bits(oracle.decode_mxfp4(w2[e], w2s[e]).astype(np.float32)) for e in range(E)])
    yb = oracle.grouped_ffn(c.x, "bf16", 2, w1b, w2b, "bf16", counts, offsets, r2s)
    assert np.array_equal(y4, yb)


def test_sampled_rows_match_full_grouped():
    c = synth.tiny_layer(0)
    res = oracle.moe_layer(c)
    rows = np.array([0, 5, 17, 31])
    ys = oracle.grouped_ffn_rows(rows, c.x, "f32", c.K, c.w1, c.w2, "f32", res["offsets"], res["row_to_slot"])
    np.testing.assert_allclose(ys, res["y"][rows], rtol=1e-12, atol=1e-14)


def test_layer_all_remote_is_exact_zero():
    c = synth.mxfp4_case(T=3, routes="uniform", seed=0, E_local=2, E_global=8, K=2, H=64, F=32,
                         with_weights=False)
    c.expert_map = synth.contiguous_expert_map(8, 2, rank=1)
    c.w1 = np.zeros((2, 64, 32), np.uint8)
    c.w1_scale = np.full((2, 64, 2), 127, np.uint8)
    c.w2 = np.zeros((2, 64, 16), np.uint8)
    c.w2_scale = np.full((2, 64, 1), 127, np.uint8)
    c.topk_ids = np.array([[0, 1], [6, 7], [5, 4]], dtype=np.int32)  # all remote
    res = oracle.moe_layer(c)
    assert res["offsets"][-1] == 0
    assert np.all(res["out"] == 0.0)


def test_ffn_rows_closed_form_and_row_independence():
    # H = 2, F = 1: gate row (1, 0), up row (0, 1), W2 = [[2], [-1]]:
    # y = silu(x0) * x1 * (2, -1) for each row, written out by hand
    w1 = np.array([[1.0, 0.0], [0.0, 1.0]])
    w2 = np.array([[2.0], [-1.0]])
    x = np.array([[2.0, 3.0], [0.0, 5.0], [-1.0, -2.0]])
    s = lambda v: v / (1.0 + math.exp(-v))
    want = np.array([[2 * s(2.0) * 3.0, -s(2.0) * 3.0], [0.0, 0.0], [2 * s(-1.0) * -2.0, -s(-1.0) * -2.0]])
    got = oracle.ffn_rows(x, w1, w2)
    assert np.allclose(got, want, rtol=0, atol=1e-15)
    # a row's result does not depend on the other rows
    assert np.array_equal(oracle.ffn_rows(x[1:2], w1, w2)[0], got[1])


def test_decode_weights_selects_the_storage_format():
    # MXFP4: byte 0x21 holds element 0 in its low nibble (code 1 = 0.5) and
    # element 1 in its high nibble (code 2 = 1.0); e8m0 128 scales by 2
    codes = np.zeros((2, 1, 16), dtype=np.uint8)
    codes[1, 0, 0] = 0x21
    scales = np.full((2, 1, 1), 127, dtype=np.uint8)
    scales[1, 0, 0] = 128
    d = oracle.decode_weights(codes, scales, "mxfp4", 1)
    assert d.shape == (1, 32) and d[0, 0] == 1.0 and d[0, 1] == 2.0 and not d[0, 2:].any()
    # bf16 bits 0x3FC0 = 1.5, 0xC000 = -2; f32 passes through
    bits = np.array([[[0x3FC0, 0xC000]]], dtype=np.uint16)
    assert np.array_equal(oracle.decode_weights(bits, None, "bf16", 0), [[1.5, -2.0]])
    f = np.array([[[0.25, -3.0]]], dtype=np.float32)
    assert np.array_equal(oracle.decode_weights(f, None, "f32", 0), [[0.25, -3.0]])


def test_top1_unit_weight_layer_is_a_dense_swiglu_ffn():
    # With K = 1, weight 1 and every expert local, the whole layer reduces to
    # the textbook SwiGLU FFN of each token's expert:
    #   out[t][i] = sum_f W2[e][i][f] * silu(sum_h W1[e][f][h] x[t][h])
    #                                 * (sum_h W1[e][F+f][h] x[t][h])
    # written out here with scalar loops and math.exp, independent of the
    # oracle's matrix formulation.
    rng = np.random.default_rng(11)
    T, E, H, F = 7, 3, 8, 4
    x = rng.standard_normal((T, H)).astype(np.float32)
    w1 = (0.3 * rng.standard_normal((E, 2 * F, H))).astype(np.float32)
    w2 = (0.3 * rng.standard_normal((E, H, F))).astype(np.float32)
    ids = np.array([[0], [2], [1], [2], [2], [0], [1]], dtype=np.int32)
    c = synth.MoECase(name="dense", T=T, E_global=E, E_local=E, K=1, H=H, F=F, renormalize=False,
                      x_dtype="f32", w_dtype="f32", out_dtype="f32", x=x, w1=w1, w2=w2,
                      topk_ids=ids, topk_weights=np.ones((T, 1), np.float32))
    out = oracle.moe_layer(c)["out"]
    for t in range(T):
        e = int(ids[t, 0])
        for i in range(H):
            acc = 0.0
            for f in range(F):
                g = sum(float(w1[e, f, h]) * float(x[t, h]) for h in range(H))
                u = sum(float(w1[e, F + f, h]) * float(x[t, h]) for h in range(H))
                acc += float(w2[e, i, f]) * (g / (1.0 + math.exp(-g))) * u
            assert out[t, i] == pytest.approx(acc, rel=1e-12, abs=1e-14)
