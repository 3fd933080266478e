"""The seeded generators: determinism, bf16 rounding, workload shapes (CPU)."""
import numpy as np
import torch

import synth


def test_bf16_rounding_is_round_to_nearest_even():
    rng = np.random.default_rng(0)
    a = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10,
                        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 0.0, -0.0], np.float32)])
    ours = synth.round_to_bf16_bits(a)
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_generators_are_deterministic_and_subset_stable():
    a = synth.bf16_normal((3, 5), 2.0, 0, 1)
    b = synth.bf16_normal((3, 5), 2.0, 0, 1)
    assert np.array_equal(a, b)
    c1 = synth.decode_case("cross_row", "random", seed=3, with_weights=False)
    c2 = synth.decode_case("cross_row", "random", seed=3, with_weights=False)
    assert np.array_equal(c1.topk_ids, c2.topk_ids) and np.array_equal(c1.expert_map, c2.expert_map)


def test_decode_patterns_use_the_map():
    for kind in ("contiguous", "random"):
        for p in synth.DECODE_PATTERNS:
            c = synth.decode_case(p, kind, seed=1, with_weights=False)
            loc = c.expert_map[c.topk_ids]
            exp = np.array([[-1 if l is None else l for l in row] for row in synth.DECODE_PATTERNS[p]])
            assert np.array_equal(loc, exp)
            np.testing.assert_allclose(c.topk_weights.sum(axis=1), 1.0, rtol=1e-6)


def test_mxfp4_case_shapes_and_scale_range():
    c = synth.mxfp4_case(16, "uniform", seed=0, E_local=4, H=256, F=128)
    assert c.w1.shape == (4, 256, 128) and c.w1_scale.shape == (4, 256, 8)
    assert c.w2.shape == (4, 256, 64) and c.w2_scale.shape == (4, 256, 4)
    assert c.w1_scale.min() >= 119 and c.w1_scale.max() <= 127
    for t in range(16):
        assert len(set(c.topk_ids[t].tolist())) == 8


def test_gate_case_has_boundary_ties():
    # half of the ~1% injected rows tie exactly at the K-th place: the value
    # ranked K-th equals the value ranked (K+1)-th
    T, E, K = 65536, 128, 8
    c = synth.gate_case(E, T=T, K=K, seed=0)
    f = (c.logits.astype(np.uint32) << np.uint32(16)).view(np.float32)
    srt = -np.sort(-f, axis=1)
    boundary = int(np.count_nonzero(srt[:, K - 1] == srt[:, K]))
    injected = int(round(T * 0.01))
    assert boundary >= injected // 2
    top = int(np.count_nonzero(srt[:, 0] == srt[:, 1]))
    assert top >= injected // 2
