"""Boundary fusion for decode batches (moe_fused_experts): compaction inside
the first FFN kernel, combine inside the second.  Checked against the oracle
(compaction bit-exact, out within the FFN bound) and against the three
separate calls it replaces, on every decode route pattern, MXFP4, ragged and
maximal shapes, empty batches, repeat runs and HIP-graph replays."""
import dataclasses

import numpy as np
import pytest
import torch

import mixture_experts_routing_amd as moe
import oracle
import synth
from gpu_util import case_to_device, dev_bf16, host_f64, host_i, rel_max_err

pytestmark = pytest.mark.gpu

TOL = {"bf16": 1e-2, "mxfp4": 3e-2}


def run_fused(c, d, out_dtype=None):
    out, routes = moe.moe_fused_experts(d["x"], d["topk_ids"], d["topk_weights"], d["w1"], d["w2"],
                                        d["expert_map"], c.E_global, d["w1_scale"], d["w2_scale"],
                                        out_dtype=out_dtype)
    torch.cuda.synchronize()
    return out, routes


def run_separate(c, d, out_dtype=None):
    counts, offsets, s2r, r2s = moe.moe_route_compact(d["topk_ids"], d["expert_map"], c.E_local, E_global=c.E_global)
    y = moe.moe_grouped_ffn(d["x"], c.K, d["w1"], d["w2"], counts, offsets, r2s, d["w1_scale"], d["w2_scale"],
                            y_dtype=torch.bfloat16)
    out = moe.moe_combine(y, d["topk_weights"], s2r, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return out, (counts, offsets, s2r, r2s)


def check(c, d, tag, out_dtype=None, bit_equal_separate=False):
    print(f"[fused] {tag} {c.name} T={c.T} K={c.K} E_local={c.E_local} H={c.H} F={c.F}", flush=True)
    ref = oracle.moe_layer(c)
    out, routes = run_fused(c, d, out_dtype)
    for name, got in zip(("counts", "offsets", "slot_to_row", "row_to_slot"), routes):
        assert np.array_equal(host_i(got), ref[name]), name
    err = rel_max_err(host_f64(out), ref["out"])
    print(f"[fused] {tag}: out err {err:.3e}", flush=True)
    assert err <= TOL[c.w_dtype]
    sep, sep_routes = run_separate(c, d, out_dtype)
    for a, b in zip(routes, sep_routes):
        assert torch.equal(a, b)
    if bit_equal_separate:
        assert torch.equal(out, sep)
    else:
        assert rel_max_err(host_f64(out), host_f64(sep)) <= TOL[c.w_dtype]
    out2, _ = run_fused(c, d, out_dtype)
    assert torch.equal(out2, out), "repeat run differs"
    return out


@pytest.fixture(scope="module")
def decode_weights():
    w1, w2 = synth.decode_weights(0)
    return w1, w2, dev_bf16(w1), dev_bf16(w2)


def decode_case(pattern, map_kind, seed, weights):
    """The decode case with the module's shared weights, on host and device."""
    c = synth.decode_case(pattern, map_kind, seed=seed, with_weights=False)
    d = case_to_device(c)
    d["w1"], d["w2"] = weights[2], weights[3]
    d["w1_scale"] = d["w2_scale"] = None
    return dataclasses.replace(c, w1=weights[0], w2=weights[1]), d


@pytest.mark.parametrize("map_kind", ["contiguous", "random"])
@pytest.mark.parametrize("pattern", synth.decode_patterns())
def test_fused_decode_patterns(pattern, map_kind, decode_weights):
    c, d = decode_case(pattern, map_kind, 5, decode_weights)
    # all-duplicate: every local row is in one 16-row tile, so the second
    # GEMM splits its reduction exactly as the separate FFN does
    out = check(c, d, "decode", bit_equal_separate=pattern in ("all_dup", "all_remote"))
    if pattern == "all_remote":
        assert not out.float().abs().any()


@pytest.mark.parametrize("T,routes", [(2, "uniform"), (2, "all_local"), (8, "all_local")])
def test_fused_mxfp4(T, routes):
    c = synth.mxfp4_case(T, routes, seed=6)
    check(c, case_to_device(c), "mxfp4")


@pytest.mark.parametrize("H,F", [(256, 160), (256, 2080), (4128, 64)])
def test_fused_mxfp4_uneven_units(H, F):
    # MXFP4 GEMM2 operands in the batched layout with partial batches (5 K
    # units over 16 waves: one each, the rest none), the unpipelined GEMM2
    # (65 units: more than 4 per wave), and GEMM1 rows longer than the LDS
    # staging holds (H = 4128)
    T, K, Eg, El = 5, 4, 16, 6
    rng = np.random.default_rng(H + F)
    emap = synth.random_expert_map(Eg, El, seed=H + F)
    ids = np.stack([rng.choice(Eg, size=K, replace=False) for _ in range(T)]).astype(np.int32)
    w = rng.dirichlet(np.ones(K), size=T).astype(np.float32)
    c = synth.MoECase(name=f"mx_uneven_{H}_{F}", T=T, E_global=Eg, E_local=El, K=K, H=H, F=F, renormalize=False,
                      x_dtype="bf16", w_dtype="mxfp4", out_dtype="bf16", x=synth.bf16_normal((T, H), 1.0, 9, 1),
                      w1=rng.integers(0, 256, size=(El, 2 * F, H // 2), dtype=np.uint8),
                      w2=rng.integers(0, 256, size=(El, H, F // 2), dtype=np.uint8),
                      w1_scale=rng.integers(119, 128, size=(El, 2 * F, H // 32), dtype=np.uint8),
                      w2_scale=rng.integers(119, 128, size=(El, H, F // 32), dtype=np.uint8),
                      topk_ids=ids, topk_weights=w, expert_map=emap)
    check(c, case_to_device(c), "mxfp4 uneven")


def small_case(name, T, K, Eg, El, H, F, ids, seed, emap=None):
    rng = np.random.default_rng([seed, 77])
    w = rng.dirichlet(np.ones(K), size=T).astype(np.float32)
    return synth.MoECase(name=name, T=T, E_global=Eg, E_local=El, K=K, H=H, F=F, renormalize=False,
                         x_dtype="bf16", w_dtype="bf16", out_dtype="bf16",
                         x=synth.bf16_normal((T, H), 1.0, seed, 1),
                         w1=synth.bf16_normal((El, 2 * F, H), 0.05, seed, 2),
                         w2=synth.bf16_normal((El, H, F), 0.05, seed, 3),
                         topk_ids=np.asarray(ids, np.int32), topk_weights=w, expert_map=emap)


def test_fused_max_slots_and_experts():
    # 64 slots (one full wave) over 64 local experts of 128, random map
    T, K, Eg, El = 8, 8, 128, 64
    emap = synth.random_expert_map(Eg, El, 11)
    ids = np.random.default_rng([11, 1]).integers(0, Eg, size=(T, K))
    c = small_case("max_slots", T, K, Eg, El, 256, 128, ids, 11, emap)
    d = case_to_device(c)
    check(c, d, "max")
    check(c, d, "max_f32out", out_dtype=torch.float32)


def test_fused_ragged_tiles_and_duplicates():
    # one expert with more than 16 rows (a ragged last tile) plus duplicates
    # within rows and a remote route
    T, K, Eg, El = 17, 2, 8, 4
    emap = np.array([0, 1, 2, 3, -1, -1, -1, -1], np.int32)
    ids = np.zeros((T, K), np.int32)
    ids[:, 0] = 2
    ids[:, 1] = np.arange(T) % 3
    ids[5, 1] = 2          # duplicate of the row's first route
    ids[7, 1] = 6          # remote
    c = small_case("ragged", T, K, Eg, El, 128, 64, ids, 12, emap)
    check(c, case_to_device(c), "ragged")


def test_fused_single_slot():
    c = small_case("single", 1, 1, 8, 8, 64, 32, [[5]], 13)
    check(c, case_to_device(c), "single")


def test_fused_empty_batch():
    dev = torch.device("cuda")
    x = torch.empty((0, 4096), dtype=torch.bfloat16, device=dev)
    ids = torch.empty((0, 6), dtype=torch.int32, device=dev)
    w = torch.empty((0, 6), dtype=torch.float32, device=dev)
    w1 = torch.zeros((4, 2 * 64, 4096), dtype=torch.bfloat16, device=dev)
    w2 = torch.zeros((4, 4096, 64), dtype=torch.bfloat16, device=dev)
    emap = torch.full((16,), -1, dtype=torch.int32, device=dev)
    emap[:4] = torch.arange(4, dtype=torch.int32, device=dev)
    routes = (torch.full((4,), 7, dtype=torch.int32, device=dev), torch.full((5,), 7, dtype=torch.int32, device=dev),
              torch.empty(0, dtype=torch.int32, device=dev), torch.empty(0, dtype=torch.int32, device=dev))
    out, routes = moe.moe_fused_experts(x, ids, w, w1, w2, emap, 16, routes=routes)
    torch.cuda.synchronize()
    assert out.shape == (0, 4096)
    assert not routes[0].any() and not routes[1].any()


def test_fused_rejects_large_batches(decode_weights):
    c, d = decode_case("disjoint", "contiguous", 0, decode_weights)
    w1, w2 = d["w1"], d["w2"]
    ids = d["topk_ids"].repeat(6, 1)  # 12 tokens x 6 = 72 slots
    x = d["x"].repeat(6, 1)
    w = d["topk_weights"].repeat(6, 1)
    with pytest.raises(moe.MoeError):
        moe.moe_fused_experts(x, ids, w, w1, w2, d["expert_map"], c.E_global)


def test_fused_graph_replays(decode_weights):
    c, d = decode_case("twelve_local", "random", 7, decode_weights)
    w1, w2 = d["w1"], d["w2"]
    ref_counts = oracle.moe_layer(c)["counts"]
    eager, _ = moe.moe_fused_experts(d["x"], d["topk_ids"], d["topk_weights"], w1, w2, d["expert_map"], c.E_global)
    eager = eager.clone()
    out = torch.empty_like(eager)
    routes = tuple(torch.empty_like(t) for t in moe.moe_route_compact(d["topk_ids"], d["expert_map"], c.E_local,
                                                                       E_global=c.E_global))
    ws = torch.empty(moe.fused_experts_workspace_bytes(c.T, c.K, c.H, c.F, c.E_local, moe.MOE_BF16),
                     dtype=torch.uint8, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        moe.moe_fused_experts(d["x"], d["topk_ids"], d["topk_weights"], w1, w2, d["expert_map"], c.E_global,
                              out=out, routes=routes, workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        moe.moe_fused_experts(d["x"], d["topk_ids"], d["topk_weights"], w1, w2, d["expert_map"], c.E_global,
                              out=out, routes=routes, workspace=ws)
    for i in range(3):
        out.zero_()
        routes[0].fill_(-5)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {i}"
        assert np.array_equal(host_i(routes[0]), ref_counts), f"replay {i}"
        _ = (torch.ones(1024, device="cuda") * 2).sum().item()  # eager work between replays
