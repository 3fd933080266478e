"""moe_topk_compact: the gate and the route compaction in one call, with the
compaction's count pass inside the gate kernel for bf16 logits, K = 8 and
more than 4096 slots.  Every output must equal, bit for bit, what the two
separate calls produce (moe_topk_softmax / moe_topk_sigmoid, then
moe_route_compact), and the ids and compaction arrays must equal the
oracle's (weights within 1e-6 relative)."""
import numpy as np
import pytest
import torch

import mixture_experts_routing_amd as moe
import oracle
import synth
from gpu_util import dev_any, dev_i32, host_i

pytestmark = pytest.mark.gpu

W_RTOL = 1e-6


def check(logits_host, dtype, K, renorm, scoring, emap=None, E_local=None, tag=""):
    T, E = logits_host.shape
    E_local = E if E_local is None else E_local
    print(f"[gate+compact] {tag} {scoring} T={T} E={E} K={K} renorm={renorm} dtype={dtype} E_local={E_local}",
          flush=True)
    logits = dev_any(logits_host, dtype)
    emap_d = dev_i32(emap) if emap is not None else None
    (w, ids, tei), routes = moe.moe_topk_compact(logits, K, renorm, scoring, emap_d, E_local)
    torch.cuda.synchronize()
    # the two separate calls
    gate = moe.moe_topk_softmax if scoring == "softmax" else moe.moe_topk_sigmoid
    w2, ids2, tei2 = gate(logits, K, renorm)
    routes2 = moe.moe_route_compact(ids2, emap_d, E_local, E_global=E)
    torch.cuda.synchronize()
    assert torch.equal(ids, ids2) and torch.equal(tei, tei2) and torch.equal(w, w2)
    for name, a, b in zip(("counts", "offsets", "slot_to_row", "row_to_slot"), routes, routes2):
        assert torch.equal(a, b), name
    # the oracle
    ref = oracle.topk_softmax if scoring == "softmax" else oracle.topk_sigmoid
    w_ref, ids_ref, _ = ref(logits_host, K, renorm, dtype)
    assert np.array_equal(host_i(ids), ids_ref)
    wr = w.cpu().numpy().astype(np.float64)
    err = np.maximum(np.abs(wr - w_ref) - 2.0 ** -126, 0.0) / np.abs(w_ref)
    assert err.max() <= W_RTOL
    c_ref = oracle.route_compact(ids_ref, emap, E_local)
    for name, got, want in zip(("counts", "offsets", "slot_to_row", "row_to_slot"), routes, c_ref):
        assert np.array_equal(host_i(got), want), name


@pytest.mark.parametrize("scoring", ["softmax", "sigmoid"])
def test_prefill_shape(scoring):
    # T=4096, E=128 all local, top-8 renormalised: 32 count blocks, fused path
    check(synth.gate_logits_bf16(4096, 128, seed=21), "bf16", 8, True, scoring, tag="prefill")


@pytest.mark.parametrize("E", [64, 96, 160, 192])
def test_ragged_rows_expert_map(E):
    # 1000 rows: the last block holds 104 of its 128 rows; one rank of a
    # 4-way expert-parallel split with a random map
    El = E // 4
    emap = synth.random_expert_map(E, El, seed=E)
    check(synth.gate_logits_bf16(1000, E, seed=E + 1), "bf16", 8, False, "softmax", emap, El, tag="ragged")


def test_many_count_blocks():
    # 8320 rows = 66560 slots = 65 count blocks: the scan runs as its own pass
    check(synth.gate_logits_bf16(8320, 64, seed=23), "bf16", 8, True, "sigmoid", tag="65 blocks")


@pytest.mark.parametrize("T,E,K,dtype", [(1000, 128, 6, "bf16"), (300, 128, 8, "bf16"), (1000, 160, 8, "f32"),
                                         (700, 200, 8, "bf16")])
def test_unfused_shapes(T, E, K, dtype):
    # K != 8, at most 4096 slots, fp32 logits, E outside the fast set: the
    # gate and the compaction run one after the other
    rng = np.random.default_rng(T + E + K)
    logits = synth.gate_logits_bf16(T, E, seed=T + K) if dtype == "bf16" else \
        rng.standard_normal((T, E)).astype(np.float32)
    check(logits, dtype, K, True, "softmax", tag="unfused")


def test_empty_batch():
    dev = torch.device("cuda")
    logits = torch.empty((0, 128), dtype=torch.bfloat16, device=dev)
    route_out = (torch.full((128,), 9, dtype=torch.int32, device=dev),
                 torch.full((129,), 9, dtype=torch.int32, device=dev),
                 torch.empty(0, dtype=torch.int32, device=dev), torch.empty(0, dtype=torch.int32, device=dev))
    _, routes = moe.moe_topk_compact(logits, 8, True, route_out=route_out)
    torch.cuda.synchronize()
    assert not routes[0].any() and not routes[1].any()
