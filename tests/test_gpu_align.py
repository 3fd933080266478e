"""GPU parity of moe_route_align (block-aligned layout) against the oracle:
every output bit for bit."""
import numpy as np
import pytest
import torch

import mixture_experts_routing_amd as moe
import oracle
import synth
from gpu_util import DEV, dev_i32, host_i

pytestmark = pytest.mark.gpu


def check_align(ids, emap, El, Eg, bs, tag=""):
    print(f"[align] {tag} N={ids.size} E_local={El} block={bs}", flush=True)
    ref = oracle.route_align(ids, emap, El, bs)
    got = moe.moe_route_align(dev_i32(ids), None if emap is None else dev_i32(emap), El, bs, E_global=Eg)
    torch.cuda.synchronize()
    for name, g, r in zip(("padded_offsets", "sorted_slots", "block_expert", "slot_to_row"), got, ref):
        g = host_i(g)
        assert g.shape == r.shape, name
        bad = np.flatnonzero(g != r)
        assert bad.size == 0, f"{name}: {bad.size} differ, first at {bad[:3]}: got {g[bad[:3]]} want {r[bad[:3]]}"


@pytest.mark.parametrize("pattern", synth.decode_patterns())
@pytest.mark.parametrize("bs", [1, 8, 16])
def test_decode_patterns(pattern, bs):
    for map_kind in ("contiguous", "random"):
        for seed in range(3):
            c = synth.decode_case(pattern, map_kind, seed=seed, with_weights=False)
            check_align(c.topk_ids, c.expert_map, c.E_local, c.E_global, bs, f"{pattern}/{map_kind}/{seed}")


@pytest.mark.parametrize("T,K,Eg,El,bs", [
    (4096, 8, 128, 128, 64), (4096, 8, 128, 128, 256), (513, 8, 128, 128, 128), (3000, 8, 1024, 768, 16),
    (1000, 6, 256, 1, 32), (8, 8, 64, 64, 4096), (65536, 8, 160, 160, 128),
])
def test_random_routes(T, K, Eg, El, bs):
    rng = np.random.default_rng(T + El + bs)
    ids = rng.integers(0, Eg, size=(T, K)).astype(np.int32)
    emap = None if El == Eg else synth.random_expert_map(Eg, El, seed=T)
    check_align(ids, emap, El, Eg, bs, "random")


def test_all_remote_and_skewed():
    emap = synth.contiguous_expert_map(256, 32)
    remote = np.flatnonzero(emap < 0)
    rng = np.random.default_rng(3)
    check_align(remote[rng.integers(0, remote.size, size=(512, 8))].astype(np.int32), emap, 32, 256, 64, "remote")
    check_align(np.full((700, 8), 40, np.int32), emap, 32, 256, 128, "one-hot")


def test_empty_batch():
    emap = dev_i32(synth.contiguous_expert_map(256, 40))
    poff, ss, be, s2r = moe.moe_route_align(torch.empty((0, 6), dtype=torch.int32, device=DEV), emap, 40, 16,
                                            E_global=256)
    torch.cuda.synchronize()
    assert host_i(poff).tolist() == [0] * 41
    assert np.all(host_i(ss) == -1) and np.all(host_i(be) == -1)
