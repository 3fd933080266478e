"""Determinism and buffer bounds of every entry point: each call runs 20 times
eagerly and 3 times from a HIP-graph replay; every run's outputs must be
bitwise identical to the first, and sentinel words placed after each output
buffer (and, for the grouped FFN, the rows past R that are never written)
must be unchanged."""
import numpy as np
import pytest
import torch

import mixture_experts_routing_amd as moe
import synth
from gpu_util import dev_bf16, dev_i32, dev_f32

pytestmark = pytest.mark.gpu

RUNS = 20
PAD = 64  # sentinel elements after each output


def guarded(shape, dtype, fill):
    """A tensor of `shape` that is a view into a buffer with PAD sentinel
    elements after it; returns (view, whole buffer)."""
    n = int(np.prod(shape)) if len(shape) else 1
    whole = torch.full((n + PAD,), fill, dtype=dtype, device="cuda")
    return whole[:n].view(shape), whole


def check_repeats(run, outs, wholes, fills, tag):
    """run() writes `outs`; compare 20 eager runs and 3 graph replays bitwise,
    and the sentinels after each output."""
    print(f"[determinism] {tag}", flush=True)
    run()
    torch.cuda.synchronize()
    first = [o.clone() for o in outs]
    for i in range(RUNS - 1):
        run()
        torch.cuda.synchronize()
        for a, b in zip(first, outs):
            assert torch.equal(a, b), f"{tag}: eager run {i + 1} differs"
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for i in range(3):
        for o in outs:
            o.zero_()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(first, outs):
            assert torch.equal(a, b), f"{tag}: graph replay {i} differs"
    for w, f, o in zip(wholes, fills, outs):
        tail = w[o.numel():]
        assert bool((tail == f).all()), f"{tag}: a sentinel after an output was overwritten"


@pytest.mark.parametrize("scoring", ["softmax", "sigmoid"])
@pytest.mark.parametrize("E", [128, 200])
def test_gate(scoring, E):
    T, K = 3001, 8
    logits = dev_bf16(synth.gate_logits_bf16(T, E, seed=E))
    w, ww = guarded((T, K), torch.float32, -7.0)
    ids, wi = guarded((T, K), torch.int32, -7)
    tei, wt = guarded((T, K), torch.int32, -7)
    fn = moe.moe_topk_softmax if scoring == "softmax" else moe.moe_topk_sigmoid
    check_repeats(lambda: fn(logits, K, True, w, ids, tei), [w, ids, tei], [ww, wi, wt], [-7.0, -7, -7],
                  f"gate {scoring} E={E}")


@pytest.mark.parametrize("T,K,El", [(2, 6, 40), (500, 8, 64), (6000, 8, 128)])
def test_route_compact_and_align(T, K, El):
    # one wave, one block and the multi-block passes
    Eg = 256
    emap = synth.random_expert_map(Eg, El, seed=T)
    ids = dev_i32(np.random.default_rng(T).integers(0, Eg, size=(T, K)))
    emap_d = dev_i32(emap)
    N = T * K
    counts, wc = guarded((El,), torch.int32, -9)
    offsets, wo = guarded((El + 1,), torch.int32, -9)
    s2r, ws = guarded((N,), torch.int32, -9)
    r2s, wr = guarded((N,), torch.int32, -9)
    cws = torch.empty(max(moe.route_compact_workspace_bytes(T, K, El), 16), dtype=torch.uint8, device="cuda")
    check_repeats(lambda: moe.moe_route_compact(ids, emap_d, El, E_global=Eg, out=(counts, offsets, s2r, r2s),
                                                workspace=cws),
                  [counts, offsets, s2r, r2s], [wc, wo, ws, wr], [-9] * 4, f"compact T={T}")
    B = 16
    cap_rows, cap_blocks = N + El * (B - 1), -(-N // B) + El
    poff, wp = guarded((El + 1,), torch.int32, -9)
    srt, wsr = guarded((cap_rows,), torch.int32, -9)
    bex, wb = guarded((cap_blocks,), torch.int32, -9)
    ps2r, wps = guarded((N,), torch.int32, -9)
    aws = torch.empty(max(moe.route_align_workspace_bytes(T, K, El), 16), dtype=torch.uint8, device="cuda")
    check_repeats(lambda: moe.moe_route_align(ids, emap_d, El, B, E_global=Eg, out=(poff, srt, bex, ps2r),
                                              workspace=aws),
                  [poff, srt, bex, ps2r], [wp, wsr, wb, wps], [-9] * 4, f"align T={T}")


def test_topk_compact():
    T, E, K = 4096, 128, 8
    logits = dev_bf16(synth.gate_logits_bf16(T, E, seed=5))
    N = T * K
    w, ww = guarded((T, K), torch.float32, -7.0)
    ids, wi = guarded((T, K), torch.int32, -7)
    tei, wt = guarded((T, K), torch.int32, -7)
    routes = [guarded(s, torch.int32, -9) for s in ((E,), (E + 1,), (N,), (N,))]
    outs = [w, ids, tei] + [r[0] for r in routes]
    cws = torch.empty(moe.route_compact_workspace_bytes(T, K, E), dtype=torch.uint8, device="cuda")
    check_repeats(lambda: moe.moe_topk_compact(logits, K, True, gate_out=(w, ids, tei),
                                               route_out=tuple(r[0] for r in routes), workspace=cws),
                  outs, [ww, wi, wt] + [r[1] for r in routes], [-7.0, -7, -7] + [-9] * 4, "topk_compact")


def ffn_case(T, K, El, H, F, seed):
    rng = np.random.default_rng(seed)
    ids = np.stack([rng.choice(El, size=K, replace=False) for _ in range(T)]).astype(np.int32)
    x = dev_bf16(synth.bf16_normal((T, H), 1.0, seed, 1))
    w1 = dev_bf16(synth.bf16_normal((El, 2 * F, H), 0.05, seed, 2))
    w2 = dev_bf16(synth.bf16_normal((El, H, F), 0.05, seed, 3))
    tw = dev_f32(rng.dirichlet(np.ones(K), size=T).astype(np.float32))
    counts, offsets, s2r, r2s = moe.moe_route_compact(dev_i32(ids), None, El)
    return x, w1, w2, tw, counts, offsets, s2r, r2s, dev_i32(ids)


@pytest.mark.parametrize("name,T,K,El,H,F", [("decode", 2, 6, 16, 1024, 512), ("mid", 96, 4, 8, 512, 256),
                                             ("prefill", 1024, 8, 16, 512, 256)])
def test_grouped_ffn_and_combine(name, T, K, El, H, F):
    x, w1, w2, tw, counts, offsets, s2r, r2s, ids = ffn_case(T, K, El, H, F, seed=T)
    N = T * K
    R = int(offsets[-1].item())
    sentinel = -12345
    y_whole = torch.full((N * H + PAD,), sentinel, dtype=torch.int16, device="cuda")
    y = y_whole[:N * H].view(torch.bfloat16).view(N, H)
    ws = torch.empty(moe.grouped_ffn_workspace_bytes(T, K, H, F, El, moe.MOE_BF16), dtype=torch.uint8,
                     device="cuda")

    def run():
        moe.moe_grouped_ffn(x, K, w1, w2, counts, offsets, r2s, y=y, workspace=ws)

    check_repeats(run, [y[:R]], [y_whole], [sentinel], f"grouped_ffn {name}")
    # rows past R are never written
    assert bool((y_whole[R * H:N * H] == sentinel).all())
    out, wo = guarded((T, H), torch.float32, -3.0)
    check_repeats(lambda: moe.moe_combine(y, tw, s2r, out=out), [out], [wo], [-3.0], f"combine {name}")
    if name == "prefill":
        t1, t2 = moe.moe_pack_ffn_weights(w1, w2)
        check_repeats(lambda: moe.moe_grouped_ffn(x, K, t1, t2, counts, offsets, r2s, y=y, workspace=ws,
                                                  tiled=True),
                      [y[:R]], [y_whole], [sentinel], "grouped_ffn packed")
    if name == "decode":
        cws = torch.empty(moe.grouped_ffn_control_workspace_bytes(T, K, H, F, El, moe.MOE_BF16),
                          dtype=torch.uint8, device="cuda")
        check_repeats(lambda: moe.moe_grouped_ffn_control(x, K, w1, w2, counts, offsets, r2s, y=y, workspace=cws),
                      [y[:R]], [y_whole], [sentinel], "grouped_ffn control")
        fout, wf = guarded((T, H), torch.bfloat16, 0.5)
        routes = [guarded(s, torch.int32, -9) for s in ((El,), (El + 1,), (N,), (N,))]
        fws = torch.empty(moe.fused_experts_workspace_bytes(T, K, H, F, El, moe.MOE_BF16), dtype=torch.uint8,
                          device="cuda")
        check_repeats(lambda: moe.moe_fused_experts(x, ids, tw, w1, w2, out=fout,
                                                    routes=tuple(r[0] for r in routes), workspace=fws),
                      [fout] + [r[0] for r in routes], [wf] + [r[1] for r in routes], [0.5] + [-9] * 4,
                      "fused_experts")
