"""The C ABI library loads, exports every symbol the public header declares,
and rejects bad arguments on the host before touching the GPU (CPU only: no
call here launches a kernel)."""
import ctypes

import pytest
import torch

from mixture_experts_routing_amd import _lib


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def test_every_header_symbol_is_exported(lib):
    names = _lib.header_symbols()
    assert set(names) == set(_lib.SIGNATURES), "binding signatures must cover the header exactly"
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    assert _lib.status_string(0) == "MOE_OK"
    assert _lib.status_string(1) == "MOE_ERR_INVALID_ARG"
    assert _lib.status_string(4) == "MOE_ERR_WORKSPACE"
    assert _lib.status_string(5) == "MOE_ERR_SCRATCH_LIMIT"
    assert lib.moe_version().decode().startswith("moe_routing")


NULL = None
FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails validation first

# The validation tests pass fake device pointers that host checks must
# reject; keep them off machines with a GPU so that a mistake in a test can
# never reach a kernel launch.
_no_gpu = pytest.mark.skipif(torch.cuda.device_count() > 0, reason="fake-pointer validation runs only without a GPU")


@_no_gpu
def test_topk_softmax_validation(lib):
    f = lib.moe_topk_softmax
    assert f(NULL, 1, 0, 8, 2, 0, NULL, NULL, NULL, NULL) == 0            # T == 0: no-op
    assert f(FAKE, 1, 4, 8, 9, 0, FAKE, FAKE, NULL, NULL) == 1            # K > E
    assert f(FAKE, 1, 4, 8, 0, 0, FAKE, FAKE, NULL, NULL) == 1            # K == 0
    assert f(FAKE, 1, -1, 8, 2, 0, FAKE, FAKE, NULL, NULL) == 1           # T < 0
    assert f(FAKE, 7, 4, 8, 2, 0, FAKE, FAKE, NULL, NULL) == 2            # bad dtype
    assert f(FAKE, 1, 4, 2048, 2, 0, FAKE, FAKE, NULL, NULL) == 2         # E too large
    assert f(FAKE, 1, 4, 64, 33, 0, FAKE, FAKE, NULL, NULL) == 2          # K too large
    assert f(NULL, 1, 4, 8, 2, 0, FAKE, FAKE, NULL, NULL) == 1            # null logits


@_no_gpu
def test_route_compact_validation(lib):
    f = lib.moe_route_compact
    assert f(FAKE, 2, 6, NULL, 256, 40, FAKE, FAKE, FAKE, FAKE, NULL, 0, NULL) == 1   # no map, E_l != E_g
    assert f(FAKE, 2, 6, FAKE, 32, 40, FAKE, FAKE, FAKE, FAKE, NULL, 0, NULL) == 1    # E_l > E_g
    assert f(FAKE, 2, 6, FAKE, 4096, 1000, FAKE, FAKE, FAKE, FAKE, NULL, 0, NULL) == 2  # E_l > 768
    assert f(FAKE, 2, 6, FAKE, 256, 40, NULL, FAKE, FAKE, FAKE, NULL, 0, NULL) == 1   # null counts
    need = lib.moe_route_compact_workspace_bytes(65536, 8, 128)
    assert need > 0
    assert lib.moe_route_compact_workspace_bytes(2, 6, 40) == 0
    assert f(FAKE, 65536, 8, NULL, 128, 128, FAKE, FAKE, FAKE, FAKE, NULL, 0, NULL) == 4          # workspace
    assert f(FAKE, 65536, 8, NULL, 128, 128, FAKE, FAKE, FAKE, FAKE, FAKE, need - 1, NULL) == 4


@_no_gpu
def test_grouped_ffn_validation(lib):
    f = lib.moe_grouped_ffn
    def args(xdt, wdt, H, F, ws=FAKE, wsb=1 << 40, ydt=1, sc=NULL):
        return (FAKE, xdt, 2, 6, H, F, 40, FAKE, sc, FAKE, sc, wdt, FAKE, FAKE, FAKE, FAKE, ydt, ws, wsb, NULL)

    assert f(*args(0, 1, 4096, 2048)) == 2        # f32 x with bf16 weights
    assert f(*args(1, 0, 4096, 2048)) == 2        # bf16 x with f32 weights
    assert f(*args(1, 1, 4001, 2048)) == 2        # H not a multiple of 32
    assert f(*args(1, 1, 4096, 2048, ydt=2)) == 2  # y as MXFP4
    assert f(*args(1, 2, 4096, 2048)) == 1        # MXFP4 codes without scales
    assert f(*args(1, 1, 4096, 2048, ws=NULL)) == 4
    need = lib.moe_grouped_ffn_workspace_bytes(2, 6, 4096, 2048, 40, 1)
    assert need == 2 * 6 * 2048 * 2  # the bf16 act rows
    assert lib.moe_grouped_ffn_workspace_bytes(4096, 8, 2048, 768, 128, 1) == 4096 * 8 * 768 * 2
    assert f(*args(1, 1, 4096, 2048, wsb=need - 1)) == 4
    mis = ctypes.c_void_p(0x1002)  # bf16 operands must be 16-byte aligned
    a = list(args(1, 1, 4096, 2048))
    a[0] = mis
    assert f(*a) == 1


@_no_gpu
def test_grouped_ffn_noalloc_validation(lib):
    # same checks as moe_grouped_ffn (no workspace), plus the fixed 64 MiB
    # scratch: a call whose act rows exceed it is refused before any HIP call
    f = lib.moe_grouped_ffn_noalloc
    def args(T, xdt, wdt, H, F, ydt=1, sc=NULL, E=40):
        return (FAKE, xdt, T, 6, H, F, E, FAKE, sc, FAKE, sc, wdt, FAKE, FAKE, FAKE, FAKE, ydt, NULL)

    assert f(*args(0, 1, 1, 4096, 2048)) == 0          # T == 0: no-op
    assert f(*args(2, 0, 1, 4096, 2048)) == 2          # f32 x with bf16 weights
    assert f(*args(2, 1, 2, 4096, 2048)) == 1          # MXFP4 codes without scales
    limit = 64 << 20
    T_fit = limit // (6 * 2048 * 2)                     # act rows exactly fill the scratch
    assert lib.moe_grouped_ffn_workspace_bytes(T_fit, 6, 4096, 2048, 40, 1) <= limit
    assert lib.moe_grouped_ffn_workspace_bytes(T_fit + 1, 6, 4096, 2048, 40, 1) > limit
    assert f(*args(T_fit + 1, 1, 1, 4096, 2048)) == 5   # MOE_ERR_SCRATCH_LIMIT
    assert f(*args(12288, 1, 3, 2048, 768, E=128)) == 5  # three prefill batches of act rows
    mis = ctypes.c_void_p(0x1002)
    a = list(args(2, 1, 1, 4096, 2048))
    a[0] = mis
    assert f(*a) == 1


@_no_gpu
def test_combine_validation(lib):
    f = lib.moe_combine
    assert f(FAKE, 1, FAKE, FAKE, 0, 6, 4096, FAKE, 1, NULL) == 0   # T == 0
    assert f(FAKE, 2, FAKE, FAKE, 2, 6, 4096, FAKE, 1, NULL) == 2   # y dtype
    assert f(FAKE, 1, NULL, FAKE, 2, 6, 4096, FAKE, 1, NULL) == 1   # null weights
    assert f(FAKE, 1, FAKE, FAKE, 2, 0, 4096, FAKE, 1, NULL) == 1   # K == 0


@_no_gpu
def test_fused_experts_validation(lib):
    f = lib.moe_fused_experts
    def args(T=2, K=6, H=4096, F=2048, El=40, Eg=256, emap=FAKE, xdt=1, wdt=1, odt=1, sc=NULL, ws=FAKE,
             wsb=1 << 40, counts=FAKE, x=FAKE):
        return (x, xdt, T, K, H, F, FAKE, FAKE, emap, Eg, El, FAKE, sc, FAKE, sc, wdt, counts, FAKE, FAKE, FAKE,
                FAKE, odt, ws, wsb, NULL)

    assert f(*args(T=9, K=8)) == 2              # 72 slots: more than one wave's worth
    assert f(*args(El=65, Eg=256)) == 2         # more than 64 local experts
    assert f(*args(H=4008)) == 2                # H not a multiple of 32
    assert f(*args(F=2040)) == 2                # F not a multiple of 32
    assert f(*args(xdt=0, wdt=0)) == 2          # fp32 pair: not on this path
    assert f(*args(wdt=3)) == 2                 # tile-packed weights: not on this path
    assert f(*args(odt=2)) == 2                 # out as MXFP4
    assert f(*args(wdt=2)) == 1                 # MXFP4 codes without scales
    assert f(*args(emap=NULL)) == 1             # no map while E_local != E_global
    assert f(*args(El=40, Eg=32)) == 1          # E_local > E_global
    assert f(*args(counts=NULL)) == 1           # null counts
    assert f(*args(ws=NULL)) == 4
    need = lib.moe_fused_experts_workspace_bytes(2, 6, 4096, 2048, 40, 1)
    assert need == 2 * 6 * 2048 * 2             # the bf16 act rows
    assert f(*args(wsb=need - 1)) == 4
    assert f(*args(x=ctypes.c_void_p(0x1002))) == 1  # x must be 16-byte aligned


@_no_gpu
def test_topk_compact_validation(lib):
    f = lib.moe_topk_compact
    def args(T=4096, E=128, K=8, scoring=0, emap=NULL, El=128, ws=FAKE, wsb=1 << 40, counts=FAKE, s2r=FAKE):
        return (FAKE, 1, T, E, K, 1, scoring, FAKE, FAKE, NULL, emap, El, counts, FAKE, s2r, FAKE, ws, wsb, NULL)

    assert f(*args(scoring=2)) == 2             # unknown scoring
    assert f(*args(K=9, E=8)) == 1              # K > E
    assert f(*args(El=40)) == 1                 # no map while E_local != E
    assert f(*args(El=200, emap=FAKE)) == 1     # E_local > E
    assert f(*args(E=1000, El=800, emap=FAKE)) == 2  # E_local > 768
    assert f(*args(counts=NULL)) == 1
    assert f(*args(s2r=NULL)) == 1
    assert f(*args(ws=NULL)) == 4               # 32768 slots need the count table
    need = lib.moe_route_compact_workspace_bytes(4096, 8, 128)
    assert f(*args(wsb=need - 1)) == 4


def test_binding_checks_dtypes_shapes_and_sizes():
    # The binding refuses tensors whose dtype, shape or size differs from what
    # the C call reads or writes, before any pointer reaches the library (CPU
    # tensors: the checks run before the device check).
    import mixture_experts_routing_amd as moe

    i32, i64, f32, bf16, u8 = torch.int32, torch.int64, torch.float32, torch.bfloat16, torch.uint8
    z = lambda shape, dt: torch.zeros(shape, dtype=dt)
    with pytest.raises(moe.MoeError, match="dtype"):
        moe.moe_topk_softmax(z((4, 8), i64), 2)                       # integer logits
    with pytest.raises(moe.MoeError, match="elements"):
        moe.moe_topk_softmax(z((4, 8), bf16), 2, topk_ids=z(7, i32))  # ids buffer too short
    with pytest.raises(moe.MoeError, match="dtype"):
        moe.moe_route_compact(z((2, 6), i64), None, 8)                # int64 ids (torch.topk's)
    with pytest.raises(moe.MoeError, match="elements"):
        moe.moe_route_compact(z((2, 6), i32), z(100, i32), 40, E_global=256)  # map shorter than E_global
    with pytest.raises(moe.MoeError, match="elements"):
        moe.moe_route_compact(z((2, 6), i32), None, 8, out=(z(8, i32), z(8, i32), z(12, i32), z(12, i32)))
    x, w1, w2 = z((2, 64), bf16), z((3, 256, 64), bf16), z((3, 64, 128), bf16)
    c, o, r = z(3, i32), z(4, i32), z(12, i32)
    moe_args = dict(K=6, counts=c, offsets=o, row_to_slot=r)
    with pytest.raises(moe.MoeError, match="shape"):
        moe.moe_grouped_ffn(x, w1=z((3, 200, 64), bf16), w2=w2, **moe_args)  # W1 rows != 2F
    with pytest.raises(moe.MoeError, match="shape"):
        moe.moe_grouped_ffn(z((2, 32), bf16), w1=w1, w2=w2, **moe_args)      # x width != H
    with pytest.raises(moe.MoeError, match="dtype"):
        moe.moe_grouped_ffn(x, w1=w1, w2=z((3, 64, 128), f32), **moe_args)   # mixed weight dtypes
    with pytest.raises(moe.MoeError, match="elements"):
        moe.moe_grouped_ffn(x, w1=w1, w2=w2, y=z((4, 64), bf16), **moe_args)  # y rows < T*K
    with pytest.raises(moe.MoeError, match="scale"):
        moe.moe_grouped_ffn(x, w1=z((3, 256, 32), u8), w2=z((3, 64, 64), u8), **moe_args)
    with pytest.raises(moe.MoeError, match="elements"):
        moe.moe_grouped_ffn_noalloc(x, w1=w1, w2=w2, K=6, counts=z(2, i32), offsets=o, row_to_slot=r)
    with pytest.raises(moe.MoeError, match="elements"):
        moe.moe_combine(z((12, 64), bf16), z((2, 6), f32), z(11, i32))         # slot_to_row short
    with pytest.raises(moe.MoeError, match="dtype"):
        moe.moe_combine(z((12, 64), bf16), z((2, 6), torch.float64), z(12, i32))
    with pytest.raises(moe.MoeError, match="shape"):
        moe.moe_fused_experts(x, z((2, 6), i32), z((3, 6), f32), w1, w2)      # weights [T, K]
    with pytest.raises(moe.MoeError, match="shape"):
        moe.moe_pack_ffn_weights(z((3, 256, 64), bf16), z((3, 64, 96), bf16))


def test_mxfp4_mma_mode(lib):
    # host-side state only: no kernel launch
    prev = lib.moe_get_mxfp4_mma()
    assert lib.moe_set_mxfp4_mma(1) == 0 and lib.moe_get_mxfp4_mma() == 1
    assert lib.moe_set_mxfp4_mma(0) == 0 and lib.moe_get_mxfp4_mma() == 0
    assert lib.moe_set_mxfp4_mma(2) == 1 and lib.moe_set_mxfp4_mma(-1) == 1  # MOE_ERR_INVALID_ARG
    assert lib.moe_get_mxfp4_mma() == 0
    lib.moe_set_mxfp4_mma(prev)


@_no_gpu
def test_probe_validation(lib):
    f = lib.moe_probe_mfma_clock
    assert f(0, 4, 0, FAKE, NULL, NULL) == 1       # iters < 1
    assert f(10, 0, 0, FAKE, NULL, NULL) == 1      # blocks < 1
    assert f(10, 4, 2, FAKE, NULL, NULL) == 1      # toggle not 0/1
    assert f(10, 4, 1, NULL, NULL, NULL) == 1      # null out
    assert lib.moe_probe_mfma(0, 4, FAKE, NULL) == 1
    assert lib.moe_probe_read(FAKE, 24, FAKE, 4096 * 256, NULL) == 1      # bytes % 16
    assert lib.moe_probe_read(FAKE, 32, FAKE, 100, NULL) == 4             # out too short
    assert lib.moe_probe_copy(FAKE, FAKE, 8, NULL) == 1
