"""C ABI checks that need no GPU: exports, validation errors, buffer sizing (no compute calls).

Every error below is returned by host-side validation before anything is enqueued. The fake
device addresses passed here are never dereferenced.
"""
import ctypes

import pytest

from mixture_experts_layer_32_amd import binding as b

FAKE = 1 << 20          # a 256-byte-aligned non-null address, never touched on the host


def desc(**kw):
    base = dict(T=256, H=256, F=128, E_total=8, topk=2, mode="bf16")
    base.update(kw)
    return b.Desc.make(**base)


def test_library_exports_every_declared_function():
    L = b.lib()
    names = b.header_functions()
    assert {"moe_fwd", "moe_bwd", "moe_route", "moe_query_sizes", "moe_saved_layout"} <= set(names)
    for n in names:
        assert hasattr(L, n), n
    assert "gfx950" in b.version()


@pytest.mark.parametrize("kw,code", [
    (dict(T=0), "MOE_ERR_INVALID_ARG"),
    (dict(topk=9), "MOE_ERR_INVALID_ARG"),
    (dict(topk=0), "MOE_ERR_INVALID_ARG"),
    (dict(E_local=4, expert_offset=5), "MOE_ERR_INVALID_ARG"),
    (dict(H=384), "MOE_ERR_UNSUPPORTED_SHAPE"),
    (dict(F=192), "MOE_ERR_UNSUPPORTED_SHAPE"),
    (dict(E_total=513, topk=2), "MOE_ERR_UNSUPPORTED_SHAPE"),
    (dict(E_total=64, topk=33), "MOE_ERR_UNSUPPORTED_SHAPE"),
    (dict(T=1 << 28, topk=8), "MOE_ERR_UNSUPPORTED_SHAPE"),
    (dict(mode=7), "MOE_ERR_UNSUPPORTED_MODE"),
    (dict(mode=-1), "MOE_ERR_UNSUPPORTED_MODE"),
    (dict(H=384, mode="mxfp8"), "MOE_ERR_UNSUPPORTED_SHAPE"),
    (dict(F=192, mode="fp8_bwd"), "MOE_ERR_UNSUPPORTED_SHAPE"),
    (dict(H=384, mode="fp8"), "MOE_ERR_UNSUPPORTED_SHAPE"),
    (dict(mode=5), "MOE_ERR_UNSUPPORTED_MODE"),
    (dict(recompute=2), "MOE_ERR_INVALID_ARG"),
    (dict(recompute=-1), "MOE_ERR_INVALID_ARG"),
])
def test_validation_errors(kw, code):
    with pytest.raises(b.MoEError) as ei:
        b.query_sizes(desc(**kw))
    assert ei.value.code == code
    assert b.lib().moe_last_error().decode()


def test_fwd_bwd_reject_bad_pointers_and_small_workspace_without_launching():
    d = desc()
    fwd, bwd, saved = b.query_sizes(d)
    with pytest.raises(b.MoEError, match="MOE_ERR_INVALID_ARG"):
        b.moe_fwd(d, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, fwd, stream=0)
    with pytest.raises(b.MoEError, match="not 16-byte aligned"):
        b.moe_fwd(d, FAKE + 2, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, fwd, stream=0)
    with pytest.raises(b.MoEError, match="MOE_ERR_WORKSPACE_TOO_SMALL"):
        b.moe_fwd(d, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, fwd - 1, stream=0)
    with pytest.raises(b.MoEError, match="MOE_ERR_WORKSPACE_TOO_SMALL"):
        b.moe_bwd(d, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, bwd - 256, stream=0)
    with pytest.raises(b.MoEError, match="dlogits is null"):
        b.moe_bwd(d, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, bwd, stream=0)
    with pytest.raises(b.MoEError, match="saved is not 256-byte aligned"):
        b.moe_route(d, FAKE, FAKE + 16, FAKE, fwd, stream=0)


def test_sizes_cover_the_layout():
    d = desc(T=1000, H=512, F=256, E_total=16, topk=4)
    fwd, bwd, saved = b.query_sizes(d)
    rows = 1000 * 4
    assert all(v % 256 == 0 for v in (fwd, bwd, saved))
    assert saved >= rows * (4 * 4) + rows * 3 * 256 * 2           # routing + a, b and the copy of hw (bf16)
    assert fwd >= rows * 512 * 2                                  # per-pair expert outputs
    assert bwd >= rows * 512 * 2 + rows * 2 * 256 * 2 + rows * 4 * (256 // 64)
    off = b.saved_layout(d)
    assert off["idx"] == 0 and off["weight"] >= rows * 4
    assert off["pair_pos"] + rows * 4 <= saved
    f32 = b.query_sizes(desc(T=1000, H=512, F=256, E_total=16, topk=4, mode="fp32"))
    assert f32[2] > saved                                        # fp32 activations are wider


@pytest.mark.parametrize("mode", ["mxfp8", "fp8_bwd", "fp8"])
def test_mx_sizes_cover_the_layout(mode):
    T, H, F, E, k = 1000, 512, 256, 16, 4
    d = desc(T=T, H=H, F=F, E_total=E, topk=k, mode=mode)
    fwd, bwd, saved = b.query_sizes(d)
    rows = T * k
    qc = -(-(rows + 128 * E) // 128) * 128                    # pair columns, segments padded to 128
    assert all(v % 256 == 0 for v in (fwd, bwd, saved))
    # routing + a, b (bf16) + the fp8 pair-contiguous hw copy with its scales
    assert saved >= rows * (4 * 4) + rows * 2 * F * 2 + qc * F * (1 + 1 / 32)
    if mode in ("mxfp8", "fp8"):    # quantised x, weights and hw, plus the per-pair outputs; the
        # weights' backward orientation is kept in saved
        assert fwd >= rows * H * 2 + T * H * (1 + 1 / 32) + 3 * E * F * H * (1 + 1 / 32) + rows * F * (1 + 1 / 32)
        assert saved >= rows * 2 * F * 2 + (qc * F + 3 * E * F * H) * (1 + 1 / 32)
        wq = 0
    else:                  # bf16 hw (its fp8 transposed copy is in saved), plus the per-pair outputs
        assert fwd >= rows * H * 2 + rows * F * 2
        wq = 3 * E * F * H
    # quantised dy, weights (FP8_BWD), dY^T, x^T, da/db (both orientations), partials, dX'
    assert bwd >= (T * H + wq + 2 * H * qc + rows * 2 * F + 2 * F * qc) * (1 + 1 / 32) \
        + rows * 4 * 2 * ((F + 255) // 256) + rows * H * 2


@pytest.mark.parametrize("args,code,msg", [
    ((None, 64, 64, 1), "MOE_ERR_INVALID_ARG", "in is null"),
    ((FAKE + 8, 64, 64, 1), "MOE_ERR_INVALID_ARG", "not 16-byte aligned"),
    ((FAKE, 0, 64, 1), "MOE_ERR_INVALID_ARG", "positive"),
    ((FAKE, 64, 64, 2), "MOE_ERR_INVALID_ARG", "axis"),
    ((FAKE, 64, 48, 1), "MOE_ERR_UNSUPPORTED_SHAPE", "multiple of 32"),
    ((FAKE, 192, 128, 0), "MOE_ERR_UNSUPPORTED_SHAPE", "multiple of 128"),
    ((FAKE, 128, 96, 0), "MOE_ERR_UNSUPPORTED_SHAPE", "multiple of 128"),
    ((FAKE, 1 << 17, 1 << 17, 1), "MOE_ERR_UNSUPPORTED_SHAPE", r"2\^34"),
])
def test_mx_quantize_validation(args, code, msg):
    x, rows, cols, axis = args
    with pytest.raises(b.MoEError, match=msg) as ei:
        b.moe_mx_quantize(x, rows, cols, axis, FAKE, FAKE, stream=0)
    assert ei.value.code == code


@pytest.mark.parametrize("args,code,msg", [
    ((None, 128, 128, 0), "MOE_ERR_INVALID_ARG", "in is null"),
    ((FAKE + 8, 128, 128, 0), "MOE_ERR_INVALID_ARG", "not 16-byte aligned"),
    ((FAKE, 0, 128, 0), "MOE_ERR_INVALID_ARG", "positive"),
    ((FAKE, 128, 128, 2), "MOE_ERR_INVALID_ARG", "weight"),
    ((FAKE, 64, 96, 0), "MOE_ERR_UNSUPPORTED_SHAPE", "cols must be a multiple of 128"),
    ((FAKE, 64, 128, 1), "MOE_ERR_UNSUPPORTED_SHAPE", "rows must be a multiple of 128"),
    ((FAKE, 1 << 17, 1 << 17, 0), "MOE_ERR_UNSUPPORTED_SHAPE", r"2\^34"),
])
def test_fp8_block_quantize_validation(args, code, msg):
    x, rows, cols, weight = args
    with pytest.raises(b.MoEError, match=msg) as ei:
        b.moe_fp8_block_quantize(x, rows, cols, weight, FAKE, FAKE, FAKE, FAKE, stream=0)
    assert ei.value.code == code
    with pytest.raises(b.MoEError, match="qt is null"):
        b.moe_fp8_block_quantize(FAKE, 128, 128, 1, FAKE, FAKE, None, FAKE, stream=0)


def test_status_strings():
    L = b.lib()
    for code in range(6):
        assert L.moe_status_string(code)
    assert L.moe_profile_kernel(10 ** 6, None, None, None) != 0


def test_router_validation_without_launching():
    d = desc(T=300, E_total=40, topk=2)
    fwd, bwd = b.query_router_sizes(d)
    assert min(b.query_router_sizes(desc(mode="fp32"))) >= 256     # fp32 test mode: no partials
    with pytest.raises(b.MoEError, match="MOE_ERR_UNSUPPORTED_MODE"):
        b.query_router_sizes(desc(mode=7))
    with pytest.raises(b.MoEError, match="w_router is null"):
        b.moe_router_fwd(d, FAKE, None, FAKE, FAKE, fwd, stream=0)
    with pytest.raises(b.MoEError, match="logits is not 16-byte aligned"):
        b.moe_router_fwd(d, FAKE, FAKE, FAKE + 4, FAKE, fwd, stream=0)
    with pytest.raises(b.MoEError, match="MOE_ERR_WORKSPACE_TOO_SMALL"):
        b.moe_router_fwd(d, FAKE, FAKE, FAKE, FAKE, fwd - 1, stream=0)
    with pytest.raises(b.MoEError, match="dw_router is null"):
        b.moe_router_bwd(d, FAKE, FAKE, FAKE, FAKE, None, FAKE, bwd, stream=0)
    with pytest.raises(b.MoEError, match="MOE_ERR_WORKSPACE_TOO_SMALL"):
        b.moe_router_bwd(d, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, bwd - 256, stream=0)
    with pytest.raises(b.MoEError, match="ws is not 256-byte aligned"):
        b.moe_router_bwd(d, FAKE, FAKE, FAKE + 4, FAKE, FAKE, FAKE + 16, bwd, stream=0)


@pytest.mark.parametrize("T,H,E", [(300, 256, 40), (16384, 2048, 128), (5, 512, 512), (70000, 1024, 64)])
def test_router_sizes_cover_the_partials(T, H, E):
    fwd, bwd = b.query_router_sizes(desc(T=T, H=H, E_total=E, topk=2))
    Ep = (E + 63) // 64 * 64
    assert fwd % 256 == 0 and bwd % 256 == 0
    assert fwd >= T * Ep * 4                        # at least one slice of fp32 partial logits
    assert bwd >= 1024 + T * Ep * 2 + E * H * 4     # zero page, bf16 dlogits, at least one dW_r slice


def test_layer_rejects_mismatched_tensors_before_the_library():
    """layer.py checks device, dtype, shape and contiguity of every tensor it hands to the C ABI,
    which receives bare pointers (a host pointer or a wrong-sized buffer would reach the kernels)."""
    import torch
    from mixture_experts_layer_32_amd.layer import _expect
    cpu = torch.device("cpu")
    ok = torch.zeros(4, 8, dtype=torch.bfloat16)
    _expect(ok, "x", (4, 8), torch.bfloat16, cpu)
    with pytest.raises(ValueError, match="dtype"):
        _expect(ok.float(), "x", (4, 8), torch.bfloat16, cpu)
    with pytest.raises(ValueError, match="shape"):
        _expect(ok, "x", (4, 16), torch.bfloat16, cpu)
    with pytest.raises(ValueError, match="contiguous"):
        _expect(torch.zeros(8, 4, dtype=torch.bfloat16).t(), "x", (4, 8), torch.bfloat16, cpu)
    with pytest.raises(ValueError, match="tensor on"):
        _expect(ok, "x", (4, 8), torch.bfloat16, torch.device("cuda", 0))
    with pytest.raises(ValueError, match="torch.Tensor"):
        _expect(12345, "x", (4, 8), torch.bfloat16, cpu)


@pytest.mark.parametrize("mode", ["fp32", "bf16", "mxfp8", "fp8_bwd", "fp8"])
def test_recompute_keeps_only_routing_in_saved(mode):
    """Activation checkpointing: `saved` shrinks to the routing results (no activation, no quantised
    weight), and the backward workspace grows by the recomputed activations."""
    T, H, F, E, k = 1000, 512, 256, 16, 4
    rows = T * k
    kw = dict(T=T, H=H, F=F, E_total=E, topk=k, mode=mode)
    fwd0, bwd0, saved0 = b.query_sizes(desc(**kw))
    fwd1, bwd1, saved1 = b.query_sizes(desc(recompute=1, **kw))
    elem = 4 if mode == "fp32" else 2
    # routing: idx, weight, perm, ptok, pair_pos, M-tile tables, counts, offsets, zero page, qoff
    routing = rows * 4 * 5 + (rows // 128 + E + 1) * 8 + (rows // 256 + E + 1) * 8 + 1024 + 4 * 256
    assert saved1 <= routing + 16 * 256
    assert saved0 - saved1 >= rows * 2 * F * elem                 # a and b at least
    assert bwd1 - bwd0 >= rows * 2 * F * elem                     # recomputed a and b
    off0, off1 = b.saved_layout(desc(**kw)), b.saved_layout(desc(recompute=1, **kw))
    for n in ("idx", "weight", "counts", "offsets", "perm", "pair_pos", "qoff", "qcols"):
        assert off1[n] == off0[n], n
    for n in ("hwt", "hwt_scales", "wdt", "wdt_scales", "wgut", "wgut_scales"):
        assert off1[n] == 0, n
    assert fwd1 >= fwd0 - 256
