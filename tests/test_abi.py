"""C-ABI checks that need no GPU: the library loads, exports every entry point
include/moe.h declares, reports geometry, and rejects bad arguments on the
host before anything is enqueued."""
import ctypes
import os
import re

import pytest

import bit_dequant_expert_moe_amd as moe
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HDR = os.path.join(ROOT, "include", "moe.h")

D = moe.Dims()  # hidden 4096, inter 1024, 512 experts, top-4, group 64, 4-bit, shared


def _declared():
    src = open(HDR).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    L = moe.lib()
    names = _declared()
    assert set(names) == set(moe.EXPORTS)
    for n in names:
        assert hasattr(L, n), n


def test_abi_version_and_status_strings():
    assert moe.moe_abi_version() == 1
    assert moe.moe_status_str(0) == "ok"
    assert moe.moe_status_str(-5) == "workspace too small"
    assert moe.moe_status_str(123) == "unknown status"


def test_expert_bytes_and_layout_match_format():
    assert moe.moe_expert_bytes(D) == 7_077_888
    assert moe.moe_expert_bytes(moe.Dims(bits=2)) == 3_932_160
    for dims in [D, moe.Dims(bits=2), moe.Dims(hidden=512, inter=256, n_experts=8, top_k=2)]:
        od = oracle.Dims(H=dims.hidden, I=dims.inter, E=dims.n_experts, K=dims.top_k,
                         bits=dims.bits)
        assert moe.moe_blob_layout(dims) == [oracle.section_offset(od, s) for s in range(6)]
        assert moe.moe_expert_bytes(dims) == oracle.blob_bytes(od)


@pytest.mark.parametrize("field,value,status", [
    ("group", 32, -3), ("bits", 8, -3), ("bits", 3, -3),
    ("hidden", 4000, -2), ("hidden", 128, -2), ("hidden", 32768, -2),
    ("inter", 768, -2), ("n_experts", 0, -2), ("n_experts", 2048, -2),
    ("top_k", 0, -2), ("top_k", 9, -2), ("has_shared", 2, -2)])
def test_check_dims_rejects(field, value, status):
    kw = dict(D.__dict__)
    kw[field] = value
    assert moe.moe_check_dims(moe.Dims(**kw)) == status
    assert moe.moe_expert_bytes(moe.Dims(**kw)) == 0


def test_top_k_above_expert_count_rejected():
    assert moe.moe_check_dims(moe.Dims(n_experts=3, top_k=4)) == -2
    assert moe.moe_check_dims(moe.Dims(n_experts=4, top_k=4)) == 0


def test_workspace_bytes():
    n1 = moe.moe_workspace_bytes(D, 1)
    n64 = moe.moe_workspace_bytes(D, 64)
    assert 0 < n1 < n64
    # h [T][K+1][I] fp32 dominates
    assert n64 >= 64 * 5 * 1024 * 4
    assert moe.moe_workspace_bytes(D, 0) == 0
    assert moe.moe_workspace_bytes(D, 4097) == 0
    assert moe.moe_workspace_bytes(D, 4096) > moe.moe_workspace_bytes(D, 256)
    assert n1 % 256 == 0


# Fake, well-aligned device addresses: every call below must fail validation
# before touching them.
A = 0x7f0000000000
L_OK = moe.make_layer(A, A + 0x100000, 7_077_888, A + 0x40000000)
WS = A + 0x80000000


def _route(**kw):
    args = dict(d=D, router=A, x=A + 4096, T=1, ids=A + 8192, w=A + 12288, logits=None,
                ws=WS, ws_bytes=moe.moe_workspace_bytes(D, 1), stream=0)
    args.update(kw)
    return args


def _status(fn, **kw):
    with pytest.raises(moe.MoeError) as ei:
        fn(**kw)
    return ei.value.status


def test_route_validation():
    assert _status(moe.moe_route, **_route(router=None)) == -1
    assert _status(moe.moe_route, **_route(ids=None)) == -1
    assert _status(moe.moe_route, **_route(ws=None)) == -1
    assert _status(moe.moe_route, **_route(T=0)) == -2
    assert _status(moe.moe_route, **_route(T=4097)) == -2
    assert _status(moe.moe_route, **_route(x=A + 8)) == -4
    assert _status(moe.moe_route, **_route(ws=WS + 16)) == -4
    assert _status(moe.moe_route, **_route(ws_bytes=100)) == -5
    assert _status(moe.moe_route, **_route(d=moe.Dims(group=128))) == -3


def _fwd(**kw):
    args = dict(d=D, layer=L_OK, x=A, T=1, ids=A + 4096, w=A + 8192, y=A + 16384, ws=WS,
                ws_bytes=moe.moe_workspace_bytes(D, 1), stream=0)
    args.update(kw)
    return args


def test_expert_forward_validation():
    f = moe.moe_expert_forward
    assert _status(f, **_fwd(y=None)) == -1
    assert _status(f, **_fwd(layer=moe.make_layer(A, None, 7_077_888, A))) == -1
    assert _status(f, **_fwd(layer=moe.make_layer(A, A, 7_077_888, None))) == -1
    nosh = moe.Dims(has_shared=0)
    assert _status(f, **_fwd(d=nosh, ws_bytes=moe.moe_workspace_bytes(nosh, 1))) == -2
    assert _status(f, **_fwd(layer=moe.make_layer(A, A, 7_077_000, A))) == -2   # stride < blob
    assert _status(f, **_fwd(layer=moe.make_layer(A, A, 7_077_888 + 16, A))) == -4
    assert _status(f, **_fwd(layer=moe.make_layer(A, A + 64, 7_077_888, A))) == -4
    assert _status(f, **_fwd(y=A + 4)) == -4
    assert _status(f, **_fwd(T=2)) == -5   # workspace sized for T=1


def test_layer_decode_validation():
    f = moe.moe_layer_decode
    args = dict(d=D, layer=L_OK, x=A, T=1, y=A + 65536, ids=None, w=None, ws=WS,
                ws_bytes=moe.moe_workspace_bytes(D, 1), stream=0)
    assert _status(f, **{**args, "x": None}) == -1
    assert _status(f, **{**args, "ids": A + 2}) == -4
    assert _status(f, **{**args, "d": moe.Dims(bits=3)}) == -3
    assert _status(f, **{**args, "ws_bytes": 256}) == -5


def test_dequantize_and_misc_validation():
    assert _status(moe.moe_dequantize, d=D, blob=A, which=3, out=A, stream=0) == -2
    assert _status(moe.moe_dequantize, d=D, blob=A + 16, which=0, out=A, stream=0) == -4
    assert _status(moe.moe_dequantize, d=D, blob=None, which=0, out=A, stream=0) == -1
    f = moe.moe_dequantize_as
    assert _status(f, d=D, blob=A, which=0, decoder=5, out=A, stream=0) == -2
    assert _status(f, d=D, blob=A, which=0, decoder=-1, out=A, stream=0) == -2
    assert _status(f, d=D, blob=A, which=-1, decoder=0, out=A, stream=0) == -2
    assert _status(f, d=D, blob=A, which=0, decoder=0, out=A + 4, stream=0) == -4
    assert _status(moe.moe_workspace_init, ws=None, ws_bytes=256, stream=0) == -1
    assert _status(moe.moe_workspace_init, ws=WS, ws_bytes=16, stream=0) == -5
    assert moe.lib().moe_get_device_error(None, None, ctypes.byref(ctypes.c_int32())) == -1


def test_layer_decode_residual_validation():
    f = moe.moe_layer_decode_residual
    args = dict(d=D, layer=L_OK, resid=A, T=1, x_out=None, y=None, ids=None, w=None, ws=WS,
                ws_bytes=moe.moe_workspace_bytes(D, 1), stream=0)
    assert _status(f, **{**args, "resid": None}) == -1
    assert _status(f, **{**args, "layer": moe.make_layer(None, A, 7_077_888, A)}) == -1
    assert _status(f, **{**args, "resid": A + 4}) == -4
    assert _status(f, **{**args, "x_out": A + 8}) == -4
    assert _status(f, **{**args, "y": A + 4}) == -4
    assert _status(f, **{**args, "T": 0}) == -2
    assert _status(f, **{**args, "d": moe.Dims(bits=3)}) == -3
    assert _status(f, **{**args, "ws_bytes": 256}) == -5
    assert _status(f, **{**args, "T": 4}) == -5   # workspace sized for T=1


def test_stack_decode_validation():
    f = moe.moe_stack_decode
    args = dict(d=D, layers=[L_OK, L_OK], x=A, y=A + 65536, ids=None, w=None, ws=WS,
                ws_bytes=moe.moe_workspace_bytes(D, 1), stream=0)
    assert _status(f, **{**args, "x": None}) == -1
    assert _status(f, **{**args, "layers": [L_OK, moe.make_layer(None, A, 7_077_888, A)]}) == -1
    assert _status(f, **{**args, "layers": [L_OK, moe.make_layer(A + 8, A, 7_077_888, A)]}) == -4
    assert _status(f, **{**args, "layers": []}) == -2
    assert _status(f, **{**args, "y": A + 4}) == -4
    assert _status(f, **{**args, "ws_bytes": 256}) == -5
    assert _status(f, **{**args, "d": moe.Dims(bits=3)}) == -3


@pytest.mark.parametrize("fn", ["moe_stack_decode_residual", "moe_stack_decode_residual_noalloc"])
def test_stack_decode_residual_validation(fn):
    # every check runs before the no-allocation variant's first HIP call
    f = getattr(moe, fn)
    args = dict(d=D, layers=[L_OK] * 3, resid=A, x_out=None, y=None, ids=None, w=None, stream=0)
    if fn == "moe_stack_decode_residual":
        args.update(ws=WS, ws_bytes=moe.moe_workspace_bytes(D, 1))
    assert _status(f, **{**args, "resid": None}) == -1
    assert _status(f, **{**args, "layers": [L_OK, moe.make_layer(A, None, 7_077_888, A)]}) == -1
    assert _status(f, **{**args, "layers": []}) == -2
    assert _status(f, **{**args, "resid": A + 4}) == -4
    assert _status(f, **{**args, "x_out": A + 2}) == -4
    assert _status(f, **{**args, "ids": A + 1}) == -4
    assert _status(f, **{**args, "d": moe.Dims(group=32)}) == -3
    nosh = moe.Dims(has_shared=0)
    assert _status(f, **{**args, "d": nosh}) == -2   # layer has a shared blob


def test_noalloc_scratch_covers_every_valid_dims():
    # the one-token workspace of the largest dims fits the per-GPU array
    worst = 0
    for H in (256, 4096, 16384):
        for I in (256, 1024, 16384):
            for E in (1, 512, 1024):
                for K in (1, 8):
                    for bits in (2, 4):
                        d = moe.Dims(hidden=H, inter=I, n_experts=E, top_k=min(K, E), bits=bits)
                        worst = max(worst, moe.moe_workspace_bytes(d, 1))
    assert 0 < worst <= moe.NOALLOC_SCRATCH_BYTES
    hdr = open(HDR).read()
    assert "#define MOE_NOALLOC_SCRATCH_BYTES (2u * 1024u * 1024u)" in hdr
    assert moe.NOALLOC_SCRATCH_BYTES == 2 * 1024 * 1024


def test_stream_read_and_flush_validation():
    assert moe.moe_stream_read_sink_words(1 << 20) > 0
    assert _status(moe.moe_stream_read, src=None, nbytes=4096, sink=A, stream=0) == -1
    assert _status(moe.moe_stream_read, src=A, nbytes=4096, sink=None, stream=0) == -1
    assert _status(moe.moe_stream_read, src=A, nbytes=0, sink=A, stream=0) == -2
    assert _status(moe.moe_stream_read, src=A, nbytes=4100, sink=A, stream=0) == -2
    assert _status(moe.moe_stream_read, src=A + 8, nbytes=4096, sink=A, stream=0) == -4
    assert _status(moe.moe_flush, dst=None, nbytes=4096, stream=0) == -1
    assert _status(moe.moe_flush, dst=A, nbytes=24, stream=0) == -2
    assert _status(moe.moe_flush, dst=A + 4, nbytes=4096, stream=0) == -4


def test_timing_switch_and_empty_read():
    # no GPU call: with nothing recorded a read only copies the totals
    moe.moe_timing_set(True)
    assert moe.moe_timing_read(reset=True) == {}
    moe.moe_timing_set(False)
    assert moe.moe_timing_read() == {}
    assert moe.lib().moe_timing_read(None, 0) == -1  # MOE_ERR_NULL
