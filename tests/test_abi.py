"""C-ABI checks that need no GPU: the library loads, exports every function
include/gdn.h declares, and rejects bad arguments on the host with the
documented status before anything is launched."""
import ctypes
import os
import re

import pytest

import gated_deltanet_mixer_amd as gdn
from gated_deltanet_mixer_amd import gdn_dims

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")

OK, NULL, SHAPE, DTYPE, ALIGN, UNSUP, WS = 0, 1, 2, 3, 4, 5, 6
P = 0x10000  # a 256-byte-aligned fake device address: never dereferenced on these paths


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z_0-9]+)\s*\(", text)))


def test_header_and_exports():
    L = gdn.lib()
    names = declared_functions()
    assert {"gdn_conv_silu", "gdn_prefill", "gdn_decode_rows", "gdn_gated_rmsnorm",
            "gdn_prefill_workspace_bytes", "gdn_status_str", "gdn_abi_version",
            "gdn_mixer_prefill", "gdn_mixer_prefill_workspace_bytes", "gdn_prefill_slots",
            "gdn_prefill_slots_workspace_bytes", "gdn_decode_rows_multi", "gdn_gate_proj",
            "gdn_linear", "gdn_linear_tune", "gdn_linear_kernel", "gdn_linear_workspace_bytes",
            "gdn_gate_proj_workspace_bytes"} <= set(names)
    for n in names:
        assert hasattr(L, n), n
    assert gdn.gdn_abi_version() == 2
    for s in range(9):
        assert gdn.gdn_status_str(s).startswith("GDN_")
    assert gdn.gdn_status_str(99) == "unknown gdn_status"


def _vp(x):
    return ctypes.c_void_p(x) if x else None


def conv(x=P, y=2 * P, dt=1, ydt=1, w=3 * P, cs=None, B=1, T=8, C=1024, W=4, l2=0, hd=128,
         xts=None):
    xts = C if xts is None else xts
    return gdn.lib().gdn_conv_silu(_vp(x), xts, dt, _vp(y), ydt, _vp(w), _vp(cs), B, T, C, W, l2,
                                   hd, 1e-6, None)


def test_conv_validation():
    assert conv(x=0) == NULL
    assert conv(w=0) == NULL
    assert conv(dt=7) == DTYPE
    assert conv(ydt=-1) == DTYPE
    assert conv(W=3) == UNSUP
    assert conv(W=0) == SHAPE
    assert conv(C=1020) == SHAPE
    assert conv(l2=2048) == SHAPE        # more than C
    assert conv(xts=1016) == SHAPE       # token stride below C
    assert conv(xts=1028) == ALIGN       # token stride not a multiple of 8
    # y starts inside the last token's row of a strided x
    assert conv(xts=16384, B=2, T=4, y=P + (7 * 16384 + 1024) * 2 - 64) == SHAPE
    assert conv(l2=100, hd=64) == SHAPE  # not a whole number of heads
    assert conv(l2=128, hd=64) == UNSUP
    assert conv(x=P + 8) == ALIGN
    assert conv(cs=P + 4) == ALIGN
    assert conv(y=P + 512) == SHAPE      # y overlaps x
    assert conv(T=0) == OK               # no-op, nothing launched
    assert conv(B=0) == OK


D16 = gdn_dims(16, 48, 128, 128)


def prefill(q=P, qs=2048, k=2 * P, ks=2048, v=3 * P, vs=6144, qdt=1, a=4 * P, b=5 * P, gdt=0,
            Al=6 * P, db=7 * P, si=None, so=None, o=8 * P, odt=1, B=1, T=64, dims=D16, algo=0,
            ws=None, wsb=0):
    return gdn.lib().gdn_prefill(_vp(q), qs, _vp(k), ks, _vp(v), vs, qdt, _vp(a), _vp(b), gdt,
                                 _vp(Al), _vp(db), _vp(si), _vp(so), _vp(o), odt, B, T, dims, 1.0,
                                 algo, _vp(ws), wsb, None)


def test_prefill_validation():
    assert prefill(q=0) == NULL
    assert prefill(o=0) == NULL
    assert prefill(qdt=2) == DTYPE
    assert prefill(odt=4) == DTYPE
    assert prefill(dims=gdn_dims(16, 40, 128, 128)) == SHAPE
    assert prefill(dims=gdn_dims(16, 48, 64, 64)) == UNSUP
    assert prefill(qs=1024) == SHAPE                 # stride shorter than the heads
    assert prefill(qs=2052) == ALIGN
    assert prefill(q=P + 2) == ALIGN
    assert prefill(si=P + 8) == ALIGN
    assert prefill(algo=9) == SHAPE
    assert prefill(B=-1) == SHAPE
    assert prefill(B=0) == OK
    need = gdn.lib().gdn_prefill_workspace_bytes(1, 64, D16, 1, 0)
    if need > 0:
        assert prefill(ws=None, wsb=0) == WS
        assert prefill(ws=9 * P, wsb=need - 1) == WS
    assert gdn.lib().gdn_prefill_workspace_bytes(1, 64, D16, 0, 0) == 0  # f32: sequential
    assert gdn.lib().gdn_prefill_workspace_bytes(1, 64, D16, 1, 1) == 0
    # the chunked algorithm is bf16-only: f32 q/k/v need no workspace and an
    # explicit CHUNKED request with them is refused before any launch
    assert gdn.lib().gdn_prefill_workspace_bytes(1, 64, D16, 0, 2) == 0
    assert prefill(qdt=0, algo=2) == UNSUP
    assert prefill(qdt=0, algo=2, B=0) == UNSUP


def test_prefill_noalloc_rejects_sizes_beyond_its_scratch():
    # The fixed scratch holds the chunked workspace of B*T <= 1152 tokens at
    # 16/48 heads; larger calls are refused on the host before any launch.
    L = gdn.lib()
    assert L.gdn_prefill_workspace_bytes(1, 1152, D16, 1, 0) <= (64 << 20)
    assert L.gdn_prefill_workspace_bytes(1, 1153, D16, 1, 0) > (64 << 20)

    def na(B, T, qdt=1, algo=0):
        return L.gdn_prefill_noalloc(_vp(P), 2048, _vp(2 * P), 2048, _vp(3 * P), 6144, qdt,
                                     _vp(4 * P), _vp(5 * P), 0, _vp(6 * P), _vp(7 * P), None,
                                     None, _vp(8 * P), 1, B, T, D16, 1.0, algo, None)
    assert na(1, 1153) == 8            # GDN_ERR_SCRATCH
    assert na(2, 4096) == 8
    assert na(1, 64, qdt=0, algo=2) == UNSUP   # validation as gdn_prefill
    assert na(0, 64) == OK


def decode(q=P, k=2 * P, v=3 * P, qdt=1, st=4 * P, o=5 * P, R=4, dims=D16, lengths=None):
    return gdn.lib().gdn_decode_rows(_vp(q), 2048, _vp(k), 2048, _vp(v), 6144, qdt, _vp(6 * P),
                                     _vp(7 * P), 1, _vp(8 * P), _vp(9 * P), _vp(st), _vp(lengths),
                                     _vp(o), R, dims, 1.0, None)


def test_decode_validation():
    assert decode(st=0) == NULL
    assert decode(qdt=5) == DTYPE
    assert decode(dims=gdn_dims(16, 48, 96, 128)) == UNSUP
    assert decode(R=-1) == SHAPE
    assert decode(st=P + 4) == ALIGN
    assert decode(lengths=P + 2) == ALIGN
    assert decode(R=0) == OK


def decode_multi(q=P, k=2 * P, v=3 * P, qdt=1, st=4 * P, snap=None, o=5 * P, R=4, K=3,
                 dims=D16, lengths=None, qts=2048, vts=6144):
    return gdn.lib().gdn_decode_rows_multi(_vp(q), 3 * 2048, qts, _vp(k), 3 * 2048, qts, _vp(v),
                                           3 * 6144, vts, qdt, _vp(6 * P), _vp(7 * P), 1,
                                           _vp(8 * P), _vp(9 * P), _vp(st), _vp(snap),
                                           _vp(lengths), _vp(o), R, K, dims, 1.0, None)


def test_decode_multi_validation():
    assert decode_multi(st=0) == NULL
    assert decode_multi(qdt=5) == DTYPE
    assert decode_multi(dims=gdn_dims(16, 48, 96, 128)) == UNSUP
    assert decode_multi(R=-1) == SHAPE
    assert decode_multi(K=-2) == SHAPE
    assert decode_multi(qts=1024) == SHAPE       # token stride shorter than the heads
    assert decode_multi(qts=2052) == ALIGN
    assert decode_multi(snap=P + 4) == ALIGN
    assert decode_multi(snap=4 * P) == SHAPE     # snapshots on top of the state
    assert decode_multi(R=0) == OK
    assert decode_multi(K=0) == OK


def test_norm_validation():
    L = gdn.lib()
    f = lambda x=P, z=2 * P, y=3 * P, w=4 * P, dt=1, N=4, H=48, D=128, zts=None: \
        L.gdn_gated_rmsnorm(_vp(x), _vp(z), H * D if zts is None else zts, _vp(y), dt, _vp(w),
                            N, H, D, 1e-6, None)
    assert f(z=0) == NULL
    assert f(dt=3) == DTYPE
    assert f(D=64) == UNSUP
    assert f(N=-2) == SHAPE
    assert f(w=P + 4) == ALIGN
    assert f(zts=48 * 128 - 8) == SHAPE
    assert f(zts=16384 + 4) == ALIGN
    assert f(zts=16384, N=0) == OK
    assert f(N=0) == OK


def mixer(qkv=P, z=2 * P, dt=1, cw=3 * P, cs=None, a=4 * P, b=5 * P, gdt=1, Al=6 * P, db=7 * P,
          nw=8 * P, si=None, so=None, y=9 * P, B=1, T=64, dims=D16, ws=64 * P, wsb=None,
          qts=None, zts=None):
    L = gdn.lib()
    if wsb is None:
        wsb = L.gdn_mixer_prefill_workspace_bytes(B, T, dims)
    C = (2 * dims.n_qk_heads + dims.n_v_heads) * 128
    qts = C if qts is None else qts
    zts = dims.n_v_heads * 128 if zts is None else zts
    return L.gdn_mixer_prefill(_vp(qkv), qts, _vp(z), zts, dt, _vp(cw), _vp(cs), _vp(a), _vp(b), gdt,
                               _vp(Al), _vp(db), _vp(nw), _vp(si), _vp(so), _vp(y), B, T, dims,
                               1.0, 1e-6, 1e-6, _vp(ws), wsb, None)


def test_mixer_prefill_validation():
    L = gdn.lib()
    need = L.gdn_mixer_prefill_workspace_bytes(1, 64, D16)
    # q|k f32 + v bf16 conv output, then the chunked workspace
    assert need >= 64 * 4096 * 4 + 64 * 6144 * 2 + L.gdn_prefill_workspace_bytes(1, 64, D16, 1, 2)
    assert L.gdn_mixer_prefill_workspace_bytes(0, 64, D16) == 0
    assert L.gdn_mixer_prefill_workspace_bytes(1, 64, gdn_dims(16, 40, 128, 128)) == 0
    assert mixer(qkv=0) == NULL
    assert mixer(cw=0) == NULL
    assert mixer(nw=0) == NULL
    assert mixer(dt=2) == DTYPE
    assert mixer(gdt=9) == DTYPE
    assert mixer(dims=gdn_dims(16, 40, 128, 128)) == SHAPE
    assert mixer(dims=gdn_dims(16, 48, 64, 64)) == UNSUP
    assert mixer(B=-1) == SHAPE
    assert mixer(qkv=P + 8) == ALIGN
    assert mixer(nw=P + 4) == ALIGN
    assert mixer(cs=P + 4) == ALIGN
    assert mixer(ws=None) == WS
    assert mixer(wsb=need - 1) == WS
    assert mixer(ws=64 * P + 128) == ALIGN
    assert mixer(y=64 * P) == SHAPE      # y inside the workspace
    assert mixer(y=2 * P) == SHAPE       # y on top of z
    C = (2 * D16.n_qk_heads + D16.n_v_heads) * 128
    assert mixer(qts=C - 8) == SHAPE
    assert mixer(zts=D16.n_v_heads * 128 - 8) == SHAPE
    assert mixer(qts=C + 4) == ALIGN
    assert mixer(zts=D16.n_v_heads * 128 + 12) == ALIGN
    # a wide z stride reaches y: the last token's z row ends inside y's bytes
    assert mixer(y=40 * P, z=40 * P - (63 * 16384 + 6144) * 2 + 64, zts=16384) == SHAPE
    assert mixer(qts=0, zts=0, B=0, T=0) == OK  # no tokens: strides unused
    assert mixer(B=0) == OK


def slots(q=P, k=2 * P, v=3 * P, qdt=1, a=4 * P, b=5 * P, gdt=0, cu=6 * P, st=7 * P, o=8 * P,
          R=4, max_len=100, total=300, dims=D16, ws=64 * P, wsb=None):
    L = gdn.lib()
    if wsb is None:
        wsb = L.gdn_prefill_slots_workspace_bytes(R, max_len, dims)
    return L.gdn_prefill_slots(_vp(q), 2048, _vp(k), 2048, _vp(v), 6144, qdt, _vp(a), _vp(b), gdt,
                               _vp(9 * P), _vp(10 * P), _vp(cu), _vp(st), _vp(o), 1, R, max_len,
                               total, dims, 1.0, _vp(ws), wsb, None)


def test_prefill_slots_validation():
    L = gdn.lib()
    assert L.gdn_prefill_slots_workspace_bytes(4, 100, D16) == \
        L.gdn_prefill_workspace_bytes(4, 100, D16, 1, 2)
    assert L.gdn_prefill_slots_workspace_bytes(0, 100, D16) == 0
    assert slots(cu=0) == NULL
    assert slots(st=0) == NULL
    assert slots(q=0) == NULL
    assert slots(qdt=3) == DTYPE
    assert slots(dims=gdn_dims(16, 40, 128, 128)) == SHAPE
    assert slots(R=-1) == SHAPE
    assert slots(max_len=-5) == SHAPE
    assert slots(cu=6 * P + 2) == ALIGN
    assert slots(st=7 * P + 8) == ALIGN
    assert slots(ws=None) == WS
    assert slots(wsb=100) == WS
    assert slots(R=0) == OK
    assert slots(total=0, q=0, k=0, v=0, a=0, b=0, o=0) == OK   # no tokens: nothing to do


def test_gate_proj_validation():
    L = gdn.lib()
    need = L.gdn_gate_proj_workspace_bytes(8, 5120, 48)
    assert need > 0 and need % 256 == 0
    assert L.gdn_gate_proj_workspace_bytes(8, 5000, 48) == 0
    assert L.gdn_gate_proj_workspace_bytes(0, 5120, 48) == 0

    def f(x=P, xld=5120, xdt=1, wa=2 * P, wb=3 * P, a=4 * P, b=5 * P, ld=48, M=8, K=5120, H=48,
          ws=64 * P, wsb=None):
        if wsb is None:
            wsb = need
        return L.gdn_gate_proj(_vp(x), xld, xdt, _vp(wa), _vp(wb), _vp(a), _vp(b), ld, M, K, H,
                               _vp(ws), wsb, None)
    assert f(wa=0) == NULL
    assert f(b=0) == NULL
    assert f(xdt=5) == DTYPE
    assert f(xdt=0) == UNSUP           # f32 activations are not implemented
    assert f(H=80, ld=80) == UNSUP     # more than 64 outputs per projection
    assert f(K=5000) == SHAPE          # K % 32
    assert f(H=40) == SHAPE            # H % 16
    assert f(xld=4096) == SHAPE        # row stride below K
    assert f(ld=32) == SHAPE           # output row stride below H
    assert f(M=-1) == SHAPE
    assert f(xld=5124) == ALIGN
    assert f(wa=2 * P + 4) == ALIGN
    assert f(ws=None) == WS
    assert f(wsb=need - 256) == WS
    assert f(ws=64 * P + 16) == ALIGN
    assert f(a=P + 64) == SHAPE        # a overlaps x
    assert f(b=64 * P) == SHAPE        # b overlaps the workspace
    assert f(M=0, x=0, wa=0, wb=0, a=0, b=0, ws=None, wsb=0) == OK


def test_linear_validation():
    L = gdn.lib()
    assert L.gdn_linear_workspace_bytes() == 32 << 20

    def f(x=P, xld=5120, W=64 * P, wld=5120, y=4096 * P, yld=10240, ydt=1, M=8, N=10240,
          K=5120, ws=None, wsb=0):
        return L.gdn_linear(_vp(x), xld, _vp(W), wld, _vp(y), yld, ydt, M, N, K, _vp(ws), wsb,
                            None)
    assert f(x=0) == NULL
    assert f(W=0) == NULL
    assert f(ydt=2) == DTYPE
    assert f(N=0) == SHAPE
    assert f(K=0) == SHAPE
    assert f(M=-3) == SHAPE
    assert f(xld=100) == SHAPE         # below K
    assert f(yld=10000) == SHAPE       # below N
    assert f(xld=5124) == ALIGN
    assert f(y=4096 * P + 8) == ALIGN
    assert f(ws=P * 8192 + 64, wsb=1024) == ALIGN
    assert f(ws=None, wsb=1024) == WS
    assert f(y=P + 1024) == SHAPE      # y overlaps x
    assert f(ws=P + 4096, wsb=1024) == SHAPE           # workspace overlaps x
    assert f(ws=4096 * P + 256, wsb=1024) == SHAPE     # workspace overlaps y
    assert f(M=0, x=0, W=0, y=0) == OK
    # the timing variant validates the same way, before touching the device
    assert L.gdn_linear_tune(None, 5120, _vp(64 * P), 5120, _vp(4096 * P), 10240, 1, 8, 10240,
                             5120, None, 0, None) == NULL
    assert L.gdn_linear_tune(_vp(P), 100, _vp(64 * P), 5120, _vp(4096 * P), 10240, 1, 8, 10240,
                             5120, None, 0, None) == SHAPE
    # the engine query validates its shape before it asks the device anything
    assert L.gdn_linear_kernel(8, 0, 64, 64, 64, 0) == -SHAPE
    assert L.gdn_linear_kernel(-1, 64, 64, 64, 64, 0) == -SHAPE
    assert L.gdn_linear_kernel(8, 64, 64, 32, 64, 0) == -SHAPE   # x_ld below K
    assert L.gdn_linear_kernel(8, 64, 64, 64, 0, 0) == -SHAPE    # w_ld below K


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    from gated_deltanet_mixer_amd import _binding
    monkeypatch.setattr(_binding, "_lib", None)
    monkeypatch.setattr(_binding, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="libgdn.so not found"):
        _binding.lib()
