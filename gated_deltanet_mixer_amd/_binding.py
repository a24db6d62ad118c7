"""ctypes binding of libgdn.so (include/gdn.h), one wrapper per C entry point
with the same name.  Only argument marshalling happens here: torch supplies
device memory and the current stream; every step of the computation runs in
the library's HIP kernels.  There is no fallback: if the library is missing
or fails to load, every call raises.
"""
import ctypes
import os

import torch  # loaded first so libgdn binds to the HIP runtime torch uses

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libgdn.so")

GDN_F32, GDN_BF16 = 0, 1
GDN_ALGO_AUTO, GDN_ALGO_SEQUENTIAL, GDN_ALGO_CHUNKED = 0, 1, 2
_ALGOS = {"auto": GDN_ALGO_AUTO, "sequential": GDN_ALGO_SEQUENTIAL, "chunked": GDN_ALGO_CHUNKED}


class GDNError(RuntimeError):
    def __init__(self, status, fn):
        self.status = status
        super().__init__(f"{fn}: {gdn_status_str(status)} (status {status})")


class gdn_dims(ctypes.Structure):
    _fields_ = [("n_qk_heads", ctypes.c_int32), ("n_v_heads", ctypes.c_int32),
                ("head_k_dim", ctypes.c_int32), ("head_v_dim", ctypes.c_int32)]


_lib = None


def lib():
    """The loaded libgdn.so; raises if it was never built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libgdn.so not found at {LIB_PATH}; build it with "
                               "`python -m gated_deltanet_mixer_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
        L.gdn_status_str.argtypes = [ctypes.c_int]
        L.gdn_status_str.restype = ctypes.c_char_p
        L.gdn_abi_version.argtypes = []
        L.gdn_abi_version.restype = ctypes.c_int
        L.gdn_conv_silu.argtypes = [P, i64, i32, P, i32, P, P, i32, i32, i32, i32, i32, i32, f32,
                                    P]
        L.gdn_conv_silu.restype = ctypes.c_int
        L.gdn_prefill_workspace_bytes.argtypes = [i32, i32, gdn_dims, i32, i32]
        L.gdn_prefill_workspace_bytes.restype = sz
        L.gdn_prefill.argtypes = [P, i64, P, i64, P, i64, i32, P, P, i32, P, P, P, P, P, i32, i32,
                                  i32, gdn_dims, f32, i32, P, sz, P]
        L.gdn_prefill.restype = ctypes.c_int
        L.gdn_decode_rows.argtypes = [P, i64, P, i64, P, i64, i32, P, P, i32, P, P, P, P, P, i32,
                                      gdn_dims, f32, P]
        L.gdn_decode_rows.restype = ctypes.c_int
        L.gdn_decode_rows_multi.argtypes = [P, i64, i64, P, i64, i64, P, i64, i64, i32, P, P,
                                            i32, P, P, P, P, P, P, i32, i32, gdn_dims, f32, P]
        L.gdn_decode_rows_multi.restype = ctypes.c_int
        L.gdn_gated_rmsnorm.argtypes = [P, P, i64, P, i32, P, i32, i32, i32, f32, P]
        L.gdn_gated_rmsnorm.restype = ctypes.c_int
        L.gdn_prefill_slots_workspace_bytes.argtypes = [i32, i32, gdn_dims]
        L.gdn_prefill_slots_workspace_bytes.restype = sz
        L.gdn_prefill_slots.argtypes = [P, i64, P, i64, P, i64, i32, P, P, i32, P, P, P, P, P,
                                        i32, i32, i32, i32, gdn_dims, f32, P, sz, P]
        L.gdn_prefill_slots.restype = ctypes.c_int
        L.gdn_mixer_prefill_workspace_bytes.argtypes = [i32, i32, gdn_dims]
        L.gdn_mixer_prefill_workspace_bytes.restype = sz
        L.gdn_mixer_prefill.argtypes = [P, i64, P, i64, i32, P, P, P, P, i32, P, P, P, P, P, P,
                                        i32, i32, gdn_dims, f32, f32, f32, P, sz, P]
        L.gdn_mixer_prefill.restype = ctypes.c_int
        L.gdn_gate_proj_workspace_bytes.argtypes = [i32, i32, i32]
        L.gdn_gate_proj_workspace_bytes.restype = sz
        L.gdn_gate_proj.argtypes = [P, i64, i32, P, P, P, P, i64, i32, i32, i32, P, sz, P]
        L.gdn_gate_proj.restype = ctypes.c_int
        L.gdn_prefill_noalloc.argtypes = [P, i64, P, i64, P, i64, i32, P, P, i32, P, P, P, P, P,
                                          i32, i32, i32, gdn_dims, f32, i32, P]
        L.gdn_prefill_noalloc.restype = ctypes.c_int
        L.gdn_linear_workspace_bytes.argtypes = []
        L.gdn_linear_workspace_bytes.restype = sz
        L.gdn_linear.argtypes = [P, i64, P, i64, P, i64, i32, i32, i32, i32, P, sz, P]
        L.gdn_linear.restype = ctypes.c_int
        L.gdn_linear_tune.argtypes = L.gdn_linear.argtypes
        L.gdn_linear_tune.restype = ctypes.c_int
        L.gdn_linear_kernel.argtypes = [i32, i32, i32, i64, i64, ctypes.c_size_t]
        L.gdn_linear_kernel.restype = ctypes.c_int
        _lib = L
    return _lib


def gdn_status_str(status):
    return lib().gdn_status_str(int(status)).decode()


def gdn_abi_version():
    return int(lib().gdn_abi_version())


def _dt(t):
    if t.dtype == torch.bfloat16:
        return GDN_BF16
    if t.dtype == torch.float32:
        return GDN_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _check(status, fn):
    if status != 0:
        raise GDNError(status, fn)


def _need_cuda(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("all tensors must be on the GPU")


def _tok_stride(t, heads, d):
    """Token stride of a [B, T, heads, d] view whose heads are packed."""
    B, T = t.shape[0], t.shape[1]
    if t.shape[2:] != (heads, d):
        raise ValueError(f"expected a [B, T, {heads}, {d}] view")
    if t.numel() == 0:
        return heads * d
    if t.stride(3) != 1 or t.stride(2) != d:
        raise ValueError(f"expected a [B, T, {heads}, {d}] view with packed heads")
    if B > 1 and t.stride(0) != T * t.stride(1):
        raise ValueError("batch stride must be T * token stride")
    return t.stride(1)


def _seq_stride(t, name):
    """Token stride of a [B, T, C] view with contiguous channels, whose tokens
    lie at (b*T + t) * stride (a column range of a wider buffer is fine)."""
    B, T, C = t.shape
    if t.numel() == 0 or B * T == 1:
        return C
    if C > 1 and t.stride(2) != 1:
        raise ValueError(f"{name} must have contiguous channels")
    if T > 1:
        ts = t.stride(1)
        if B > 1 and t.stride(0) != T * ts:
            raise ValueError(f"{name}: batch stride must be T * token stride")
        return ts
    return t.stride(0)


def gdn_conv_silu(x, w, conv_state=None, l2_channels=0, head_dim=128, l2_eps=1e-6, y=None,
                  y_dtype=None):
    """Depthwise causal conv (width 4) + silu over x [B, T, C] (a view with a
    token stride is accepted), optional L2 of the first l2_channels channels
    per head; conv_state [B, 3, C] f32 in/out.  y_dtype (default x.dtype)
    selects the output dtype when y is not given."""
    _need_cuda(x, w, conv_state, y)
    B, T, C = x.shape
    if y is None:
        y = torch.empty(x.shape, dtype=y_dtype or x.dtype, device=x.device)
    assert y.is_contiguous() and w.is_contiguous()
    if conv_state is not None:
        assert conv_state.is_contiguous() and conv_state.dtype == torch.float32
    _check(lib().gdn_conv_silu(_ptr(x), _seq_stride(x, "x"), _dt(x), _ptr(y), _dt(y), _ptr(w),
                               _ptr(conv_state), B, T, C, w.shape[1], l2_channels, head_dim,
                               l2_eps, _stream(x)),
           "gdn_conv_silu")
    return y


def gdn_prefill_workspace_bytes(B, T, Hk, Hv, dk=128, dv=128, qkv_dtype=torch.bfloat16,
                                algo="auto"):
    dt = GDN_BF16 if qkv_dtype == torch.bfloat16 else GDN_F32
    return int(lib().gdn_prefill_workspace_bytes(B, T, gdn_dims(Hk, Hv, dk, dv), dt,
                                                 _ALGOS[algo]))


def gdn_prefill(q, k, v, a, b, A_log, dt_bias, state_in=None, state_out=None, o=None,
                q_scale=1.0, algo="auto", workspace=None, o_dtype=None):
    """Gated delta rule over q, k [B,T,Hk,dk] and v [B,T,Hv,dv] (views with a
    token stride are accepted), gates a, b [B,T,Hv].  Returns o [B,T,Hv,dv]
    (dtype o_dtype, default v.dtype, when o is not given)."""
    _need_cuda(q, k, v, a, b, A_log, dt_bias, state_in, state_out, o, workspace)
    B, T, Hk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    qs, ks, vs = _tok_stride(q, Hk, dk), _tok_stride(k, Hk, dk), _tok_stride(v, Hv, dv)
    if o is None:
        o = torch.empty((B, T, Hv, dv), dtype=o_dtype or v.dtype, device=v.device)
    assert o.is_contiguous() and a.is_contiguous() and b.is_contiguous()
    for s in (state_in, state_out):
        if s is not None:
            assert s.is_contiguous() and s.dtype == torch.float32
    need = gdn_prefill_workspace_bytes(B, T, Hk, Hv, dk, dv, q.dtype, algo)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().gdn_prefill(_ptr(q), qs, _ptr(k), ks, _ptr(v), vs, _dt(q), _ptr(a), _ptr(b),
                             _dt(a), _ptr(A_log), _ptr(dt_bias), _ptr(state_in), _ptr(state_out),
                             _ptr(o), _dt(o), B, T, gdn_dims(Hk, Hv, dk, dv), q_scale,
                             _ALGOS[algo],
                             _ptr(workspace), ws_bytes, _stream(q)),
           "gdn_prefill")
    return o


def gdn_prefill_noalloc(q, k, v, a, b, A_log, dt_bias, state_in=None, state_out=None, o=None,
                        q_scale=1.0, algo="auto", o_dtype=None):
    """gdn_prefill with the library's fixed device scratch instead of a
    workspace (for callers that cannot allocate).  o is allocated here when
    not given; pass it to allocate nothing."""
    _need_cuda(q, k, v, a, b, A_log, dt_bias, state_in, state_out, o)
    B, T, Hk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    qs, ks, vs = _tok_stride(q, Hk, dk), _tok_stride(k, Hk, dk), _tok_stride(v, Hv, dv)
    if o is None:
        o = torch.empty((B, T, Hv, dv), dtype=o_dtype or v.dtype, device=v.device)
    assert o.is_contiguous() and a.is_contiguous() and b.is_contiguous()
    for s in (state_in, state_out):
        if s is not None:
            assert s.is_contiguous() and s.dtype == torch.float32
    _check(lib().gdn_prefill_noalloc(_ptr(q), qs, _ptr(k), ks, _ptr(v), vs, _dt(q), _ptr(a),
                                     _ptr(b), _dt(a), _ptr(A_log), _ptr(dt_bias), _ptr(state_in),
                                     _ptr(state_out), _ptr(o), _dt(o), B, T,
                                     gdn_dims(Hk, Hv, dk, dv), q_scale, _ALGOS[algo], _stream(q)),
           "gdn_prefill_noalloc")
    return o


def gdn_decode_rows(q, k, v, a, b, A_log, dt_bias, state, lengths=None, o=None, q_scale=1.0):
    """One token per fixed row: q, k [R,Hk,dk], v [R,Hv,dv], a, b [R,Hv]; state
    [R,Hv,dv,dk] f32 updated in place; lengths [R] int32 (<0 = idle row)."""
    _need_cuda(q, k, v, a, b, A_log, dt_bias, state, lengths, o)
    R, Hk, dk = q.shape
    Hv, dv = v.shape[1], v.shape[2]
    for t, hh, d in ((q, Hk, dk), (k, Hk, dk), (v, Hv, dv)):
        if t.stride(2) != 1 or t.stride(1) != d:
            raise ValueError("heads must be packed")
    if o is None:
        o = torch.empty((R, Hv, dv), dtype=v.dtype, device=v.device)
    assert state.is_contiguous() and state.dtype == torch.float32
    if lengths is not None:
        assert lengths.dtype == torch.int32 and lengths.is_contiguous()
    _check(lib().gdn_decode_rows(_ptr(q), q.stride(0), _ptr(k), k.stride(0), _ptr(v), v.stride(0),
                                 _dt(q), _ptr(a), _ptr(b), _dt(a), _ptr(A_log), _ptr(dt_bias),
                                 _ptr(state), _ptr(lengths), _ptr(o), R,
                                 gdn_dims(Hk, Hv, dk, dv), q_scale, _stream(q)),
           "gdn_decode_rows")
    return o


def gdn_gated_rmsnorm(x, z, w, eps=1e-6, y=None):
    """y = x / sqrt(mean(x^2) + eps) * (1 + w) * silu(z) over the last axis
    (width 128); x viewed as [N, H, 128]; z of x's shape, contiguous or a view
    whose tokens (all but the last two axes) lie one token stride apart."""
    _need_cuda(x, z, w, y)
    D = x.shape[-1]
    H = x.shape[-2]
    N = x.numel() // (H * D) if x.numel() else 0
    if y is None:
        y = torch.empty_like(x)
    assert x.is_contiguous() and y.is_contiguous() and y.numel() == x.numel()
    if z.is_contiguous():
        assert z.numel() == x.numel()
        zts = H * D
    else:
        assert z.shape == x.shape
        zts = _head_tok_stride(z, H, D)
    _check(lib().gdn_gated_rmsnorm(_ptr(x), _ptr(z), zts, _ptr(y), _dt(x),
                                   _ptr(w), N, H, D, eps, _stream(x)),
           "gdn_gated_rmsnorm")
    return y


def _head_tok_stride(t, H, D):
    """Token stride of a [..., H, D] view with packed heads whose leading axes
    collapse to one token stride."""
    if t.numel() == 0 or t.numel() == H * D:
        return H * D
    if (D > 1 and t.stride(-1) != 1) or (H > 1 and t.stride(-2) != D):
        raise ValueError("expected packed heads of contiguous channels")
    lead = [(n, st) for n, st in zip(t.shape[:-2], t.stride()[:-2]) if n > 1]
    ts = lead[-1][1]
    expect = ts
    for (_, st), (n_inner, _) in zip(reversed(lead[:-1]), reversed(lead[1:])):
        expect *= n_inner
        if st != expect:
            raise ValueError("leading axes must collapse to one token stride")
    return ts


def gdn_mixer_prefill_workspace_bytes(B, T, Hk, Hv, dk=128, dv=128):
    return int(lib().gdn_mixer_prefill_workspace_bytes(B, T, gdn_dims(Hk, Hv, dk, dv)))


def gdn_mixer_prefill(qkv, z, conv_w, a, b, A_log, dt_bias, norm_w, Hk, Hv, conv_state=None,
                      state_in=None, state_out=None, y=None, q_scale=1.0, l2_eps=1e-6,
                      norm_eps=1e-6, workspace=None):
    """Whole mixer between the projections: conv + silu + L2 over qkv [B,T,C],
    the gated delta rule (state carried in/out) and the gated RMSNorm with z
    [B,T,Hv*128].  qkv and z may be views with a token stride (the two column
    ranges of one in_proj_qkvz output).  Returns y [B,T,Hv*128] in qkv's
    dtype."""
    _need_cuda(qkv, z, conv_w, a, b, A_log, dt_bias, norm_w, conv_state, state_in, state_out, y,
               workspace)
    B, T, C = qkv.shape
    if C != 2 * Hk * 128 + Hv * 128:
        raise ValueError(f"qkv has {C} channels, expected {2 * Hk * 128 + Hv * 128}")
    if y is None:
        y = torch.empty((B, T, Hv * 128), dtype=qkv.dtype, device=qkv.device)
    for t in (y, conv_w, a, b, norm_w):
        assert t.is_contiguous()
    assert z.dtype == qkv.dtype and y.dtype == qkv.dtype and z.shape == y.shape
    for s in (conv_state, state_in, state_out):
        if s is not None:
            assert s.is_contiguous() and s.dtype == torch.float32
    need = gdn_mixer_prefill_workspace_bytes(B, T, Hk, Hv)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=qkv.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().gdn_mixer_prefill(_ptr(qkv), _seq_stride(qkv, "qkv"), _ptr(z),
                                   _seq_stride(z, "z"), _dt(qkv), _ptr(conv_w), _ptr(conv_state),
                                   _ptr(a), _ptr(b), _dt(a), _ptr(A_log), _ptr(dt_bias),
                                   _ptr(norm_w), _ptr(state_in), _ptr(state_out), _ptr(y), B, T,
                                   gdn_dims(Hk, Hv, 128, 128), q_scale, l2_eps, norm_eps,
                                   _ptr(workspace), ws_bytes, _stream(qkv)),
           "gdn_mixer_prefill")
    return y


def gdn_prefill_slots_workspace_bytes(R, max_len, Hk, Hv, dk=128, dv=128):
    return int(lib().gdn_prefill_slots_workspace_bytes(R, max_len, gdn_dims(Hk, Hv, dk, dv)))


def _packed_stride(t, heads, d):
    """Token stride of a packed [N, heads, d] view."""
    if t.shape[1:] != (heads, d):
        raise ValueError(f"expected a [N, {heads}, {d}] view")
    if t.numel() and (t.stride(2) != 1 or t.stride(1) != d):
        raise ValueError(f"expected a [N, {heads}, {d}] view with packed heads")
    return t.stride(0) if t.numel() else heads * d


def gdn_prefill_slots(q, k, v, a, b, A_log, dt_bias, cu_seqlens, state, max_len, o=None,
                      q_scale=1.0, workspace=None, o_dtype=None):
    """Ragged prefill of fixed rows: the rows' new tokens packed as q, k
    [N,Hk,dk], v [N,Hv,dv], a, b [N,Hv]; cu_seqlens [R+1] int32 on the GPU;
    state [R,Hv,dv,dk] f32 updated in place; max_len the longest row."""
    _need_cuda(q, k, v, a, b, A_log, dt_bias, cu_seqlens, state, o, workspace)
    N, Hk, dk = q.shape
    Hv, dv = v.shape[1], v.shape[2]
    R = cu_seqlens.numel() - 1
    qs, ks, vs = _packed_stride(q, Hk, dk), _packed_stride(k, Hk, dk), _packed_stride(v, Hv, dv)
    if o is None:
        o = torch.empty((N, Hv, dv), dtype=o_dtype or v.dtype, device=v.device)
    assert o.is_contiguous() and a.is_contiguous() and b.is_contiguous()
    assert cu_seqlens.dtype == torch.int32 and cu_seqlens.is_contiguous()
    assert state.is_contiguous() and state.dtype == torch.float32 and state.shape[0] == R
    need = gdn_prefill_slots_workspace_bytes(R, max_len, Hk, Hv, dk, dv)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().gdn_prefill_slots(_ptr(q), qs, _ptr(k), ks, _ptr(v), vs, _dt(q), _ptr(a),
                                   _ptr(b), _dt(a), _ptr(A_log), _ptr(dt_bias), _ptr(cu_seqlens),
                                   _ptr(state), _ptr(o), _dt(o), R, max_len, N,
                                   gdn_dims(Hk, Hv, dk, dv), q_scale, _ptr(workspace), ws_bytes,
                                   _stream(q)),
           "gdn_prefill_slots")
    return o


def gdn_decode_rows_multi(q, k, v, a, b, A_log, dt_bias, state, snapshots=None, lengths=None,
                          o=None, q_scale=1.0):
    """K tokens per fixed row: q, k [R,K,Hk,dk], v [R,K,Hv,dv], a, b [R,K,Hv];
    state [R,Hv,dv,dk] f32 advanced in place through the K tokens; snapshots
    [R,K,Hv,dv,dk] f32 (optional) gets the state after each token; lengths
    [R] int32 (<0 = idle row).  Returns o [R,K,Hv,dv]."""
    _need_cuda(q, k, v, a, b, A_log, dt_bias, state, snapshots, lengths, o)
    R, K, Hk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    for t, d in ((q, dk), (k, dk), (v, dv)):
        if t.numel() and (t.stride(3) != 1 or t.stride(2) != d):
            raise ValueError("heads must be packed")
    if o is None:
        o = torch.empty((R, K, Hv, dv), dtype=v.dtype, device=v.device)
    assert o.is_contiguous() and a.is_contiguous() and b.is_contiguous()
    assert state.is_contiguous() and state.dtype == torch.float32
    if snapshots is not None:
        assert snapshots.is_contiguous() and snapshots.dtype == torch.float32
        assert snapshots.shape == (R, K, Hv, dv, dk)
    if lengths is not None:
        assert lengths.dtype == torch.int32 and lengths.is_contiguous()
    _check(lib().gdn_decode_rows_multi(_ptr(q), q.stride(0), q.stride(1), _ptr(k), k.stride(0),
                                       k.stride(1), _ptr(v), v.stride(0), v.stride(1), _dt(q),
                                       _ptr(a), _ptr(b), _dt(a), _ptr(A_log), _ptr(dt_bias),
                                       _ptr(state), _ptr(snapshots), _ptr(lengths), _ptr(o), R, K,
                                       gdn_dims(Hk, Hv, dk, dv), q_scale, _stream(q)),
           "gdn_decode_rows_multi")
    return o


def _row_ld(t, name):
    """Row stride of a 2-D view whose rows are contiguous."""
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D")
    if t.shape[1] > 1 and t.stride(1) != 1:
        raise ValueError(f"{name} must have contiguous rows")
    return t.stride(0) if t.shape[0] > 1 else t.shape[1]


def gdn_gate_proj_workspace_bytes(M, K, H):
    return int(lib().gdn_gate_proj_workspace_bytes(M, K, H))


def gdn_gate_proj(x, W_a, W_b, a=None, b=None, workspace=None):
    """a = x W_a^T, b = x W_b^T with f32 weights [H, K] (the mixer's in_proj_a
    and in_proj_b); x [M, K] bf16.  Returns (a, b), each [M, H] f32.  The
    workspace (a uint8 tensor) is allocated here when not given."""
    _need_cuda(x, W_a, W_b, a, b, workspace)
    M, K = x.shape
    H = W_a.shape[0]
    if W_a.shape != (H, K) or W_b.shape != (H, K):
        raise ValueError("W_a and W_b must be [H, K]")
    if not (W_a.is_contiguous() and W_b.is_contiguous()):
        raise ValueError("W_a and W_b must be contiguous")
    if a is None:
        a = torch.empty(M, H, dtype=torch.float32, device=x.device)
    if b is None:
        b = torch.empty(M, H, dtype=torch.float32, device=x.device)
    if a.shape != (M, H) or b.shape != (M, H):
        raise ValueError("a and b must be [M, H]")
    ab_ld = _row_ld(a, "a")
    if _row_ld(b, "b") != ab_ld:
        raise ValueError("a and b must share a row stride")
    need = gdn_gate_proj_workspace_bytes(M, K, H) if M else 0
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().gdn_gate_proj(_ptr(x), _row_ld(x, "x"), _dt(x), _ptr(W_a), _ptr(W_b), _ptr(a),
                               _ptr(b), ab_ld, M, K, H, _ptr(workspace), wsb, _stream(x)),
           "gdn_gate_proj")
    return a, b


def gdn_linear_workspace_bytes():
    return int(lib().gdn_linear_workspace_bytes())


def _linear(fn, name, x, W, y, out_dtype, workspace):
    _need_cuda(x, W, y, workspace)
    M, K = x.shape
    N = W.shape[0]
    if W.shape != (N, K):
        raise ValueError("W must be [N, K]")
    if y is None:
        y = torch.empty(M, N, dtype=out_dtype, device=x.device)
    if y.shape != (M, N):
        raise ValueError("y must be [M, N]")
    if workspace is None:
        wsb = 0
    else:
        wsb = workspace.numel() * workspace.element_size()
    _check(fn(_ptr(x), _row_ld(x, "x"), _ptr(W), _row_ld(W, "W"), _ptr(y), _row_ld(y, "y"),
              _dt(y), M, N, K, _ptr(workspace), wsb, _stream(x)), name)
    return y


def gdn_linear(x, W, y=None, out_dtype=torch.bfloat16, workspace=None):
    """y = x W^T for bf16 x [M, K] and W [N, K] (a Linear layer's weight),
    f32 accumulation; y [M, N] in out_dtype (bf16 or f32)."""
    return _linear(lib().gdn_linear, "gdn_linear", x, W, y, out_dtype, workspace)


def gdn_linear_tune(x, W, y=None, out_dtype=torch.bfloat16, workspace=None):
    """gdn_linear that also times the shape's candidate algorithms and keeps
    the fastest for later gdn_linear calls of the same shape (synchronises)."""
    return _linear(lib().gdn_linear_tune, "gdn_linear_tune", x, W, y, out_dtype, workspace)


def gdn_linear_kernel(M, N, K, x_ld=None, w_ld=None, workspace_bytes=None):
    """Which engine an untimed gdn_linear call of this shape uses on the
    current device: the library GEMM's block width (160, 192, 256 or 320 for
    its tiled form, 64 for its few-row form), or 0 for hipBLASLt.  x_ld and
    w_ld default to K, workspace_bytes to gdn_linear_workspace_bytes()."""
    if workspace_bytes is None:
        workspace_bytes = lib().gdn_linear_workspace_bytes()
    r = lib().gdn_linear_kernel(M, N, K, K if x_ld is None else x_ld,
                                K if w_ld is None else w_ld, workspace_bytes)
    if r < 0:
        raise GDNError(-r, "gdn_linear_kernel")
    return r
