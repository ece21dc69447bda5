"""MI355X (gfx950) per-chunk WY/UT preparation of chunkwise (Gated) DeltaNet.

Thin Python binding over the C ABI in ``include/wyprep.h`` (libwyprep.so, built in-tree by
``chunkwise_gated_deltanet_amd.build``).  This module only checks and marshals arguments:
every step of the computation runs in the library's HIP kernels.  PyTorch provides device
memory and the current stream.  There is no CPU fallback: if the library is missing the calls
raise.

Page cited: "TileLang 实战：单位下三角矩阵求逆" (TileLang in practice: inverting a unit
lower-triangular matrix), section 1 -- for every chunk of C tokens and value head:
A = I + strictLower(diag(beta) K K^T), T = A^{-1}, W = T diag(beta) K, U = T diag(beta) V;
section 5, item 12 for the gated coefficient diag(beta)(Gamma o K K^T).  With log gates g
[B,T,Hv] (the FlashQLA usage section passes g beside beta): G_i = g_0 + ... + g_i within the
chunk, Gamma[i][j] = exp(G_i - G_j), and W = T diag(beta exp(G)) K.
"""
from __future__ import annotations

import ctypes
import os

__all__ = ["wy_prepare", "kkt_solve", "wu_prepare", "solve_rhs", "wy_backward", "chunk_fwd",
           "chunk_gated_delta_rule", "wyp_wy_prepare", "wyp_kkt_solve", "wyp_wu_prepare",
           "wyp_solve_rhs", "wyp_wy_backward", "wyp_chunk_fwd", "cp_segment_chunks",
           "auto_segment_chunks", "load_library", "Problem", "LIB_PATH", "WyprepError"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libwyprep.so")

WYP_OK, WYP_ERR_INVALID_ARGUMENT, WYP_ERR_UNSUPPORTED, WYP_ERR_HIP = 0, 1, 2, 3
WYP_BF16, WYP_F32 = 0, 1
ABI_VERSION = 8


class WyprepError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{_STATUS.get(status, status)}: {detail}")
        self.status = status


_STATUS = {0: "WYP_OK", 1: "WYP_ERR_INVALID_ARGUMENT", 2: "WYP_ERR_UNSUPPORTED", 3: "WYP_ERR_HIP"}


class Problem(ctypes.Structure):
    """Mirror of wyp_problem."""
    _fields_ = [(n, ctypes.c_int32) for n in (
        "batch", "seqlen", "num_qk_heads", "num_v_heads", "head_dim_k", "head_dim_v",
        "chunk_size", "num_seqs", "kv_dtype")]


_P = ctypes.c_void_p
_lib = None


def load_library(path: str | None = None):
    """Loads libwyprep.so (raises if it has not been built)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is missing: build it with chunkwise_gated_deltanet_amd.build "
                           "(or __graft_entry__.build()); there is no fallback path")
    lib = ctypes.CDLL(p)
    lib.wyp_abi_version.restype = ctypes.c_int32
    lib.wyp_abi_version.argtypes = []
    lib.wyp_status_string.restype = ctypes.c_char_p
    lib.wyp_status_string.argtypes = [ctypes.c_int32]
    lib.wyp_last_error.restype = ctypes.c_char_p
    lib.wyp_last_error.argtypes = []
    lib.wyp_kkt_solve.restype = ctypes.c_int32
    lib.wyp_kkt_solve.argtypes = [ctypes.POINTER(Problem), _P, _P, _P, _P, _P, _P]
    lib.wyp_wy_prepare.restype = ctypes.c_int32
    lib.wyp_wy_prepare.argtypes = [ctypes.POINTER(Problem), _P, _P, _P, _P, _P, _P, _P, _P, _P]
    lib.wyp_wu_prepare.restype = ctypes.c_int32
    lib.wyp_wu_prepare.argtypes = [ctypes.POINTER(Problem), _P, _P, _P, _P, _P, _P, _P, _P]
    lib.wyp_solve_rhs.restype = ctypes.c_int32
    lib.wyp_solve_rhs.argtypes = [ctypes.POINTER(Problem), _P, _P, _P, _P, _P, _P, _P]
    lib.wyp_chunk_fwd.restype = ctypes.c_int32
    lib.wyp_chunk_fwd.argtypes = [ctypes.POINTER(Problem), _P, _P, _P, _P, _P, _P, ctypes.c_float,
                                  _P, _P, _P, _P]
    lib.wyp_chunk_fwd_cp.restype = ctypes.c_int32
    lib.wyp_chunk_fwd_cp.argtypes = [ctypes.POINTER(Problem), _P, _P, _P, _P, _P, _P,
                                     ctypes.c_float, _P, ctypes.c_int32, _P, ctypes.c_int64, _P,
                                     _P, _P]
    lib.wyp_chunk_fwd_cp_noalloc.restype = ctypes.c_int32
    lib.wyp_chunk_fwd_cp_noalloc.argtypes = [ctypes.POINTER(Problem), _P, _P, _P, _P, _P, _P,
                                             ctypes.c_float, _P, ctypes.c_int32, _P, _P, _P]
    lib.wyp_chunk_fwd_cp_workspace_bytes.restype = ctypes.c_int64
    lib.wyp_chunk_fwd_cp_workspace_bytes.argtypes = [ctypes.POINTER(Problem), _P, ctypes.c_int32]
    lib.wyp_wy_backward.restype = ctypes.c_int32
    lib.wyp_wy_backward.argtypes = [ctypes.POINTER(Problem)] + [_P] * 13
    if lib.wyp_abi_version() != ABI_VERSION:
        raise RuntimeError(f"{p} has ABI version {lib.wyp_abi_version()}, this binding expects "
                           f"{ABI_VERSION}: rebuild it")
    if path is None:
        _lib = lib
    return lib


def _check(lib, status: int):
    if status != WYP_OK:
        detail = lib.wyp_last_error().decode(errors="replace")
        if status in (WYP_ERR_INVALID_ARGUMENT, WYP_ERR_UNSUPPORTED):
            raise ValueError(f"{_STATUS[status]}: {detail}")
        raise WyprepError(status, detail)


def _kv_dtype(t):
    import torch
    if t.dtype == torch.bfloat16:
        return WYP_BF16
    if t.dtype == torch.float32:
        return WYP_F32
    raise TypeError(f"k/v must be bfloat16 or float32, got {t.dtype}")


def _require(t, name, ndim, device):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _gate_ptr(g, beta):
    """Device pointer of the log gates g [B,T,Hv] float32 (shape of beta), or None."""
    import torch
    if g is None:
        return None
    _require(g, "g", 3, beta.device)
    if g.dtype != torch.float32:
        raise TypeError("g must be float32")
    if g.shape != beta.shape:
        raise ValueError(f"g shape {tuple(g.shape)} must match beta {tuple(beta.shape)}")
    return g.data_ptr()


def _problem(k, beta, chunk_size, cu_seqlens, v=None):
    import torch
    device = k.device
    _require(k, "k", 4, device)
    _require(beta, "beta", 3, device)
    if beta.dtype != torch.float32:
        raise TypeError("beta must be float32")
    B, T, Hq, dk = k.shape
    if beta.shape[:2] != (B, T):
        raise ValueError(f"beta shape {tuple(beta.shape)} does not match k {tuple(k.shape)}")
    Hv = beta.shape[2]
    dv = dk
    if v is not None:
        _require(v, "v", 4, device)
        if v.dtype != k.dtype:
            raise TypeError("k and v must share a dtype")
        if v.shape[:3] != (B, T, Hv):
            raise ValueError(f"v shape {tuple(v.shape)} does not match beta {tuple(beta.shape)}")
        dv = v.shape[3]
    n = 0
    if cu_seqlens is not None:
        _require(cu_seqlens, "cu_seqlens", 1, device)
        if cu_seqlens.dtype != torch.int32:
            raise TypeError("cu_seqlens must be int32")
        n = cu_seqlens.numel() - 1
    return Problem(B, T, Hq, Hv, dk, dv, int(chunk_size), n, _kv_dtype(k))


def _stream(device):
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _out(t, shape, dtype, device, name):
    import torch
    if t is None:
        return torch.empty(shape, dtype=dtype, device=device)
    _require(t, name, len(shape), device)
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} of shape {tuple(shape)}")
    return t


def kkt_solve(k, beta, chunk_size, cu_seqlens=None, T_out=None, g=None):
    """T [B,T,Hv,C] (float32) from k [B,T,Hq,128], beta [B,T,Hv] and optional log gates g
    [B,T,Hv]; see wyp_kkt_solve."""
    import torch
    lib = load_library()
    p = _problem(k, beta, chunk_size, cu_seqlens)
    gp = _gate_ptr(g, beta)
    B, T = k.shape[:2]
    T_out = _out(T_out, (B, T, p.num_v_heads, p.chunk_size), torch.float32, k.device, "T_out")
    st = lib.wyp_kkt_solve(ctypes.byref(p), k.data_ptr(), gp, beta.data_ptr(),
                           cu_seqlens.data_ptr() if cu_seqlens is not None else None,
                           T_out.data_ptr(), _stream(k.device))
    _check(lib, st)
    return T_out


def wy_prepare(k, v, beta, chunk_size, cu_seqlens=None, T_out=None, W_out=None, U_out=None,
               g=None):
    """(T, W, U): T [B,T,Hv,C] float32, W [B,T,Hv,128] and U [B,T,Hv,128] in k's dtype.
    g: optional log gates [B,T,Hv] float32."""
    import torch
    lib = load_library()
    p = _problem(k, beta, chunk_size, cu_seqlens, v=v)
    gp = _gate_ptr(g, beta)
    B, T = k.shape[:2]
    Hv = p.num_v_heads
    T_out = _out(T_out, (B, T, Hv, p.chunk_size), torch.float32, k.device, "T_out")
    W_out = _out(W_out, (B, T, Hv, p.head_dim_k), k.dtype, k.device, "W_out")
    U_out = _out(U_out, (B, T, Hv, p.head_dim_v), k.dtype, k.device, "U_out")
    st = lib.wyp_wy_prepare(ctypes.byref(p), k.data_ptr(), v.data_ptr(), gp, beta.data_ptr(),
                            cu_seqlens.data_ptr() if cu_seqlens is not None else None,
                            T_out.data_ptr(), W_out.data_ptr(), U_out.data_ptr(),
                            _stream(k.device))
    _check(lib, st)
    return T_out, W_out, U_out


def wu_prepare(k, v, beta, chunk_size, cu_seqlens=None, W_out=None, U_out=None, g=None):
    """(W, U) without T in HBM: the same values as wy_prepare's W and U; see wyp_wu_prepare."""
    import torch
    lib = load_library()
    p = _problem(k, beta, chunk_size, cu_seqlens, v=v)
    gp = _gate_ptr(g, beta)
    B, T = k.shape[:2]
    Hv = p.num_v_heads
    W_out = _out(W_out, (B, T, Hv, p.head_dim_k), k.dtype, k.device, "W_out")
    U_out = _out(U_out, (B, T, Hv, p.head_dim_v), k.dtype, k.device, "U_out")
    st = lib.wyp_wu_prepare(ctypes.byref(p), k.data_ptr(), v.data_ptr(), gp, beta.data_ptr(),
                            cu_seqlens.data_ptr() if cu_seqlens is not None else None,
                            W_out.data_ptr(), U_out.data_ptr(), _stream(k.device))
    _check(lib, st)
    return W_out, U_out


def solve_rhs(k, rhs, beta, chunk_size, cu_seqlens=None, X_out=None, g=None):
    """X = A^{-1} diag(beta) R per chunk and value head, T never formed (rhs = v gives U); see
    wyp_solve_rhs.  rhs [B,T,Hv,128] in k's dtype; returns X of the same shape and dtype."""
    lib = load_library()
    p = _problem(k, beta, chunk_size, cu_seqlens, v=rhs)
    gp = _gate_ptr(g, beta)
    X_out = _out(X_out, tuple(rhs.shape), k.dtype, k.device, "X_out")
    st = lib.wyp_solve_rhs(ctypes.byref(p), k.data_ptr(), rhs.data_ptr(), gp, beta.data_ptr(),
                           cu_seqlens.data_ptr() if cu_seqlens is not None else None,
                           X_out.data_ptr(), _stream(k.device))
    _check(lib, st)
    return X_out


def wy_backward(k, v, beta, chunk_size, dW, dU, dT=None, g=None, cu_seqlens=None):
    """(dk, dv, dbeta, dg): the gradient of <dT,T> + <dW,W> + <dU,U> through wy_prepare with
    respect to k, v, beta and g (dg None without gates); see wyp_wy_backward.  dW, dU in k's
    dtype with W / U's shapes; dT [B,T,Hv,C] float32 or None."""
    import torch
    lib = load_library()
    p = _problem(k, beta, chunk_size, cu_seqlens, v=v)
    gp = _gate_ptr(g, beta)
    B, T = k.shape[:2]
    Hv = p.num_v_heads
    for t, name, shape in ((dW, "dW", (B, T, Hv, p.head_dim_k)), (dU, "dU", (B, T, Hv, p.head_dim_v))):
        _require(t, name, 4, k.device)
        if tuple(t.shape) != shape or t.dtype != k.dtype:
            raise ValueError(f"{name} must be {k.dtype} of shape {shape}")
    if dT is not None:
        _require(dT, "dT", 4, k.device)
        if dT.dtype != torch.float32 or tuple(dT.shape) != (B, T, Hv, p.chunk_size):
            raise ValueError(f"dT must be float32 of shape {(B, T, Hv, p.chunk_size)}")
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    db = torch.empty_like(beta)
    dg = torch.empty_like(beta) if g is not None else None
    st = lib.wyp_wy_backward(ctypes.byref(p), k.data_ptr(), v.data_ptr(), gp, beta.data_ptr(),
                             cu_seqlens.data_ptr() if cu_seqlens is not None else None,
                             dT.data_ptr() if dT is not None else None, dW.data_ptr(),
                             dU.data_ptr(), dk.data_ptr(), dv.data_ptr(), db.data_ptr(),
                             dg.data_ptr() if dg is not None else None, _stream(k.device))
    _check(lib, st)
    return dk, dv, db, dg


def cp_segment_chunks(batch, seqlen, num_v_heads, chunk_size=64, cus=256, target=512):
    """Chunks per segment for wyp_chunk_fwd_cp.  No split (all chunks in one segment) once the
    4 dv-slice workgroups per sequence and head give every CU one; otherwise enough segments for
    about `target` 32-column workgroups in the output pass (which the launch then runs as half
    as many 64-column ones), at least 4 chunks each.  Measured on MI355X at C = 64: B=1 T=8192
    H=16 runs 231 us unsplit, 198 / 142 / 108 / 127 / 178 us with segments of 64 / 32 / 16 / 8 /
    4 chunks; B=1 T=32768 H=8 runs 859 us unsplit, 375 / 271 / 201 / 229 / 320 us at 128 / 64 /
    32 / 16 / 8; B=2 T=8192 H=32 (256 workgroups unsplit) runs 256 us unsplit, 272 / 294 us at
    64 / 32."""
    nchunks = max(1, -(-seqlen // chunk_size))
    items = batch * num_v_heads * 4
    if items >= cus:
        return nchunks
    nseg = max(1, min(-(-target // items), nchunks // 4))
    return -(-nchunks // nseg)


def auto_segment_chunks(batch, seqlen, num_v_heads, chunk_size=64, num_seqs=None):
    """segment_chunks for the automatic split of chunk_fwd, or None where cp_segment_chunks
    would not split.  A packed batch (num_seqs sequences, `seqlen` tokens in all, batch 1)
    counts as num_seqs rows of its mean length."""
    C = int(chunk_size)
    if num_seqs is None:
        rows, mean = batch, seqlen
    else:
        rows = max(int(num_seqs), 1)
        mean = -(-seqlen // rows)
    L = cp_segment_chunks(rows, mean, num_v_heads, C)
    return L if L < -(-mean // C) else None


def chunk_fwd(q, k, w, u, chunk_size=64, g=None, initial_state=None, scale=None,
              cu_seqlens=None, output_final_state=False, o_out=None, final_state=None,
              segment_chunks=None):
    """(o, final_state) of the gated delta rule from q, k and the chunk's W, U (as returned by
    wy_prepare / wu_prepare for the same k, beta, g); see wyp_chunk_fwd.  q, k [B,T,Hq,128],
    w, u [B,T,Hv,128] bf16; g [B,T,Hv] float32 or None; initial_state [N,Hv,128,128] float32
    or None.  final_state is None unless output_final_state (or a final_state buffer).
    segment_chunks (int, or "auto") splits each sequence into segments of that many chunks run
    in parallel (wyp_chunk_fwd_cp; the workspace comes from torch).  "auto" picks it with
    auto_segment_chunks (no split where that gives None)."""
    import torch
    lib = load_library()
    device = k.device
    _require(q, "q", 4, device)
    _require(k, "k", 4, device)
    _require(w, "w", 4, device)
    _require(u, "u", 4, device)
    if q.shape != k.shape or q.dtype != k.dtype or w.dtype != k.dtype or u.dtype != k.dtype:
        raise ValueError("q must match k; w, u must share k's dtype")
    B, T, Hq, dk = k.shape
    Hv = w.shape[2]
    if w.shape[:2] != (B, T) or u.shape[:3] != (B, T, Hv):
        raise ValueError(f"w {tuple(w.shape)} / u {tuple(u.shape)} do not match k {tuple(k.shape)}")
    dv = u.shape[3]
    n = 0
    if cu_seqlens is not None:
        _require(cu_seqlens, "cu_seqlens", 1, device)
        if cu_seqlens.dtype != torch.int32:
            raise TypeError("cu_seqlens must be int32")
        n = cu_seqlens.numel() - 1
    N = n if cu_seqlens is not None else B
    gp = None
    if g is not None:
        _require(g, "g", 3, device)
        if g.dtype != torch.float32 or tuple(g.shape) != (B, T, Hv):
            raise ValueError(f"g must be float32 of shape {(B, T, Hv)}")
        gp = g.data_ptr()
    h0p = None
    if initial_state is not None:
        _require(initial_state, "initial_state", 4, device)
        if initial_state.dtype != torch.float32 or tuple(initial_state.shape) != (N, Hv, dk, dv):
            raise ValueError(f"initial_state must be float32 of shape {(N, Hv, dk, dv)}")
        h0p = initial_state.data_ptr()
    p = Problem(B, T, Hq, Hv, dk, dv, int(chunk_size), n, _kv_dtype(k))
    o_out = _out(o_out, (B, T, Hv, dv), k.dtype, device, "o_out")
    if final_state is None and output_final_state:
        final_state = torch.empty((N, Hv, dk, dv), dtype=torch.float32, device=device)
    elif final_state is not None:
        final_state = _out(final_state, (N, Hv, dk, dv), torch.float32, device, "final_state")
    sc = float(dk ** -0.5 if scale is None else scale)
    fsp = final_state.data_ptr() if final_state is not None else None
    cup = cu_seqlens.data_ptr() if cu_seqlens is not None else None
    if segment_chunks == "auto":
        segment_chunks = auto_segment_chunks(B, T, Hv, chunk_size,
                                             None if cu_seqlens is None else n)
    if segment_chunks is not None:
        nbytes = lib.wyp_chunk_fwd_cp_workspace_bytes(ctypes.byref(p), cup, int(segment_chunks))
        if nbytes < 0:
            raise ValueError(f"invalid segment_chunks {segment_chunks}")
        ws = torch.empty(max(nbytes, 16) // 4, dtype=torch.float32, device=device)
        st = lib.wyp_chunk_fwd_cp(ctypes.byref(p), q.data_ptr(), k.data_ptr(), w.data_ptr(),
                                  u.data_ptr(), gp, h0p, sc, cup, int(segment_chunks),
                                  ws.data_ptr(), nbytes, o_out.data_ptr(), fsp, _stream(device))
    else:
        st = lib.wyp_chunk_fwd(ctypes.byref(p), q.data_ptr(), k.data_ptr(), w.data_ptr(),
                               u.data_ptr(), gp, h0p, sc, cup, o_out.data_ptr(), fsp,
                               _stream(device))
    _check(lib, st)
    return o_out, final_state


def chunk_gated_delta_rule(q, k, v, g, beta, scale=None, initial_state=None,
                           output_final_state=False, cu_seqlens=None, chunk_size=64):
    """The gated DeltaNet chunked forward with the argument list of the FlashQLA usage section:
    wu_prepare (W, U for every chunk; T stays on chip) followed by chunk_fwd, which splits each
    sequence into segments run in parallel where sequences x heads would leave CUs idle
    (auto_segment_chunks; batch rows and packed sequences alike).  g may be None (no gates).
    Returns (o, final_state); final_state is None unless output_final_state."""
    w, u = wu_prepare(k, v, beta, chunk_size, cu_seqlens=cu_seqlens, g=g)
    # in-GPU sequence parallelism when sequences x heads is small
    return chunk_fwd(q, k, w, u, chunk_size, g=g, initial_state=initial_state, scale=scale,
                     cu_seqlens=cu_seqlens, output_final_state=output_final_state,
                     segment_chunks="auto")


# The C-ABI names, for callers that mirror the header.
wyp_kkt_solve = kkt_solve
wyp_wy_prepare = wy_prepare
wyp_wu_prepare = wu_prepare
wyp_solve_rhs = solve_rhs
wyp_chunk_fwd = chunk_fwd
wyp_wy_backward = wy_backward
