"""fp64 CPU oracle for the per-chunk WY/UT preparation of chunkwise (Gated) DeltaNet.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline
leg of ``bench.py`` may import this package.  It shares no code with the HIP path in
``chunkwise_gated_deltanet_amd`` and never imports it.

The arithmetic lives in plain C (``wyo_oracle.c``, IEEE double, plain loops); this module only
builds that file with gcc and marshals numpy arrays through ctypes.

Pages cited: "TileLang 实战：单位下三角矩阵求逆" (TileLang in practice: inverting a unit
lower-triangular matrix), sections 1 and 2; the FlashQLA announcement, section "使用方式"
(usage) for the tensor shapes.

Parity status of each function (what pins it is listed in tests/test_oracle_pins.py):
  row_forward_inverse        pinned (closed forms, LAPACK inverse, residuals, FMA counts)
  block_recursive_inverse    pinned (agrees with the row-wise inverse; FMA / depth counts)
  wy_prepare / units         pinned (Householder-product and delta-rule identities, closed
                             forms, degenerate cases, tail padding)
  solve_rhs                  pinned (residual A X = diag(beta) R against numpy's A, the
                             delta rule from a zero state with R = V, orthogonal keys, beta = 0,
                             agreement with the separately pinned T diag(beta) R)
  the same with gates g      pinned (gated delta-rule recurrence from zero and from an
                             identity state, the 2-token closed form, g = 0 against no gates,
                             Gamma o T_ungated, chunk restarts)
  wy_backward                pinned (central finite differences of <dT,T> + <dW,W> + <dU,U>
                             on a grid where every perturbation is exact; zero upstream;
                             g = 0 against no gates)
  gdn_forward                pinned (delta-rule read-back, beta = 0 decay of h0, orthogonal
                             keys = linear attention, the chunk form through the pinned W / U,
                             sequences independent)
  head grouping (v-head h reads k-head h // (Hv/Hq)) and the T layout [B,T,Hv,C]:
                             parity unpinned -- a stated convention, not fixed by the pages.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")
SOURCES = [os.path.join(_HERE, "wyo_oracle.c")]

BF16, F32 = 0, 1


def build(out_path: str = LIB_PATH, sources=None, extra_flags=()) -> str:
    """Compile the oracle with gcc (no fast-math, no FMA contraction)."""
    srcs = list(sources or SOURCES)
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
           "-Wall", "-Wextra", "-I", _HERE, *extra_flags, *srcs, "-o", out_path + ".tmp",
           "-lpthread", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out_path + ".tmp", out_path)
    return out_path


class Problem(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "batch", "seqlen", "num_qk_heads", "num_v_heads", "head_dim_k", "head_dim_v",
        "chunk_size", "num_seqs", "kv_dtype")]


_P = ctypes.c_void_p


def _bind(lib):
    lib.wyo_count_chunks.restype = ctypes.c_int64
    lib.wyo_count_chunks.argtypes = [ctypes.POINTER(Problem), _P]
    lib.wyo_list_chunks.restype = ctypes.c_int64
    lib.wyo_list_chunks.argtypes = [ctypes.POINTER(Problem), _P, _P, _P, ctypes.c_int64]
    lib.wyo_row_forward_inverse.restype = ctypes.c_int64
    lib.wyo_row_forward_inverse.argtypes = [ctypes.c_int32, _P, ctypes.c_int32, _P,
                                            ctypes.c_int32]
    lib.wyo_block_recursive_inverse.restype = ctypes.c_int64
    lib.wyo_block_recursive_inverse.argtypes = [ctypes.c_int32, ctypes.c_int32, _P,
                                                ctypes.c_int32, _P, ctypes.c_int32, _P]
    lib.wyo_wy_prepare.restype = ctypes.c_int32
    lib.wyo_wy_prepare.argtypes = [ctypes.POINTER(Problem), _P, _P, _P, _P, _P, _P, _P, _P,
                                   ctypes.c_int32, _P]
    lib.wyo_gdn_forward.restype = ctypes.c_int32
    lib.wyo_gdn_forward.argtypes = [ctypes.POINTER(Problem), _P, _P, _P, _P, _P, _P,
                                    ctypes.c_double, _P, _P, _P, _P, ctypes.c_int32]
    lib.wyo_wy_backward.restype = ctypes.c_int32
    lib.wyo_wy_backward.argtypes = [ctypes.POINTER(Problem), _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                    _P, _P, _P, ctypes.c_int32]
    lib.wyo_solve_rhs.restype = ctypes.c_int32
    lib.wyo_solve_rhs.argtypes = [ctypes.POINTER(Problem), _P, _P, _P, _P, _P, _P, ctypes.c_int32]
    lib.wyo_units.restype = ctypes.c_int32
    lib.wyo_units.argtypes = [ctypes.POINTER(Problem), _P, _P, _P, _P, ctypes.c_int64, _P, _P,
                              _P, _P, _P, _P, ctypes.c_int32]
    return lib


_LIB = None


def default_threads() -> int:
    """Worker threads when none are given: the usable host cores, at most 16 (the CPU share
    of one GPU on a GPU machine)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def load(path: str | None = None):
    """Load the oracle library (building it first if it is missing)."""
    global _LIB
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            build()
        _LIB = _bind(ctypes.CDLL(LIB_PATH))
    return _LIB


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _problem(k, v, beta, chunk_size, cu_seqlens):
    if k.dtype == np.uint16:
        dt = BF16
    elif k.dtype == np.float32:
        dt = F32
    else:
        raise TypeError("k must hold bf16 bit patterns (uint16) or float32")
    B, T, Hq, dk = k.shape
    Hv = beta.shape[2]
    dv = v.shape[3] if v is not None else dk
    if v is not None and v.dtype != k.dtype:
        raise TypeError("v and k must share a dtype")
    n = 0 if cu_seqlens is None else len(cu_seqlens) - 1
    return Problem(B, T, Hq, Hv, dk, dv, chunk_size, n, dt)


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def _gate(g, beta):
    """Log gates g [B,T,Hv] float32 (log alpha per token and value head) or None."""
    if g is None:
        return None
    g = np.ascontiguousarray(g, dtype=np.float32)
    if g.shape != beta.shape:
        raise ValueError(f"g shape {g.shape} must match beta {beta.shape}")
    return g


def list_chunks(batch, seqlen, chunk_size, cu_seqlens=None, lib=None):
    """(chunk_start[int64], chunk_len[int32]) in sequence order."""
    lib = lib or load()
    cu = _c(cu_seqlens, np.int32)
    p = Problem(batch, seqlen, 1, 1, 1, 1, chunk_size, 0 if cu is None else len(cu) - 1, BF16)
    n = lib.wyo_count_chunks(ctypes.byref(p), _ptr(cu))
    if n < 0:
        raise ValueError("invalid chunking arguments")
    start = np.zeros(max(n, 1), np.int64)
    length = np.zeros(max(n, 1), np.int32)
    lib.wyo_list_chunks(ctypes.byref(p), _ptr(cu), _ptr(start), _ptr(length), n)
    return start[:n], length[:n]


def row_forward_inverse(L, lib=None):
    """X = L^{-1} (unit lower triangular; strict lower part of L read).  Returns (X, fma)."""
    lib = lib or load()
    L = np.ascontiguousarray(L, dtype=np.float64)
    n = L.shape[0]
    X = np.zeros_like(L)
    fma = lib.wyo_row_forward_inverse(n, _ptr(L), n, _ptr(X), n)
    return X, int(fma)


def block_recursive_inverse(L, base=16, lib=None):
    """Recursive 2x2-block inverse.  Returns (X, fma, depth)."""
    lib = lib or load()
    L = np.ascontiguousarray(L, dtype=np.float64)
    n = L.shape[0]
    X = np.zeros_like(L)
    depth = ctypes.c_int32(0)
    fma = lib.wyo_block_recursive_inverse(n, base, _ptr(L), n, _ptr(X), n, ctypes.byref(depth))
    return X, int(fma), int(depth.value)


def wy_prepare(k, beta, chunk_size, v=None, cu_seqlens=None, nthreads=None, lib=None,
               want_wu=True, g=None):
    """Whole-tensor oracle.

    k: [B,T,Hq,dk] uint16 (bf16 bits) or float32; v: [B,T,Hv,dv] same dtype; beta: [B,T,Hv]
    float32; cu_seqlens: int32 [N+1] or None; g: [B,T,Hv] float32 log gates or None (no
    gates).  Returns (T, W, U, fma) as float64 arrays T [B,T,Hv,C], W [B,T,Hv,dk],
    U [B,T,Hv,dv] (W, U None when v is None or not want_wu).
    """
    lib = lib or load()
    k = np.ascontiguousarray(k)
    beta = _c(beta, np.float32)
    g = _gate(g, beta)
    cu = _c(cu_seqlens, np.int32)
    p = _problem(k, v, beta, chunk_size, cu)
    B, T, Hq, dk = k.shape
    Hv = beta.shape[2]
    Tm = np.zeros((B, T, Hv, chunk_size), np.float64)
    W = U = None
    if v is not None and want_wu:
        v = np.ascontiguousarray(v)
        W = np.zeros((B, T, Hv, dk), np.float64)
        U = np.zeros((B, T, Hv, v.shape[3]), np.float64)
    fma = ctypes.c_int64(0)
    rc = lib.wyo_wy_prepare(ctypes.byref(p), _ptr(k), _ptr(v if W is not None else None),
                            _ptr(g), _ptr(beta), _ptr(cu), _ptr(Tm), _ptr(W), _ptr(U),
                            nthreads or default_threads(), ctypes.byref(fma))
    if rc != 0:
        raise ValueError(f"oracle rejected the problem (code {rc})")
    return Tm, W, U, int(fma.value)


def solve_rhs(k, rhs, beta, chunk_size, cu_seqlens=None, g=None, nthreads=None, lib=None):
    """X = A^{-1} diag(beta) R per chunk and value head by forward substitution on the right-hand
    side (T never formed); rhs [B,T,Hv,dv] with k's dtype.  Returns X [B,T,Hv,dv] float64."""
    lib = lib or load()
    k = np.ascontiguousarray(k)
    rhs = np.ascontiguousarray(rhs)
    beta = _c(beta, np.float32)
    g = _gate(g, beta)
    cu = _c(cu_seqlens, np.int32)
    p = _problem(k, rhs, beta, chunk_size, cu)
    X = np.zeros(rhs.shape, np.float64)
    rc = lib.wyo_solve_rhs(ctypes.byref(p), _ptr(k), _ptr(rhs), _ptr(g), _ptr(beta), _ptr(cu),
                           _ptr(X), nthreads or default_threads())
    if rc != 0:
        raise ValueError(f"oracle rejected the problem (code {rc})")
    return X


def units(k, beta, chunk_size, chunk_start, chunk_len, v_head, v=None, nthreads=None, lib=None,
          g=None):
    """Selected units (compact outputs): T [M,C,C], W [M,C,dk], U [M,C,dv], zero-padded rows."""
    lib = lib or load()
    k = np.ascontiguousarray(k)
    beta = _c(beta, np.float32)
    g = _gate(g, beta)
    p = _problem(k, v, beta, chunk_size, None)
    cs = _c(chunk_start, np.int64)
    cl = _c(chunk_len, np.int32)
    vh = _c(v_head, np.int32)
    M = len(cs)
    C = chunk_size
    dk = k.shape[3]
    Tm = np.zeros((M, C, C), np.float64)
    W = U = None
    if v is not None:
        v = np.ascontiguousarray(v)
        W = np.zeros((M, C, dk), np.float64)
        U = np.zeros((M, C, v.shape[3]), np.float64)
    rc = lib.wyo_units(ctypes.byref(p), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), M, _ptr(cs), _ptr(cl),
                       _ptr(vh), _ptr(Tm), _ptr(W), _ptr(U), nthreads or default_threads())
    if rc != 0:
        raise ValueError(f"oracle rejected the units (code {rc})")
    return Tm, W, U


def gdn_forward(q, k, v, beta, g=None, h0=None, scale=None, cu_seqlens=None, pairs=None,
                nthreads=None, lib=None):
    """The gated delta rule token by token (fp64): returns (o [B,T,Hv,dv], hT [N,Hv,dk,dv]).

    q, k: [B,T,Hq,dk] uint16 (bf16 bits) or float32; v: [B,T,Hv,dv]; beta, g: [B,T,Hv]
    float32 (g None: alpha = 1); h0: [N,Hv,dk,dv] float32 or None (zeros); scale defaults to
    dk ** -0.5; pairs: optional iterable of (seq, value head) to compute (others stay 0).
    """
    lib = lib or load()
    k = np.ascontiguousarray(k)
    q = np.ascontiguousarray(q)
    v = np.ascontiguousarray(v)
    if q.dtype != k.dtype or q.shape != k.shape:
        raise ValueError("q must match k in shape and dtype")
    beta = _c(beta, np.float32)
    g = _gate(g, beta)
    cu = _c(cu_seqlens, np.int32)
    p = _problem(k, v, beta, 64, cu)
    B, T, Hq, dk = k.shape
    Hv, dv = beta.shape[2], v.shape[3]
    N = B if cu is None else len(cu) - 1
    if h0 is not None:
        h0 = np.ascontiguousarray(h0, dtype=np.float32)
        if h0.shape != (N, Hv, dk, dv):
            raise ValueError(f"h0 must be {(N, Hv, dk, dv)}")
    mask = None
    if pairs is not None:
        mask = np.zeros(N * Hv, np.uint8)
        for s, h in pairs:
            mask[int(s) * Hv + int(h)] = 1
    o = np.zeros((B, T, Hv, dv), np.float64)
    hT = np.zeros((N, Hv, dk, dv), np.float64)
    rc = lib.wyo_gdn_forward(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                             _ptr(h0), float(dk ** -0.5 if scale is None else scale), _ptr(cu),
                             _ptr(o), _ptr(hT), _ptr(mask), nthreads or default_threads())
    if rc != 0:
        raise ValueError(f"oracle rejected the problem (code {rc})")
    return o, hT


def wy_backward(k, v, beta, chunk_size, dW, dU, dT=None, g=None, cu_seqlens=None, nthreads=None,
                lib=None):
    """Gradient of <dT,T> + <dW,W> + <dU,U> with respect to k, v, beta, g (fp64).

    k [B,T,Hq,dk], v [B,T,Hv,dv], dW [B,T,Hv,dk], dU [B,T,Hv,dv]: uint16 (bf16 bits) or float32,
    all of one dtype; beta, g [B,T,Hv] float32 (g None: no gates); dT [B,T,Hv,C] float32 or
    None.  Returns (dk [B,T,Hq,dk], dv, dbeta [B,T,Hv], dg or None).
    """
    lib = lib or load()
    k, v = np.ascontiguousarray(k), np.ascontiguousarray(v)
    dW, dU = np.ascontiguousarray(dW), np.ascontiguousarray(dU)
    if not (k.dtype == v.dtype == dW.dtype == dU.dtype):
        raise TypeError("k, v, dW, dU must share a dtype")
    beta = _c(beta, np.float32)
    g = _gate(g, beta)
    cu = _c(cu_seqlens, np.int32)
    p = _problem(k, v, beta, chunk_size, cu)
    B, T, Hq, dk = k.shape
    Hv, dv = beta.shape[2], v.shape[3]
    if dW.shape != (B, T, Hv, dk) or dU.shape != (B, T, Hv, dv):
        raise ValueError("dW / dU shapes do not match")
    if dT is not None:
        dT = np.ascontiguousarray(dT, dtype=np.float32)
        if dT.shape != (B, T, Hv, chunk_size):
            raise ValueError("dT shape does not match")
    dko = np.zeros((B, T, Hq, dk))
    dvo = np.zeros((B, T, Hv, dv))
    dbo = np.zeros((B, T, Hv))
    dgo = np.zeros((B, T, Hv)) if g is not None else None
    rc = lib.wyo_wy_backward(ctypes.byref(p), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(cu),
                             _ptr(dT), _ptr(dW), _ptr(dU), _ptr(dko), _ptr(dvo), _ptr(dbo),
                             _ptr(dgo), nthreads or default_threads())
    if rc != 0:
        raise ValueError(f"oracle rejected the problem (code {rc})")
    return dko, dvo, dbo, dgo
