"""Pins of the fp64 oracle against what the pages and the mathematics fix (CPU only).

Pages: "TileLang 实战：单位下三角矩阵求逆" (cited [Inv]) and the FlashQLA announcement.

Each pin_* function raises AssertionError when the oracle library it is given is wrong.  The
same pins run against deliberately broken copies of the oracle (test_mutants_are_caught), so a
dropped term, a wrong sign or index, or a transposed operand anywhere in it fails at least one.
"""
import math
import os
import shutil

import numpy as np
import pytest

import oracle
from chunkwise_gated_deltanet_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------------------------------------
# helpers (test side: plain numpy statements of the definitions, used only as cross-checks)

def unit_keys(rng, n, dk=128):
    k = rng.standard_normal((n, dk)).astype(np.float32)
    return (k / np.linalg.norm(k, axis=1, keepdims=True)).astype(np.float32)


def one_unit(lib, K, V, beta, C=None, g=None):
    """Runs the oracle on one chunk [0, n) of a single-head problem (fp32 inputs; g: optional
    log gates of the n tokens)."""
    n = K.shape[0]
    C = C or n
    k = np.ascontiguousarray(K[None, :, None, :], np.float32)
    v = np.ascontiguousarray(V[None, :, None, :], np.float32)
    b = np.ascontiguousarray(beta[None, :, None], np.float32)
    gg = None if g is None else np.ascontiguousarray(g[None, :, None], np.float32)
    T, W, U = oracle.units(k, b, C, [0], [n], [0], v=v, lib=lib, nthreads=1, g=gg)
    return T[0, :n, :n], W[0, :n], U[0, :n]


def a_matrix(K, beta):
    """A = I + strictLower(diag(beta) K K^T) in fp64 ([Inv] section 1)."""
    K = K.astype(np.float64)
    G = K @ K.T
    return np.eye(len(K)) + np.tril(beta.astype(np.float64)[:, None] * G, -1)


def read_table(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


# ---------------------------------------------------------------------------------------------
# pins

def pin_closed_form_2(lib):
    """C = 2: A = [[1,0],[b1 k1.k0, 1]] so T = [[1,0],[-b1 k1.k0, 1]] (2x2 inverse)."""
    rng = np.random.default_rng(11)
    K = unit_keys(rng, 2)
    V = rng.standard_normal((2, 128)).astype(np.float32)
    beta = np.array([0.3, 0.8], np.float32)
    T, W, U = one_unit(lib, K, V, beta)
    K64, V64, b = K.astype(np.float64), V.astype(np.float64), beta.astype(np.float64)
    g = float(K64[1] @ K64[0])
    assert T[0, 0] == 1 and T[1, 1] == 1 and T[0, 1] == 0
    assert abs(T[1, 0] - (-b[1] * g)) <= 1e-15
    W_exp = np.stack([b[0] * K64[0], -b[1] * g * b[0] * K64[0] + b[1] * K64[1]])
    U_exp = np.stack([b[0] * V64[0], -b[1] * g * b[0] * V64[0] + b[1] * V64[1]])
    assert np.max(np.abs(W - W_exp)) <= 1e-14
    assert np.max(np.abs(U - U_exp)) <= 1e-14


def pin_orthogonal(lib):
    """Distinct one-hot keys: K K^T = I so A = I, T = I, W = diag(b) K, U = diag(b) V exactly."""
    rng = np.random.default_rng(12)
    n = 32
    K = np.zeros((n, 128), np.float32)
    K[np.arange(n), rng.permutation(128)[:n]] = 1.0
    V = rng.standard_normal((n, 128)).astype(np.float32)
    beta = rng.uniform(0.05, 0.95, n).astype(np.float32)
    T, W, U = one_unit(lib, K, V, beta)
    b = beta.astype(np.float64)[:, None]
    assert np.array_equal(T, np.eye(n))
    assert np.array_equal(W, b * K.astype(np.float64))
    assert np.array_equal(U, b * V.astype(np.float64))


def pin_residual_structure(lib):
    """T A = A T = I to 1e-12; unit diagonal and zero strict upper triangle exactly."""
    rng = np.random.default_rng(13)
    for n in (32, 64, 128):
        K = unit_keys(rng, n)
        V = rng.standard_normal((n, 128)).astype(np.float32)
        beta = (1 / (1 + np.exp(-rng.standard_normal(n)))).astype(np.float32)
        T, _, _ = one_unit(lib, K, V, beta)
        A = a_matrix(K, beta)
        assert np.max(np.abs(T @ A - np.eye(n))) <= 1e-12
        assert np.max(np.abs(A @ T - np.eye(n))) <= 1e-12
        assert np.all(np.diag(T) == 1.0)
        assert np.all(np.triu(T, 1) == 0.0)


def pin_lapack_inverse(lib):
    """Brute force: LAPACK's dense inverse of A (np.linalg.inv) within 1e-12."""
    rng = np.random.default_rng(14)
    for n in (2, 5, 16, 17, 32, 64, 128):
        K = unit_keys(rng, n)
        V = rng.standard_normal((n, 128)).astype(np.float32)
        beta = rng.uniform(0.0, 1.0, n).astype(np.float32)
        T, _, _ = one_unit(lib, K, V, beta)
        assert np.max(np.abs(T - np.linalg.inv(a_matrix(K, beta)))) <= 1e-12


def pin_block_identity(lib):
    """[Inv] section 2.2: lower-left of L^{-1} is -L11^{-1} L10 L00^{-1}; the recursive and the
    row-wise inverses agree; block residual L10 X00 + L11 X10 = 0."""
    rng = np.random.default_rng(15)
    for n in (32, 64, 128):
        K = unit_keys(rng, n)
        beta = rng.uniform(0.0, 1.0, n).astype(np.float32)
        A = a_matrix(K, beta)
        X, _ = oracle.row_forward_inverse(A, lib=lib)
        Xr, _, _ = oracle.block_recursive_inverse(A, 16, lib=lib)
        assert np.max(np.abs(X - Xr)) <= 1e-12
        h = n // 2
        X00, X11, X10 = X[:h, :h], X[h:, h:], X[h:, :h]
        L10, L11 = A[h:, :h], A[h:, h:]
        assert np.max(np.abs(X10 - (-X11 @ L10 @ X00))) <= 1e-12
        assert np.max(np.abs(L10 @ X00 + L11 @ X10)) <= 1e-12
        assert np.all(X[:h, h:] == 0)


def pin_beta_zero(lib):
    """[Inv] section 4, degenerate check 1: beta -> 0 gives T = I (and W = U = 0)."""
    rng = np.random.default_rng(16)
    for n in (32, 64, 128):
        K = unit_keys(rng, n)
        V = rng.standard_normal((n, 128)).astype(np.float32)
        T, W, U = one_unit(lib, K, V, np.zeros(n, np.float32))
        assert np.array_equal(T, np.eye(n))
        assert np.all(W == 0) and np.all(U == 0)


def subdiag_keys(n, half):
    """Keys making A's two diagonal half-blocks the identity while the lower-left block is not:
    rows i < half are e_i; rows half + i are c (e_i + e_{half+i}) with c = 1/sqrt(2) in fp32."""
    c = np.float32(1 / math.sqrt(2))
    K = np.zeros((n, 128), np.float32)
    for i in range(half):
        K[i, i] = 1
        K[half + i, i] = c
        K[half + i, half + i] = c
    return K


def pin_subdiag_only(lib):
    """[Inv] section 4, degenerate check 2: with L00 = L11 = I the lower-left of T is exactly
    -L10 (checks the sign of the coupling on its own)."""
    rng = np.random.default_rng(17)
    for n in (32, 64, 128):
        h = n // 2
        K = subdiag_keys(n, h)
        V = rng.standard_normal((n, 128)).astype(np.float32)
        beta = rng.uniform(0.05, 0.95, n).astype(np.float32)
        T, _, _ = one_unit(lib, K, V, beta)
        A = a_matrix(K, beta)
        assert np.array_equal(A[:h, :h], np.eye(h)) and np.array_equal(A[h:, h:], np.eye(h))
        assert np.any(A[h:, :h] != 0)
        assert np.array_equal(T[h:, :h], -A[h:, :h])
        assert np.array_equal(T[:h, :h], np.eye(h)) and np.array_equal(T[h:, h:], np.eye(h))


def pin_identical_keys(lib):
    """All keys equal (k.k = s): A[i,j] = s b_i for i > j, and
    T[i,j] = -s b_i prod_{m=j+1}^{i-1} (1 - s b_m)  (derived from [Inv] section 1 by
    eliminating row i with row i-1)."""
    rng = np.random.default_rng(18)
    for n in (32, 64):
        k = unit_keys(rng, 1)[0]
        K = np.repeat(k[None, :], n, axis=0)
        V = rng.standard_normal((n, 128)).astype(np.float32)
        beta = rng.uniform(0.0, 1.0, n).astype(np.float32)
        T, _, _ = one_unit(lib, K, V, beta)
        s = float(k.astype(np.float64) @ k.astype(np.float64))
        b = beta.astype(np.float64)
        E = np.eye(n)
        for i in range(n):
            for j in range(i):
                E[i, j] = -s * b[i] * np.prod(1 - s * b[j + 1:i])
        assert np.max(np.abs(T - E)) <= 1e-13


def pin_fma_counts(lib):
    """Necessary multiply-adds and depths printed in [Inv] sections 2.2-2.4."""
    rng = np.random.default_rng(19)
    for n in range(1, 131):
        L = np.tril(rng.uniform(-0.3, 0.3, (n, n)), -1) + np.eye(n)
        _, fma = oracle.row_forward_inverse(L, lib=lib)
        assert fma == n * (n - 1) * (n - 2) // 6, n
    for C, row_fma, rec_fma, rec_depth, row_depth, per_tok in read_table("fma_counts.txt"):
        C = int(C)
        L = np.tril(rng.uniform(-0.3, 0.3, (C, C)), -1) + np.eye(C)
        _, fma = oracle.row_forward_inverse(L, lib=lib)
        if row_fma != "-":
            assert fma == int(row_fma)
        _, rfma, depth = oracle.block_recursive_inverse(L, 16, lib=lib)
        assert rfma == int(rec_fma) and depth == int(rec_depth)
        assert C - 1 == int(row_depth)
        assert round(rfma / C) == int(per_tok)
    # the whole-tensor oracle reports the sum of C(n,3) over its units
    inp = synth.custom(1, 0, 1, 2, 32, dtype="f32", seed=3, seqlens=[40, 17, 64])
    _, _, _, fma = oracle.wy_prepare(inp["k"], inp["beta"], 32, v=inp["v"],
                                     cu_seqlens=inp["cu_seqlens"], lib=lib, nthreads=2)
    expect = 2 * sum(n * (n - 1) * (n - 2) // 6 for n in (32, 8, 17, 32, 32))
    assert fma == expect


def pin_householder_product(lib):
    """W pins: prod_{t=1..n} (I - b_t k_t k_t^T), t = 1 leftmost, equals I - W^T K -- the
    product of the chunk's Householder-like transforms that the UT transform arranges into the
    triangular system ([Inv] section 1)."""
    rng = np.random.default_rng(20)
    for n in (32, 37, 64, 128):
        K = unit_keys(rng, n)
        V = rng.standard_normal((n, 128)).astype(np.float32)
        beta = rng.uniform(0.0, 1.0, n).astype(np.float32)
        _, W, _ = one_unit(lib, K, V, beta)
        K64 = K.astype(np.float64)
        P = np.eye(128)
        for t in range(n):
            P = P @ (np.eye(128) - float(beta[t]) * np.outer(K64[t], K64[t]))
        assert np.max(np.abs(P - (np.eye(128) - W.T @ K64))) <= 1e-12


def pin_delta_rule(lib):
    """U pins: the delta rule S_t = S_{t-1}(I - b_t k_t k_t^T) + b_t v_t k_t^T from S_0 = 0 ends
    at S_n = U^T K (the chunk's contribution that U carries)."""
    rng = np.random.default_rng(21)
    for n in (32, 45, 64):
        K = unit_keys(rng, n)
        V = rng.standard_normal((n, 128)).astype(np.float32)
        beta = rng.uniform(0.0, 1.0, n).astype(np.float32)
        _, _, U = one_unit(lib, K, V, beta)
        K64, V64 = K.astype(np.float64), V.astype(np.float64)
        S = np.zeros((128, 128))
        for t in range(n):
            b = float(beta[t])
            S = S @ (np.eye(128) - b * np.outer(K64[t], K64[t])) + b * np.outer(V64[t], K64[t])
        assert np.max(np.abs(S - U.T @ K64)) <= 1e-12


def pin_tail_padding(lib):
    """A short chunk (n < C) equals the top-left of the zero-padded chunk with beta = 0 on the
    padding: A = blockdiag(A_n, I) gives T = blockdiag(T_n, I)."""
    rng = np.random.default_rng(22)
    n, C = 37, 64
    K = unit_keys(rng, C)
    V = rng.standard_normal((C, 128)).astype(np.float32)
    beta = rng.uniform(0.0, 1.0, C).astype(np.float32)
    K[n:] = 0
    beta[n:] = 0
    Tn, Wn, Un = one_unit(lib, K[:n], V[:n], beta[:n], C=C)
    Tp, Wp, Up = one_unit(lib, K, V, beta)
    assert np.array_equal(Tp[:n, :n], Tn)
    assert np.array_equal(Tp[n:, n:], np.eye(C - n)) and np.all(Tp[n:, :n] == 0)
    assert np.array_equal(Wp[:n], Wn) and np.array_equal(Up[:n], Un)


def pin_layout(lib):
    """Whole-tensor scatter: row t of T_out / W_out / U_out holds row (t - chunk start) of its
    chunk's T / W / U, with chunk-relative columns; packed chunks restart at sequence starts."""
    inp = synth.custom(1, 0, 2, 4, 32, dtype="bf16", seed=4, seqlens=[70, 5, 33])
    k, v, beta, cu = inp["k"], inp["v"], inp["beta"], inp["cu_seqlens"]
    T, W, U, _ = oracle.wy_prepare(k, beta, 32, v=v, cu_seqlens=cu, lib=lib, nthreads=3)
    starts, lens = oracle.list_chunks(1, int(cu[-1]), 32, cu, lib=lib)
    assert list(starts) == [0, 32, 64, 70, 75, 107] and list(lens) == [32, 32, 6, 5, 32, 1]
    for c in range(len(starts)):
        for h in range(4):
            Tu, Wu, Uu = oracle.units(k, beta, 32, [starts[c]], [lens[c]], [h], v=v, lib=lib)
            rows = slice(starts[c], starts[c] + lens[c])
            assert np.array_equal(T[0, rows, h], Tu[0, :lens[c]])
            assert np.array_equal(W[0, rows, h], Wu[0, :lens[c]])
            assert np.array_equal(U[0, rows, h], Uu[0, :lens[c]])
            assert np.all(T[0, rows, h, lens[c]:] == 0)


def pin_head_grouping(lib):
    """Value head h reads key head h // (Hv/Hq) (contiguous groups; the pages fix only the
    shapes, so this is a stated convention)."""
    inp = synth.custom(1, 64, 2, 4, 64, dtype="f32", seed=5)
    k, v, beta = inp["k"], inp["v"], inp["beta"]
    # value head 2 of 4 with 2 key heads reads key head 1 (2 // 2), not key head 0 (2 % 2)
    T, W, U = oracle.units(k, beta, 64, [0], [64], [2], v=v, lib=lib)
    k1 = np.ascontiguousarray(k[:, :, 1:2])
    T1, W1, U1 = oracle.units(k1, np.ascontiguousarray(beta[:, :, 2:3]), 64, [0], [64], [0],
                              v=np.ascontiguousarray(v[:, :, 2:3]), lib=lib)
    assert np.array_equal(T, T1) and np.array_equal(W, W1) and np.array_equal(U, U1)


# ---------------------------------------------------------------------------------------------
# gated pins.  [Inv] section 5 item 12 gives the gated coefficient diag(beta)(Gamma o K K^T);
# g [B,T,Hv] is the per-token log gate of [QLA] usage, alpha_t = exp(g_t) in (0, 1) the decay
# of the GDN recurrence the FlashQLA page recalls.  Reading: G_i = g_0 + ... + g_i within the
# chunk, Gamma[i][j] = exp(G_i - G_j).  The W / U forms are fixed here by the gated delta rule
# itself, stepped token by token (S_t = S_{t-1} alpha_t (I - b_t k_t k_t^T) + b_t v_t k_t^T).

def unit_gates(rng, n, mu=2.0):
    """Log gates with real decay: log sigmoid(mu + N(0,1)), plus one alpha = 1 token."""
    y = rng.standard_normal(n)
    g = -np.logaddexp(0.0, -(mu + y))
    g[n // 3] = 0.0
    return g.astype(np.float32)


def pin_gate_zero(lib):
    """g = 0 everywhere (alpha = 1) is the ungated method, bit for bit."""
    rng = np.random.default_rng(30)
    for n in (17, 64):
        K = unit_keys(rng, n)
        V = rng.standard_normal((n, 128)).astype(np.float32)
        beta = rng.uniform(0.0, 1.0, n).astype(np.float32)
        T0, W0, U0 = one_unit(lib, K, V, beta)
        Tz, Wz, Uz = one_unit(lib, K, V, beta, g=np.zeros(n, np.float32))
        assert np.array_equal(T0, Tz) and np.array_equal(W0, Wz) and np.array_equal(U0, Uz)


def pin_gated_closed_form_2(lib):
    """Two tokens: A[1,0] = b1 exp(g1) k1.k0 (the decay from token 0 to token 1 is alpha_1), so
    T[1,0] = -b1 exp(g1) k1.k0; W rows b0 e^{g0} k0 and T[1,0] b0 e^{g0} k0 + b1 e^{g0+g1} k1;
    U rows b0 v0 and T[1,0] b0 v0 + b1 v1 (one step of the gated delta rule per row)."""
    rng = np.random.default_rng(31)
    K = unit_keys(rng, 2)
    V = rng.standard_normal((2, 128)).astype(np.float32)
    beta = np.array([0.3, 0.8], np.float32)
    g = np.array([-0.25, -0.6], np.float32)
    T, W, U = one_unit(lib, K, V, beta, g=g)
    K64, V64, b, g64 = K.astype(np.float64), V.astype(np.float64), beta.astype(np.float64), \
        g.astype(np.float64)
    t10 = -b[1] * math.exp(g64[1]) * float(K64[1] @ K64[0])
    assert T[0, 0] == 1 and T[1, 1] == 1 and T[0, 1] == 0
    assert abs(T[1, 0] - t10) <= 1e-15
    e0, e01 = math.exp(g64[0]), math.exp(g64[0] + g64[1])
    W_exp = np.stack([b[0] * e0 * K64[0], t10 * b[0] * e0 * K64[0] + b[1] * e01 * K64[1]])
    U_exp = np.stack([b[0] * V64[0], t10 * b[0] * V64[0] + b[1] * V64[1]])
    assert np.max(np.abs(W - W_exp)) <= 1e-14
    assert np.max(np.abs(U - U_exp)) <= 1e-14


def pin_gated_recurrence(lib):
    """The gated delta rule stepped token by token pins both outputs: from S_0 = 0 it ends at
    S_n = U^T diag(exp(G_n - G)) K, and its transition prod_t alpha_t (I - b_t k_t k_t^T)
    (t = 1 leftmost) equals exp(G_n) I - W^T diag(exp(G_n - G)) K."""
    rng = np.random.default_rng(32)
    for n, mu in ((32, 2.0), (45, 0.5), (64, 4.0), (128, 3.0)):
        K = unit_keys(rng, n)
        V = rng.standard_normal((n, 128)).astype(np.float32)
        beta = rng.uniform(0.0, 1.0, n).astype(np.float32)
        g = unit_gates(rng, n, mu)
        _, W, U = one_unit(lib, K, V, beta, g=g)
        K64, V64 = K.astype(np.float64), V.astype(np.float64)
        S = np.zeros((128, 128))
        P = np.eye(128)
        for t in range(n):
            a, b = math.exp(float(g[t])), float(beta[t])
            M = a * (np.eye(128) - b * np.outer(K64[t], K64[t]))
            S = S @ M + b * np.outer(V64[t], K64[t])
            P = P @ M
        G = np.cumsum(g.astype(np.float64))
        d = np.exp(G[-1] - G)[:, None]
        assert np.max(np.abs(S - U.T @ (d * K64))) <= 1e-12
        assert np.max(np.abs(P - (math.exp(G[-1]) * np.eye(128) - W.T @ (d * K64)))) <= 1e-12


def pin_gated_similarity(lib):
    """Gamma[i][j] = e^{G_i} / e^{G_j}, so the gated A is D A_0 D^{-1} with D = diag(exp(G)) and
    A_0 the ungated matrix: T = Gamma o T_0 entry by entry and W = D W_0 row by row (T_0, W_0
    from the ungated oracle on the same keys and beta)."""
    rng = np.random.default_rng(33)
    for n, mu in ((32, 1.0), (64, 3.0), (128, 4.0)):
        K = unit_keys(rng, n)
        V = rng.standard_normal((n, 128)).astype(np.float32)
        beta = rng.uniform(0.0, 1.0, n).astype(np.float32)
        g = unit_gates(rng, n, mu)
        T0, W0, _ = one_unit(lib, K, V, beta)
        T, W, _ = one_unit(lib, K, V, beta, g=g)
        G = np.cumsum(g.astype(np.float64))
        Gam = np.tril(np.exp(G[:, None] - G[None, :]))
        assert np.max(np.abs(T - Gam * T0)) <= 1e-13
        assert np.max(np.abs(W - np.exp(G)[:, None] * W0)) <= 1e-13


def pin_gated_chunk_restart(lib):
    """Gates restart at every chunk: the whole-tensor oracle's chunk c equals the one-unit
    oracle run on that chunk's tokens alone (packed sequences and a ragged tail included)."""
    inp = synth.custom(1, 0, 1, 2, 32, dtype="f32", seed=34, seqlens=[70, 33], gate_mu=1.0)
    k, v, beta, g, cu = inp["k"], inp["v"], inp["beta"], inp["g"], inp["cu_seqlens"]
    T, W, U, _ = oracle.wy_prepare(k, beta, 32, v=v, cu_seqlens=cu, lib=lib, nthreads=2, g=g)
    for t0, n in ((0, 32), (32, 32), (64, 6), (70, 32), (102, 1)):
        for h in range(2):
            Tu, Wu, Uu = one_unit(lib, k[0, t0:t0 + n, 0], v[0, t0:t0 + n, h],
                                  beta[0, t0:t0 + n, h], C=32, g=g[0, t0:t0 + n, h])
            assert np.array_equal(T[0, t0:t0 + n, h, :n], Tu)
            assert np.array_equal(W[0, t0:t0 + n, h], Wu)
            assert np.array_equal(U[0, t0:t0 + n, h], Uu)


# ---------------------------------------------------------------------------------------------
# the gated delta rule, token by token (oracle.gdn_forward): the recurrence the chunk step
# serves.  S_t = alpha_t (I - b_t k_t k_t^T) S_{t-1} + b_t k_t v_t^T, o_t = scale S_t^T q_t.

def seq_inputs(rng, T, Hq=1, Hv=1, dk=128, dv=128):
    k = rng.standard_normal((1, T, Hq, dk))
    k = (k / np.linalg.norm(k, axis=-1, keepdims=True)).astype(np.float32)
    q = rng.standard_normal((1, T, Hq, dk)).astype(np.float32)
    v = rng.standard_normal((1, T, Hv, dv)).astype(np.float32)
    beta = rng.uniform(0.0, 1.0, (1, T, Hv)).astype(np.float32)
    return q, k, v, beta


def pin_gdn_read_back(lib):
    """The delta rule stores v_t under key k_t: with beta_t = 1 and |k_t| = 1, reading the
    state with q_t = k_t right after token t's write returns exactly v_t."""
    rng = np.random.default_rng(40)
    _, k, v, _ = seq_inputs(rng, 50)
    k64 = k.astype(np.float64)
    k = (k64 / np.linalg.norm(k64, axis=-1, keepdims=True)).astype(np.float32)
    beta = np.ones((1, 50, 1), np.float32)
    o, _ = oracle.gdn_forward(k, k, v, beta, scale=0.5, lib=lib, nthreads=1)
    kk = np.sum(k.astype(np.float64) ** 2, axis=-1)  # |k|^2 in fp64 (1 up to fp32 rounding)
    # exact: S_t^T k_t = S'^T k_t (1 - |k|^2) + v_t |k|^2
    assert np.max(np.abs(o - 0.5 * v.astype(np.float64) * kk[..., None])) <= 1e-6
    assert np.max(np.abs(o - 0.5 * v)) <= 1e-5


def pin_gdn_beta_zero(lib):
    """beta = 0: nothing is written, the initial state only decays, S_t = exp(G_t) h0 with G the
    running sum of g over the whole sequence; o_t = scale exp(G_t) h0^T q_t.  A non-symmetric
    h0 fixes its layout [dk][dv]."""
    rng = np.random.default_rng(41)
    T, dk, dv = 40, 128, 64
    q, k, v, _ = seq_inputs(rng, T, dv=dv)
    beta = np.zeros((1, T, 1), np.float32)
    g = (-rng.uniform(0, 0.2, (1, T, 1))).astype(np.float32)
    h0 = rng.standard_normal((1, 1, dk, dv)).astype(np.float32)
    o, hT = oracle.gdn_forward(q, k, v, beta, g=g, h0=h0, scale=0.3, lib=lib, nthreads=1)
    G = np.cumsum(g[0, :, 0].astype(np.float64))
    H = h0[0, 0].astype(np.float64)
    expect = 0.3 * np.exp(G)[:, None] * (q[0, :, 0].astype(np.float64) @ H)
    assert np.max(np.abs(o[0, :, 0] - expect)) <= 1e-12
    assert np.max(np.abs(hT[0, 0] - math.exp(G[-1]) * H)) <= 1e-12


def pin_gdn_linear_attention(lib):
    """Orthonormal keys, no decay, zero initial state: every k_t^T S_{t-1} is 0, so the rule
    is plain linear attention, o_t = scale sum_{i <= t} b_i (q_t . k_i) v_i, and the final state
    is sum_i b_i k_i v_i^T."""
    rng = np.random.default_rng(42)
    T = 96
    q, _, v, beta = seq_inputs(rng, T)
    k = np.zeros((1, T, 1, 128), np.float32)
    k[0, np.arange(T), 0, rng.permutation(128)[:T]] = 1.0
    o, hT = oracle.gdn_forward(q, k, v, beta, scale=0.7, lib=lib, nthreads=1)
    Q, K, V = (a[0, :, 0].astype(np.float64) for a in (q, k, v))
    b = beta[0, :, 0].astype(np.float64)
    expect = 0.7 * np.tril(Q @ K.T) @ (b[:, None] * V)
    assert np.max(np.abs(o[0, :, 0] - expect)) <= 1e-12
    assert np.max(np.abs(hT[0, 0] - K.T @ (b[:, None] * V))) <= 1e-12


def pin_gdn_chunk_form(lib):
    """The recurrence agrees with its chunk form built from the (separately pinned) W and U:
    per chunk with start state S, V' = U - W S, o_i = scale (e^{G_i} q_i^T S +
    sum_{j <= i} Gamma[i][j] (q_i . k_j) V'_j) and the next state e^{G_n} S +
    K^T diag(e^{G_n - G}) V'.  Grouped value heads, gates, a nonzero initial state."""
    rng = np.random.default_rng(43)
    T, C, Hq, Hv = 150, 64, 2, 4
    q, k, v, beta = seq_inputs(rng, T, Hq=Hq, Hv=Hv)
    g = np.stack([unit_gates(rng, T, mu) for mu in (3.0, 1.0, 4.0, 2.0)], -1)[None]
    g = g.astype(np.float32)
    h0 = (0.3 * rng.standard_normal((1, Hv, 128, 128))).astype(np.float32)
    o, hT = oracle.gdn_forward(q, k, v, beta, g=g, h0=h0, scale=0.25, lib=lib, nthreads=2)
    for h in range(Hv):
        hk = h // (Hv // Hq)
        S = h0[0, h].astype(np.float64)
        for t0 in range(0, T, C):
            n = min(C, T - t0)
            sl = slice(t0, t0 + n)
            _, W, U = one_unit(lib, k[0, sl, hk], v[0, sl, h], beta[0, sl, h], C=C,
                               g=g[0, sl, h])
            Q, K = q[0, sl, hk].astype(np.float64), k[0, sl, hk].astype(np.float64)
            G = np.cumsum(g[0, sl, h].astype(np.float64))
            Vn = U - W @ S
            Gam = np.tril(np.exp(G[:, None] - G[None, :]))
            oc = 0.25 * (np.exp(G)[:, None] * (Q @ S) + (Gam * (Q @ K.T)) @ Vn)
            assert np.max(np.abs(o[0, sl, h] - oc)) <= 1e-11
            S = math.exp(G[-1]) * S + K.T @ (np.exp(G[-1] - G)[:, None] * Vn)
        assert np.max(np.abs(hT[0, h] - S)) <= 1e-11


def pin_gdn_sequences_independent(lib):
    """Packed sequences each start from their own initial state (zeros here): the packed run
    equals each sequence run alone."""
    rng = np.random.default_rng(44)
    lens = [37, 64, 5]
    q, k, v, beta = seq_inputs(rng, sum(lens))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    o, hT = oracle.gdn_forward(q, k, v, beta, cu_seqlens=cu, lib=lib, nthreads=1)
    for s in range(3):
        sl = slice(cu[s], cu[s + 1])
        o1, h1 = oracle.gdn_forward(q[:, sl], k[:, sl], v[:, sl], beta[:, sl], lib=lib, nthreads=1)
        assert np.array_equal(o[:, sl], o1) and np.array_equal(hT[s], h1[0])


# ---------------------------------------------------------------------------------------------
# backward of the preparation step: the gradient of <dT,T> + <dW,W> + <dU,U>

def grid(rng, shape, scale):
    """fp32 values on the 2^-12 grid, so x +- 2^-12 is exact in fp32."""
    return (np.round(rng.standard_normal(shape) * scale * 4096) / 4096).astype(np.float32)


def bwd_problem(seed, gated=True):
    rng = np.random.default_rng(seed)
    T, Hq, Hv, d, C = 11, 1, 2, 8, 8  # two chunks: 8 tokens and a ragged tail of 3
    k = grid(rng, (1, T, Hq, d), 0.4)
    v = grid(rng, (1, T, Hv, d), 1.0)
    beta = (np.round(rng.uniform(0.1, 0.9, (1, T, Hv)) * 4096) / 4096).astype(np.float32)
    g = grid(rng, (1, T, Hv), 0.2) - np.float32(0.125) if gated else None
    dT = rng.standard_normal((1, T, Hv, C)).astype(np.float32)
    dW = rng.standard_normal((1, T, Hv, d)).astype(np.float32)
    dU = rng.standard_normal((1, T, Hv, d)).astype(np.float32)
    return dict(k=k, v=v, beta=beta, g=g, dT=dT, dW=dW, dU=dU, C=C)


def bwd_loss(lib, P, k=None, v=None, beta=None, g=None):
    k = P["k"] if k is None else k
    v = P["v"] if v is None else v
    beta = P["beta"] if beta is None else beta
    g = P["g"] if g is None else g
    T, W, U, _ = oracle.wy_prepare(k, beta, P["C"], v=v, lib=lib, nthreads=1, g=g)
    # only entries of T left of or on the diagonal exist; the rest is 0 in T_out
    return float(np.sum(P["dT"] * T) + np.sum(P["dW"] * W) + np.sum(P["dU"] * U))


def pin_bwd_finite_differences(lib):
    """Every component of the analytic gradient (k, v, beta, g; a key head read by two value
    heads; two chunks with a ragged tail; gates; dT given) equals the central difference
    (L(x + h) - L(x - h)) / 2h with h = 2^-12, every perturbed input exact in fp32."""
    P = bwd_problem(50)
    dk, dv, db, dg = oracle.wy_backward(P["k"], P["v"], P["beta"], P["C"], P["dW"], P["dU"],
                                        dT=P["dT"], g=P["g"], lib=lib, nthreads=1)
    h = np.float32(2.0 ** -12)
    worst = 0.0
    for name, grad in (("k", dk), ("v", dv), ("beta", db), ("g", dg)):
        x = P[name]
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            fd = (bwd_loss(lib, P, **{name: xp}) - bwd_loss(lib, P, **{name: xm})) / (2 * float(h))
            worst = max(worst, abs(fd - grad[idx]) / max(1.0, abs(fd)))
    assert worst <= 1e-7, worst  # measured: 1e-11 (k, v, beta), 1e-8 (g: h^2 through exp)


def pin_bwd_zero_upstream(lib):
    """No upstream gradient, no gradient: every output is exactly 0."""
    P = bwd_problem(51)
    z = np.zeros_like(P["dW"])
    dk, dv, db, dg = oracle.wy_backward(P["k"], P["v"], P["beta"], P["C"], z, z,
                                        dT=np.zeros_like(P["dT"]), g=P["g"], lib=lib)
    assert not dk.any() and not dv.any() and not db.any() and not dg.any()


def pin_bwd_gate_zero(lib):
    """g = 0 gives the ungated dk, dv, dbeta bit for bit (and a gradient for g)."""
    P = bwd_problem(52, gated=False)
    a = oracle.wy_backward(P["k"], P["v"], P["beta"], P["C"], P["dW"], P["dU"], dT=P["dT"],
                           lib=lib)
    b = oracle.wy_backward(P["k"], P["v"], P["beta"], P["C"], P["dW"], P["dU"], dT=P["dT"],
                           g=np.zeros_like(P["beta"]), lib=lib)
    assert all(np.array_equal(x, y) for x, y in zip(a[:3], b[:3])) and a[3] is None
    assert np.any(b[3] != 0)


# ---------------------------------------------------------------------------------------------
# the single right-hand-side solve ([Inv] section 5, item 10: T never formed)

def solve_one(lib, K, R, beta, g=None, C=None):
    """solve_rhs on one chunk [0, n) of a single-head problem (fp32 inputs)."""
    n = K.shape[0]
    k = np.ascontiguousarray(K[None, :, None, :], np.float32)
    r = np.ascontiguousarray(R[None, :, None, :], np.float32)
    b = np.ascontiguousarray(beta[None, :, None], np.float32)
    gg = None if g is None else np.ascontiguousarray(g[None, :, None], np.float32)
    return oracle.solve_rhs(k, r, b, C or n, g=gg, lib=lib, nthreads=1)[0, :, 0]


def gated_a(K, beta, g):
    """A = I + strictLower(diag(beta)(Gamma o K K^T)), Gamma[i][j] = exp(G_i - G_j), fp64."""
    G = np.cumsum(g.astype(np.float64))
    K = K.astype(np.float64)
    gam = np.exp(G[:, None] - G[None, :])
    return np.eye(len(K)) + np.tril(beta.astype(np.float64)[:, None] * gam * (K @ K.T), -1)


def pin_solve_rhs_residual(lib):
    """A X = diag(beta) R for A formed here in numpy, gated and ungated, several lengths."""
    rng = np.random.default_rng(40)
    for n, mu in ((32, None), (45, 2.0), (64, None), (100, 0.5), (128, 4.0)):
        K = unit_keys(rng, n)
        R = rng.standard_normal((n, 128)).astype(np.float32)
        beta = rng.uniform(0.0, 1.0, n).astype(np.float32)
        g = None if mu is None else unit_gates(rng, n, mu)
        X = solve_one(lib, K, R, beta, g)
        A = a_matrix(K, beta) if g is None else gated_a(K, beta, g)
        res = A @ X - beta.astype(np.float64)[:, None] * R.astype(np.float64)
        assert np.max(np.abs(res)) <= 1e-12


def pin_solve_rhs_delta_rule(lib):
    """With R = V the solve is U: the gated delta rule from S_0 = 0 ends at
    S_n = X^T diag(exp(G_n - G)) K (g = 0: the plain delta rule, S_n = X^T K)."""
    rng = np.random.default_rng(41)
    for n, mu in ((40, None), (64, 3.0)):
        K = unit_keys(rng, n)
        V = rng.standard_normal((n, 128)).astype(np.float32)
        beta = rng.uniform(0.0, 1.0, n).astype(np.float32)
        g = np.zeros(n, np.float32) if mu is None else unit_gates(rng, n, mu)
        X = solve_one(lib, K, V, beta, None if mu is None else g)
        K64, V64 = K.astype(np.float64), V.astype(np.float64)
        S = np.zeros((128, 128))
        for t in range(n):
            a, b = math.exp(float(g[t])), float(beta[t])
            S = S @ (a * (np.eye(128) - b * np.outer(K64[t], K64[t]))) + b * np.outer(V64[t], K64[t])
        G = np.cumsum(g.astype(np.float64))
        assert np.max(np.abs(S - X.T @ (np.exp(G[-1] - G)[:, None] * K64))) <= 1e-12


def pin_solve_rhs_degenerate(lib):
    """Orthogonal keys: A = I, so X = diag(beta) R exactly; beta = 0: X = 0 exactly."""
    rng = np.random.default_rng(42)
    n = 64
    K = np.eye(128, dtype=np.float32)[rng.permutation(128)[:n]]
    R = rng.standard_normal((n, 128)).astype(np.float32)
    beta = rng.uniform(0.0, 1.0, n).astype(np.float32)
    X = solve_one(lib, K, R, beta)
    assert np.array_equal(X, beta.astype(np.float64)[:, None] * R.astype(np.float64))
    X0 = solve_one(lib, unit_keys(rng, n), R, np.zeros(n, np.float32))
    assert np.array_equal(X0, np.zeros_like(X0))


def pin_solve_rhs_matches_u(lib):
    """Whole tensors of a packed, grouped-head, gated problem: X with rhs = v equals the separately
    pinned U = T diag(beta) V, chunk by chunk and head by head."""
    for C in (32, 64):
        inp = synth.custom(1, 0, 2, 6, C, dtype="f32", seed=43 + C, gate_mu=2.0,
                           seqlens=[3 * C + 5, 7, C])
        X = oracle.solve_rhs(inp["k"], inp["v"], inp["beta"], C, cu_seqlens=inp["cu_seqlens"],
                             g=inp["g"], lib=lib, nthreads=2)
        _, _, U, _ = oracle.wy_prepare(inp["k"], inp["beta"], C, v=inp["v"],
                                       cu_seqlens=inp["cu_seqlens"], g=inp["g"], lib=lib,
                                       nthreads=2)
        assert np.max(np.abs(X - U)) <= 1e-12 * max(1.0, float(np.max(np.abs(U))))


PINS = [pin_closed_form_2, pin_orthogonal, pin_residual_structure, pin_lapack_inverse,
        pin_block_identity, pin_beta_zero, pin_subdiag_only, pin_identical_keys,
        pin_fma_counts, pin_householder_product, pin_delta_rule, pin_tail_padding, pin_layout,
        pin_head_grouping, pin_gate_zero, pin_gated_closed_form_2, pin_gated_recurrence,
        pin_gated_similarity, pin_gated_chunk_restart, pin_gdn_read_back, pin_gdn_beta_zero,
        pin_gdn_linear_attention, pin_gdn_chunk_form, pin_gdn_sequences_independent,
        pin_bwd_finite_differences, pin_bwd_zero_upstream, pin_bwd_gate_zero,
        pin_solve_rhs_residual, pin_solve_rhs_delta_rule, pin_solve_rhs_degenerate,
        pin_solve_rhs_matches_u]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin, oracle_lib):
    pin(oracle_lib)


# ---------------------------------------------------------------------------------------------
# magnitudes and the generator's conditioning (pages' measured numbers)

def test_error_magnitudes(oracle_lib):
    """[Inv] section 4 results table: real A errors against np.linalg.inv are ~1e-16, and an
    fp16-stored T carries ~5.7e-5 relative error."""
    table = {r[0]: float(r[1]) for r in read_table("error_magnitudes.txt")}
    rng = np.random.default_rng(23)
    worst, rel16 = 0.0, []
    for _ in range(200):
        K = unit_keys(rng, 32)
        beta = (1 / (1 + np.exp(-rng.standard_normal(32)))).astype(np.float32)
        A = a_matrix(K, beta)
        T, _ = oracle.row_forward_inverse(A, lib=oracle_lib)
        worst = max(worst, float(np.max(np.abs(T - np.linalg.inv(A)))))
        T16 = T.astype(np.float16).astype(np.float64)
        rel16.append(np.linalg.norm(T16 - T) / np.linalg.norm(T))
    assert worst <= 100 * table["real_A_200_samples"]
    assert table["fp16_stored_T_relative"] / 10 <= max(rel16) <= table["fp16_stored_T_relative"] * 10
    # the general 16x16 / 32x32 cases of the table stay within 10x of their printed values
    Lg = np.tril(rng.uniform(-1, 1, (16, 16)), -1) + np.eye(16)
    X, _ = oracle.row_forward_inverse(Lg, lib=oracle_lib)
    assert np.max(np.abs(X - np.linalg.inv(Lg))) <= 10 * table["row_wise_16x16"]
    Lg = np.tril(rng.uniform(-1, 1, (32, 32)), -1) + np.eye(32)
    X, _, _ = oracle.block_recursive_inverse(Lg, 16, lib=oracle_lib)
    assert np.max(np.abs(X - np.linalg.inv(Lg))) <= 10 * table["recursive_32x32"]


@pytest.mark.parametrize("C", [32, 64, 128])
def test_generator_conditioning(C):
    """[Inv] section 2.4 cost table: measured cond(A) upper bounds 2.0 / 2.6 / 3.6 for C = 32 /
    64 / 128 and strict-lower entries within 0.358 ([Inv] section 4), on the workloads' input
    distribution (L2-normalised bf16 keys, beta = sigmoid(N(0, 1)))."""
    bound = {int(r[0]): (float(r[1]), float(r[2])) for r in read_table("conditioning.txt")}[C]
    inp = synth.custom(1, 200 * C, 1, 1, C, dtype="bf16", seed=100 + C)
    K = synth.bf16_bits_to_f32(inp["k"])[0, :, 0].astype(np.float64)
    b = inp["beta"][0, :, 0].astype(np.float64)
    cmax, lmax = 0.0, 0.0
    for c in range(200):
        A = a_matrix(K[c * C:(c + 1) * C], b[c * C:(c + 1) * C])
        cmax = max(cmax, float(np.linalg.cond(A)))
        lmax = max(lmax, float(np.max(np.abs(np.tril(A, -1)))))
    assert cmax <= bound[0]
    assert lmax <= bound[1]


# ---------------------------------------------------------------------------------------------
# planted mistakes: each mutant copy of the oracle must fail at least one pin

MUTANTS = {
    "beta_dropped": ("a = s->b[i] * decay * g;", "a = decay * g;"),
    "beta_on_columns": ("a = s->b[i] * decay * g;", "a = s->b[j] * decay * g;"),
    "gram_term_dropped": ("for (int32_t d = 0; d < dk; ++d)\n                    g +=",
                          "for (int32_t d = 1; d < dk; ++d)\n                    g +="),
    "gram_wrong_index": ("* s->K[(int64_t)j * dk + d];\n                const double decay",
                         "* s->K[(int64_t)i * dk + d];\n                const double decay"),
    "substitution_sign": ("xk[i] -= lkj * xj[i];", "xk[i] += lkj * xj[i];"),
    "substitution_unit_term_dropped": ("for (int32_t i = 0; i <= j; ++i) {",
                                       "for (int32_t i = 0; i < j; ++i) {"),
    "substitution_transposed": ("const double lkj = L[(int64_t)k * ldl + j];",
                                "const double lkj = L[(int64_t)j * ldl + k];"),
    "wu_t_transposed": ("acc += (s->X[(int64_t)i * n + j] * s->b[j] * s->E[j]) * s->K",
                        "acc += (s->X[(int64_t)j * n + i] * s->b[j] * s->E[j]) * s->K"),
    "wu_beta_index": ("acc += (s->X[(int64_t)i * n + j] * s->b[j]) * s->V",
                      "acc += (s->X[(int64_t)i * n + j] * s->b[i]) * s->V"),
    "u_uses_keys": ("* s->V[(int64_t)j * dv + e];", "* s->K[(int64_t)j * dk + e];"),
    "head_map_modulo": ("const int32_t hk = hv / (Hv / Hq);", "const int32_t hk = hv % Hq;"),
    "coupling_sign": ("X[(int64_t)(h + i) * ldx + j] = -s;", "X[(int64_t)(h + i) * ldx + j] = s;"),
    "tail_columns_leak": ("trow[j] = (j < n) ? s.X[(int64_t)i * n + j] : 0.0;",
                          "trow[j] = (j < n) ? s.X[(int64_t)i * n + j] : 1.0;"),
    # gates
    "gate_dropped_in_a": ("a = s->b[i] * decay * g;", "a = s->b[i] * g;"),
    "gate_transposed": ("exp(s->G[i] - s->G[j])", "exp(s->G[j] - s->G[i])"),
    "gate_sign": ("s->G[i - 1]) + gi;", "s->G[i - 1]) - gi;"),
    "gate_exclusive_in_w": ("s->E[i] = exp(s->G[i]);", "s->E[i] = exp(s->G[i] - gi);"),
    "gate_dropped_in_w": ("acc += (s->X[(int64_t)i * n + j] * s->b[j] * s->E[j]) * s->K",
                          "acc += (s->X[(int64_t)i * n + j] * s->b[j]) * s->K"),
    "gate_on_u": ("acc += (s->X[(int64_t)i * n + j] * s->b[j]) * s->V",
                  "acc += (s->X[(int64_t)i * n + j] * s->b[j] * s->E[j]) * s->V"),
    # the token-by-token recurrence
    "gdn_delta_sign": ("S[(int64_t)d * dv + c] += kt[d] * e[c];",
                       "S[(int64_t)d * dv + c] -= kt[d] * e[c];"),
    "gdn_beta_dropped": ("e[c] = b * (load_elem", "e[c] = (load_elem"),
    "gdn_decay_dropped": ("S[i] *= alpha;", "S[i] *= 1.0;"),
    "gdn_q_head_modulo": ("hk = hv / (Hv / Hq);\n            const int64_t s0",
                          "hk = hv % Hq;\n            const int64_t s0"),
    "gdn_h0_transposed": ("S[i] = h0 ? (double)h0[i] : 0.0;",
                          "S[i] = h0 ? (double)h0[(i % dv) * dk + i / dv] : 0.0;"),
    "gdn_scale_dropped": ("= jb->scale * r;", "= r;"),
    "gdn_state_not_reset": ("for (int64_t i = 0; i < (int64_t)dk * dv; ++i) S[i] = h0 ?",
                            "if (seq == 0) for (int64_t i = 0; i < (int64_t)dk * dv; ++i) S[i] = h0 ?"),
    # the backward
    "bwd_dA_sign": ("M[(int64_t)i * n + j] = -acc;", "M[(int64_t)i * n + j] = acc;"),
    "bwd_TdW_untransposed": ("acc += T[(int64_t)m * n + i] * dWc", "acc += T[(int64_t)i * n + m] * dWc"),
    "bwd_rt_term_dropped": ("dK[(int64_t)j * dk + d] += rr * K[(int64_t)i * dk + d];", "(void)0;"),
    "bwd_dg_forward_sum": ("for (int32_t t = n - 1; t >= 0; --t) {", "for (int32_t t = 0; t < n; ++t) {"),
    "bwd_group_overwrite": ("dK[(int64_t)i * dk + d] += b[i] * E[i] * t;",
                            "dK[(int64_t)i * dk + d] = b[i] * E[i] * t;"),
    "bwd_dbeta_gram_dropped": ("dbrow[row] += mij * gam * kk;", "dbrow[row] += 0.0;"),
    "bwd_dT_ignored": ("double a = jb->dT ?", "double a = 0.0 * (double)(jb->dT != NULL) + 0 ?"),
    # the single right-hand-side solve
    "rhs_beta_dropped": ("double x = s->b[i] * s->V[(int64_t)i * dv + e];",
                         "double x = s->V[(int64_t)i * dv + e];"),
    "rhs_sign": ("x -= s->A[(int64_t)i * n + j] * Xout", "x += s->A[(int64_t)i * n + j] * Xout"),
    "rhs_a_transposed": ("x -= s->A[(int64_t)i * n + j] * Xout", "x -= s->A[(int64_t)j * n + i] * Xout"),
    "rhs_head_scatter": ("memcpy(jb->U + ((tok0 + i) * Hv + hv) * dv",
                         "memcpy(jb->U + ((tok0 + i) * Hv + (hv + 1) % Hv) * dv"),
    "gate_not_restarted": ("s->G[i] = (i == 0 ? 0.0 : s->G[i - 1]) + gi;",
                           "s->G[i] = (i == 0 ? (gate && tok0 > 0 ? (double)gate[(tok0 - 1) * Hv + hv] "
                           ": 0.0) : s->G[i - 1]) + gi;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutants_are_caught(name, tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    old, new = MUTANTS[name]
    src = open(oracle.SOURCES[0]).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not unique/found"
    mutated = src.replace(old, new)
    path = tmp_path / "wyo_oracle.c"
    path.write_text(mutated)
    shutil.copy(os.path.join(os.path.dirname(oracle.SOURCES[0]), "wyo_oracle.h"), tmp_path)
    lib_path = str(tmp_path / "libmutant.so")
    oracle.build(lib_path, sources=[str(path)], extra_flags=("-w",))
    lib = oracle.load(lib_path)
    caught = []
    for pin in PINS:
        try:
            pin(lib)
        except (AssertionError, ValueError):
            caught.append(pin.__name__)
    assert caught, f"mutant {name} passed every pin"
