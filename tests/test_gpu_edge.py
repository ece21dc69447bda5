"""Edge cases and degenerate inputs of the HIP path (needs a GPU).

Degenerate checks from "TileLang 实战：单位下三角矩阵求逆" section 4: beta -> 0 gives T = I,
and with only the sub-diagonal block nonzero the lower-left of T is exactly -L10.
"""
import math

import numpy as np
import pytest

from chunkwise_gated_deltanet_amd import synth
from gpu_util import (T_TOL, check_structure, compare_full, rel_fro, run_wy, say, to_f64)

pytestmark = pytest.mark.gpu


def make_inp(K, V, beta, C, dtype="bf16", seqlens=None):
    """Single-sequence (or packed) inputs from [T, H, 128] arrays."""
    if dtype == "bf16":
        k, v = synth.f32_to_bf16_bits(K), synth.f32_to_bf16_bits(V)
    else:
        k, v = K.astype(np.float32), V.astype(np.float32)
    cu = None
    if seqlens is not None:
        cu = np.concatenate([[0], np.cumsum(seqlens)]).astype(np.int32)
    return dict(k=np.ascontiguousarray(k[None]), v=np.ascontiguousarray(v[None]),
                beta=np.ascontiguousarray(beta[None].astype(np.float32)), cu_seqlens=cu,
                batch=1, seqlen=K.shape[0], chunk_size=C, dtype=dtype)


@pytest.mark.parametrize("C", [32, 64, 128])
def test_tail_lengths(C, gpu):
    lens = [1, 15, 16, 17, C - 1, C, C + 1, 2 * C + 17]
    inp = synth.custom(1, 0, 2, 4, C, seed=40 + C, seqlens=lens)
    say(f"tails C={C} lens={lens}")
    T, W, U = run_wy(inp, gpu)
    check_structure(T, inp)
    compare_full(inp, T, W, U, label=f"tails C={C}")


@pytest.mark.parametrize("C", [32, 64, 128])
def test_beta_zero_gives_identity(C, gpu):
    import torch
    inp = synth.custom(1, 3 * C + 5, 2, 2, C, seed=50)
    inp["beta"][:] = 0
    say(f"beta=0 C={C}")
    T, W, U = run_wy(inp, gpu)
    check_structure(T, inp)
    rows = T.reshape(-1, 2, C)
    # every entry other than the diagonal is zero
    assert int((rows != 0).sum()) == rows.shape[0] * rows.shape[1]
    assert bool((W == 0).all()) and bool((U == 0).all())


@pytest.mark.parametrize("C", [32, 64, 128])
def test_subdiagonal_only(C, gpu):
    """Keys making A's two C/2 diagonal blocks the identity: T's lower-left must be -L10
    (the top coupling level on its own, including its sign)."""
    h = C // 2
    c = np.float32(1 / math.sqrt(2))
    K = np.zeros((C, 1, 128), np.float32)
    for i in range(h):
        K[i, 0, i] = 1
        K[h + i, 0, i] = c
        K[h + i, 0, h + i] = c
    rng = np.random.default_rng(60)
    V = rng.standard_normal((C, 1, 128)).astype(np.float32)
    beta = rng.uniform(0.05, 0.95, (C, 1)).astype(np.float32)
    inp = make_inp(K, V, beta, C)
    say(f"sub-diagonal only C={C}")
    T, W, U = run_wy(inp, gpu)
    Tg = to_f64(T)[0, :, 0, :]
    cb = float(synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(np.array([c])))[0])
    L10 = np.diag(beta[h:, 0].astype(np.float64) * cb)
    assert np.max(np.abs(Tg[h:, :h] - (-L10))) <= 1e-7
    assert np.array_equal(Tg[:h, :h], np.eye(h)) and np.array_equal(Tg[h:, h:], np.eye(h))
    compare_full(inp, T, W, U, label=f"subdiag C={C}")


@pytest.mark.parametrize("C", [32, 64, 128])
def test_orthogonal_keys(C, gpu):
    rng = np.random.default_rng(61)
    K = np.zeros((C, 1, 128), np.float32)
    K[np.arange(C), 0, rng.permutation(128)[:C]] = 1
    V = rng.standard_normal((C, 1, 128)).astype(np.float32)
    beta = rng.uniform(0.05, 0.95, (C, 1)).astype(np.float32)
    inp = make_inp(K, V, beta, C)
    T, W, U = run_wy(inp, gpu)
    assert np.array_equal(to_f64(T)[0, :, 0, :], np.eye(C))
    compare_full(inp, T, W, U, label=f"orthogonal C={C}")


@pytest.mark.parametrize("C", [32, 64, 128])
def test_identical_keys(C, gpu):
    """Every key the same unit vector: the densest T (no zero entry below the diagonal), at
    each chunk size's own block and coupling layout."""
    rng = np.random.default_rng(62)
    k = rng.standard_normal(128).astype(np.float32)
    k /= np.linalg.norm(k)
    K = np.repeat(k[None, None, :], C, axis=0)
    V = rng.standard_normal((C, 1, 128)).astype(np.float32)
    beta = rng.uniform(0.0, 1.0, (C, 1)).astype(np.float32)
    inp = make_inp(K, V, beta, C)
    say(f"identical keys C={C}")
    T, W, U = run_wy(inp, gpu)
    compare_full(inp, T, W, U, label=f"identical keys C={C}")


def test_head_grouping(gpu):
    """Value head h reads key head h // (Hv/Hq): the result for v-head 5 of (Hq=2, Hv=8)
    equals a one-head problem built from key head 1 and value head 5."""
    import torch
    inp = synth.custom(1, 150, 2, 8, 64, seed=63)
    T, W, U = run_wy(inp, gpu)
    one = dict(inp)
    one["k"] = np.ascontiguousarray(inp["k"][:, :, 1:2])
    one["v"] = np.ascontiguousarray(inp["v"][:, :, 5:6])
    one["beta"] = np.ascontiguousarray(inp["beta"][:, :, 5:6])
    T1, W1, U1 = run_wy(one, gpu)
    assert torch.equal(T[:, :, 5:6], T1)
    assert torch.equal(W[:, :, 5:6], W1) and torch.equal(U[:, :, 5:6], U1)


def test_side_stream_and_determinism(gpu):
    import torch
    inp = synth.custom(2, 300, 4, 8, 64, seed=64)
    T0, W0, U0 = run_wy(inp, gpu)
    s = torch.cuda.Stream(device=gpu)
    T1, W1, U1 = run_wy(inp, gpu, stream=s)
    assert torch.equal(T0, T1) and torch.equal(W0, W1) and torch.equal(U0, U1)


def test_empty_and_zero_token_sequences(gpu):
    import torch
    import chunkwise_gated_deltanet_amd as cg
    k = torch.empty(1, 0, 2, 128, dtype=torch.bfloat16, device=gpu)
    v = torch.empty(1, 0, 2, 128, dtype=torch.bfloat16, device=gpu)
    beta = torch.empty(1, 0, 2, dtype=torch.float32, device=gpu)
    T, W, U = cg.wy_prepare(k, v, beta, 64)
    assert T.shape == (1, 0, 2, 64)
    # packed batch where some sequences are empty
    inp = synth.custom(1, 0, 1, 2, 64, seed=65, seqlens=[0, 70, 0, 0, 5, 0])
    T, W, U = run_wy(inp, gpu)
    check_structure(T, inp)
    compare_full(inp, T, W, U, label="zero-length sequences")


def test_rejects_bad_arguments_on_device(gpu):
    import torch
    import chunkwise_gated_deltanet_amd as cg
    k = torch.zeros(1, 64, 2, 128, dtype=torch.bfloat16, device=gpu)
    v = torch.zeros(1, 64, 3, 128, dtype=torch.bfloat16, device=gpu)
    beta = torch.zeros(1, 64, 3, dtype=torch.float32, device=gpu)
    with pytest.raises(ValueError):
        cg.wy_prepare(k, v, beta, 64)      # Hv = 3 not a multiple of Hq = 2
    with pytest.raises(ValueError):
        cg.kkt_solve(k, beta[:, :, :2].contiguous(), 48)  # unsupported C
