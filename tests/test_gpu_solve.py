"""wyp_solve_rhs, one right-hand side with T never formed, against the fp64 oracle's forward
substitution on the right-hand side (oracle.solve_rhs), through the C ABI (needs a GPU).

"TileLang 实战：单位下三角矩阵求逆" section 5, item 10: T used once is not materialised; the
substitution is applied to the right-hand side.  X = A^{-1} diag(beta) R per chunk and value head.
Bar (X is stored in k's dtype, like U): relative Frobenius <= 1e-2 over the whole tensor, every
entry written (outputs pre-filled with NaN); with R = V, X also agrees with wy_prepare's U to
that bar.  The right-hand side is its own random tensor, not v, so the kernel must read rhs.
"""
import numpy as np
import pytest

import oracle
from chunkwise_gated_deltanet_amd import synth
from gpu_util import WU_TOL, gate_of, oracle_threads, rel_fro, run_wy, say, to_device, to_f64

pytestmark = pytest.mark.gpu


def rhs_of(inp, seed):
    """A right-hand side R [B,T,Hv,128] independent of v: N(0,1), in k's dtype."""
    rng = np.random.default_rng(seed)
    R = rng.standard_normal(inp["v"].shape, dtype=np.float32)
    return synth.f32_to_bf16_bits(R) if inp["dtype"] == "bf16" else R


def dev(a, device):
    import torch
    t = torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a)
    return (t.view(torch.bfloat16) if a.dtype == np.uint16 else t).to(device)


def run_solve(inp, R, device):
    import torch
    import chunkwise_gated_deltanet_amd as cg
    k, _, beta, cu = to_device(inp, device)
    rhs = dev(R, device)
    X = torch.full(rhs.shape, float("nan"), dtype=rhs.dtype, device=device)
    cg.solve_rhs(k, rhs, beta, inp["chunk_size"], cu_seqlens=cu, X_out=X, g=gate_of(inp, device))
    torch.cuda.synchronize(device)
    return X, rhs


def check(inp, R, device, label):
    import torch
    X, rhs = run_solve(inp, R, device)
    assert not torch.isnan(X).any(), "unwritten X entries"
    assert torch.equal(rhs, dev(R, device)), "rhs was modified"
    ref = oracle.solve_rhs(inp["k"], R, inp["beta"], inp["chunk_size"],
                           cu_seqlens=inp["cu_seqlens"], g=inp.get("g"), nthreads=oracle_threads())
    err = rel_fro(to_f64(X), ref)
    say(f"[{label}] X rel fro {err:.3e}")
    assert err <= WU_TOL, err
    return X, ref


CASES = {
    "tiny_fp32_C32": dict(idx=1),
    "T700_C64": dict(batch=1, seqlen=700, num_qk_heads=4, num_v_heads=4, chunk_size=64, seed=150,
                     beta_sigma=1.5),
    "B2_T333_C32_mu4": dict(batch=2, seqlen=333, num_qk_heads=4, num_v_heads=4, chunk_size=32,
                            seed=151, gate_mu=4.0),
    "B2_T333_C128": dict(batch=2, seqlen=333, num_qk_heads=4, num_v_heads=4, chunk_size=128,
                         seed=152),
    "packed_gva_C64_mu0": dict(batch=1, seqlen=0, num_qk_heads=4, num_v_heads=16, chunk_size=64,
                               seed=153, gate_mu=0.0, seqlens=[300, 517, 64, 1, 129, 250, 63, 65]),
    "packed_gva_C128_mu2": dict(batch=1, seqlen=0, num_qk_heads=2, num_v_heads=4, chunk_size=128,
                                seed=154, gate_mu=2.0, seqlens=[127, 129, 1, 300, 17]),
    "fp32_C64": dict(batch=1, seqlen=200, num_qk_heads=2, num_v_heads=2, chunk_size=64,
                     dtype="f32", seed=155),
    "fp32_packed_C128_mu3": dict(batch=1, seqlen=0, num_qk_heads=1, num_v_heads=2, chunk_size=128,
                                 dtype="f32", seed=156, gate_mu=3.0, seqlens=[300, 1, 128]),
    "empty_sequences_C32": dict(batch=1, seqlen=0, num_qk_heads=1, num_v_heads=2, chunk_size=32,
                                seed=157, seqlens=[0, 40, 0, 0, 33, 0]),
}


def inputs(spec):
    spec = dict(spec)
    if "idx" in spec:
        return synth.generate(synth.workload(spec["idx"]))
    return synth.custom(**spec)


@pytest.mark.parametrize("name", sorted(CASES))
def test_solve_rhs_small(name, gpu):
    inp = inputs(CASES[name])
    say(f"solve_rhs {name}")
    check(inp, rhs_of(inp, 7), gpu, name)


@pytest.mark.parametrize("C", [32, 64, 128])
def test_solve_rhs_with_v_is_u(C, gpu):
    """R = V: X is U, as wy_prepare computes it through T (another order of operations)."""
    inp = synth.custom(1, 0, 2, 8, C, seed=160 + C, gate_mu=4.0, seqlens=[3 * C + 9, C, 5])
    say(f"solve_rhs with R = V, C={C}")
    X, ref = check(inp, inp["v"], gpu, f"R=V C={C}")
    _, _, U = run_wy(inp, gpu)
    err = rel_fro(to_f64(X), to_f64(U))
    say(f"[R=V C={C}] X vs wy_prepare U rel fro {err:.3e}")
    assert err <= WU_TOL, err


@pytest.mark.parametrize("C", [32, 64, 128])
def test_solve_rhs_degenerate(C, gpu):
    """beta = 0: X = 0 exactly; orthogonal keys (A = I): X = diag(beta) R, one rounding."""
    import torch
    inp = synth.custom(1, 2 * C + 3, 1, 2, C, seed=170 + C)
    R = rhs_of(inp, 3)
    inp0 = dict(inp, beta=np.zeros_like(inp["beta"]))
    X0, _ = run_solve(inp0, R, gpu)
    assert bool((X0 == 0).all())
    n = inp["seqlen"]
    eye = np.eye(128, dtype=np.float32)[np.arange(n) % 128]    # distinct keys within a chunk
    inpo = dict(inp, k=synth.f32_to_bf16_bits(eye[None, :, None, :]))
    Xo, _ = run_solve(inpo, R, gpu)
    want = (inp["beta"][..., None] * synth.bf16_bits_to_f32(R))
    assert torch.equal(Xo, dev(synth.f32_to_bf16_bits(want), gpu))


FULL = [(i, c) for i in (1, 2, 3, 4, 5) for c in (32, 64, 128)]


@pytest.mark.slow
@pytest.mark.parametrize("idx,C", FULL, ids=[f"w{i}_C{c}" for i, c in FULL])
def test_solve_rhs_full_size(idx, C, gpu):
    """Whole tensors at full size, ungated then gated (mu = 4) on the same k, beta and R."""
    import torch
    w = synth.workload(idx, chunk_size=C, gate_mu=4.0)
    inp = synth.generate(w)
    R = rhs_of(inp, 1000 + idx)
    g = inp["g"]
    for gate in (None, g):
        inp["g"] = gate
        say(f"solve_rhs full {w.name} C={C} gated={gate is not None}")
        check(inp, R, gpu, f"full {w.name} C={C} gated={gate is not None}")
        torch.cuda.empty_cache()
