"""The gated coefficient on the HIP path vs the fp64 oracle, through the C ABI (needs a GPU).

"TileLang 实战：单位下三角矩阵求逆" section 5, item 12: with gating the coefficient is
diag(beta)(Gamma o K K^T); the FlashQLA usage section passes the per-token log gates g
[B,T,Hv] beside beta.  Reading: G_i = g_0 + ... + g_i within each chunk,
Gamma[i][j] = exp(G_i - G_j), W = T diag(beta exp(G)) K, U = T diag(beta) V.

Bar as for the ungated step: T within 1e-5 max-abs, W and U within 1e-2 relative Frobenius,
T's diagonal exactly 1 and strict upper triangle exactly 0, every output written.
"""
import numpy as np
import pytest

from chunkwise_gated_deltanet_amd import synth
from gpu_util import (check_structure, compare_full, gate_of, rel_fro, run_wy,
                      say, to_device, to_f64)

pytestmark = pytest.mark.gpu

# mu = 4: the seeded gated recipe (alpha ~ 0.98); mu = 0: strong decay (alpha ~ 0.5, a chunk
# of 64 decays by ~e^-45), where most of Gamma underflows towards 0.
CASES = {
    "C32_B2_mu4": dict(batch=2, seqlen=333, num_qk_heads=4, num_v_heads=4, chunk_size=32,
                       seed=80, gate_mu=4.0),
    "C64_B2_mu4": dict(batch=2, seqlen=333, num_qk_heads=4, num_v_heads=4, chunk_size=64,
                       seed=81, gate_mu=4.0),
    "C128_B2_mu4": dict(batch=2, seqlen=333, num_qk_heads=4, num_v_heads=4, chunk_size=128,
                        seed=82, gate_mu=4.0),
    "C64_packed_gva_mu4": dict(batch=1, seqlen=0, num_qk_heads=4, num_v_heads=16,
                               chunk_size=64, seed=83, gate_mu=4.0,
                               seqlens=[300, 517, 64, 1, 129, 250, 63, 65]),
    "C32_packed_gva_mu0": dict(batch=1, seqlen=0, num_qk_heads=2, num_v_heads=8,
                               chunk_size=32, seed=84, gate_mu=0.0,
                               seqlens=[31, 33, 1, 95, 200]),
    "C64_mu0": dict(batch=1, seqlen=700, num_qk_heads=4, num_v_heads=4, chunk_size=64,
                    seed=85, gate_mu=0.0),
    "C128_packed_mu1": dict(batch=1, seqlen=0, num_qk_heads=2, num_v_heads=4, chunk_size=128,
                            seed=86, gate_mu=1.0, seqlens=[127, 129, 1, 300, 17]),
    "fp32_C32_mu2": dict(batch=1, seqlen=256, num_qk_heads=2, num_v_heads=2, chunk_size=32,
                         dtype="f32", seed=87, gate_mu=2.0),
    "fp32_C64_mu4": dict(batch=1, seqlen=200, num_qk_heads=2, num_v_heads=2, chunk_size=64,
                         dtype="f32", seed=88, gate_mu=4.0),
    "fp32_C128_packed_mu3": dict(batch=1, seqlen=0, num_qk_heads=1, num_v_heads=2,
                                 chunk_size=128, dtype="f32", seed=89, gate_mu=3.0,
                                 seqlens=[300, 1, 128]),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_gated_wy_prepare_small(name, gpu):
    inp = synth.custom(**CASES[name])
    say(f"gated wy_prepare {name}")
    T, W, U = run_wy(inp, gpu)
    check_structure(T, inp)
    compare_full(inp, T, W, U, label="gated " + name)


@pytest.mark.parametrize("name", ["C32_B2_mu4", "C64_packed_gva_mu4", "C128_packed_mu1",
                                  "fp32_C64_mu4"])
def test_gated_entry_points_agree(name, gpu):
    """kkt_solve's T and wu_prepare's W, U equal wy_prepare's bit for bit with gates."""
    import torch
    import chunkwise_gated_deltanet_amd as cg
    inp = synth.custom(**CASES[name])
    say(f"gated entry points {name}")
    T0, W0, U0 = run_wy(inp, gpu)
    T1, _, _ = run_wy(inp, gpu, kkt_only=True)
    assert torch.equal(T0, T1)
    k, v, beta, cu = to_device(inp, gpu)
    W1, U1 = cg.wu_prepare(k, v, beta, inp["chunk_size"], cu_seqlens=cu, g=gate_of(inp, gpu))
    torch.cuda.synchronize(gpu)
    assert torch.equal(W0, W1) and torch.equal(U0, U1)


@pytest.mark.parametrize("C", [32, 64, 128])
def test_zero_gates_equal_no_gates(C, gpu):
    """g = 0 (alpha = 1) gives exactly the ungated T and U; W agrees to its tolerance (its T'
    operand is re-split after the scale by exp(0) = 1)."""
    import torch
    inp = synth.custom(1, 0, 2, 4, C, seed=90 + C, seqlens=[3 * C + 7, C - 1])
    T0, W0, U0 = run_wy(inp, gpu)
    inp["g"] = np.zeros_like(inp["beta"])
    say(f"zero gates C={C}")
    T1, W1, U1 = run_wy(inp, gpu)
    assert torch.equal(T0, T1) and torch.equal(U0, U1)
    assert rel_fro(to_f64(W1), to_f64(W0)) <= 1e-3
