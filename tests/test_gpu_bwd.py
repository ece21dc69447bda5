"""Backward of the preparation step (wyp_wy_backward) against the fp64 oracle's gradient of
<dT,T> + <dW,W> + <dU,U>, through the C ABI (needs a GPU).

The oracle is pinned by central finite differences.  Bar (derived from the arithmetic: T and
R + R^T enter the bf16 products as hi + lo pairs, so the only coarse rounding is the bf16 output
of dk and dv; a simulation of this arithmetic gives 1.7e-3 for dk, dv and 1e-6 for dbeta, dg):
dk and dv within 1e-2 relative Frobenius, dbeta and dg within 1e-4.
"""
import numpy as np
import pytest

import oracle
from chunkwise_gated_deltanet_amd import synth
from gpu_util import gate_of, rel_fro, say, to_device, to_f64

pytestmark = pytest.mark.gpu

KV_TOL = 1e-2
BG_TOL = 1e-4

CASES = {
    "B2_T333_H4": dict(batch=2, seqlen=333, num_qk_heads=4, num_v_heads=4, seed=120),
    "B2_T333_H4_mu4_dT": dict(batch=2, seqlen=333, num_qk_heads=4, num_v_heads=4, seed=121,
                              gate_mu=4.0, dT=True),
    "packed_gva_mu4_dT": dict(batch=1, seqlen=0, num_qk_heads=4, num_v_heads=16, seed=122,
                              gate_mu=4.0, dT=True, seqlens=[300, 517, 64, 1, 129, 250, 63, 65]),
    "packed_gva_mu0": dict(batch=1, seqlen=0, num_qk_heads=2, num_v_heads=8, seed=123,
                           gate_mu=0.0, seqlens=[31, 33, 1, 95, 200]),
    "T700_H2_dT": dict(batch=1, seqlen=700, num_qk_heads=2, num_v_heads=2, seed=124, dT=True,
                       beta_sigma=1.5),
    # C = 32: four waves per workgroup, two workgroups per CU
    "C32_B2_T333_H4_mu4_dT": dict(C=32, batch=2, seqlen=333, num_qk_heads=4, num_v_heads=4,
                                  seed=127, gate_mu=4.0, dT=True),
    "C32_packed_gva_mu0": dict(C=32, batch=1, seqlen=0, num_qk_heads=2, num_v_heads=8, seed=128,
                               gate_mu=0.0, seqlens=[31, 32, 33, 1, 0, 95, 200]),
    "C32_T700_H2_ungated_dT": dict(C=32, batch=1, seqlen=700, num_qk_heads=2, num_v_heads=2,
                                   seed=129, dT=True, beta_sigma=1.5),
    # eight value heads per key head: dk sums eight jobs in registers before its one store
    "gva8_mu4_dT": dict(batch=1, seqlen=0, num_qk_heads=2, num_v_heads=16, seed=131, gate_mu=4.0,
                        dT=True, seqlens=[200, 333, 64, 1, 129]),
    "C32_gva8_mu4_dT": dict(C=32, batch=1, seqlen=0, num_qk_heads=2, num_v_heads=16, seed=132,
                            gate_mu=4.0, dT=True, seqlens=[200, 333, 32, 1, 65]),
    # C = 128: K, T and one C x C region in LDS, V staged while X is formed, dW / dU streamed
    "C128_B2_T333_H4_mu4_dT": dict(C=128, batch=2, seqlen=333, num_qk_heads=4, num_v_heads=4,
                                   seed=133, gate_mu=4.0, dT=True),
    "C128_packed_gva_mu0": dict(C=128, batch=1, seqlen=0, num_qk_heads=2, num_v_heads=8, seed=134,
                                gate_mu=0.0, seqlens=[127, 128, 129, 1, 0, 95, 300]),
    "C128_T700_H2_ungated_dT": dict(C=128, batch=1, seqlen=700, num_qk_heads=2, num_v_heads=2,
                                    seed=135, dT=True, beta_sigma=1.5),
    "C128_gva8_mu4_dT": dict(C=128, batch=1, seqlen=0, num_qk_heads=2, num_v_heads=16, seed=136,
                             gate_mu=4.0, dT=True, seqlens=[200, 333, 128, 1, 129]),
    "C128_B1_T512_H2_ungated": dict(C=128, batch=1, seqlen=512, num_qk_heads=2, num_v_heads=2,
                                    seed=137),
}


def make_inputs(spec):
    spec = dict(spec)
    want_dT = spec.pop("dT", False)
    C = spec.pop("C", 64)
    inp = synth.custom(chunk_size=C, **spec)
    inp["C"] = C
    rng = np.random.default_rng(spec["seed"] + 2000)
    B, T, Hv = inp["beta"].shape
    dW = synth.f32_to_bf16_bits(rng.standard_normal((B, T, Hv, 128)).astype(np.float32))
    dU = synth.f32_to_bf16_bits(rng.standard_normal((B, T, Hv, 128)).astype(np.float32))
    dT = rng.standard_normal((B, T, Hv, C)).astype(np.float32) if want_dT else None
    return inp, dW, dU, dT


def run_bwd(inp, dW, dU, dT, device):
    import torch
    import chunkwise_gated_deltanet_amd as cg
    k, v, beta, cu = to_device(inp, device)
    bf = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
    out = cg.wy_backward(k, v, beta, inp.get("C", 64), bf(dW), bf(dU),
                         dT=None if dT is None else torch.from_numpy(dT).to(device),
                         g=gate_of(inp, device), cu_seqlens=cu)
    torch.cuda.synchronize(device)
    return out


def check(inp, dW, dU, dT, out, label):
    dk, dv, db, dg = out
    rk, rv, rb, rg = oracle.wy_backward(inp["k"], inp["v"], inp["beta"], inp.get("C", 64), dW, dU,
                                        dT=dT, g=inp.get("g"), cu_seqlens=inp["cu_seqlens"])
    m = {"dk": rel_fro(to_f64(dk), rk), "dv": rel_fro(to_f64(dv), rv),
         "dbeta": rel_fro(to_f64(db), rb)}
    if rg is not None:
        m["dg"] = rel_fro(to_f64(dg), rg)
    say(f"[{label}] " + ", ".join(f"{k} {v:.3e}" for k, v in m.items()))
    assert m["dk"] <= KV_TOL and m["dv"] <= KV_TOL, m
    assert m["dbeta"] <= BG_TOL and m.get("dg", 0.0) <= BG_TOL, m


@pytest.mark.parametrize("name", sorted(CASES))
def test_wy_backward_small(name, gpu):
    inp, dW, dU, dT = make_inputs(CASES[name])
    say(f"wy_backward {name}")
    out = run_bwd(inp, dW, dU, dT, gpu)
    check(inp, dW, dU, dT, out, name)


@pytest.mark.parametrize("C", [32, 64, 128])
def test_wy_backward_identical_keys(C, gpu):
    """All keys of a chunk equal: the cancellation case that makes a single bf16 rounding of T
    miss the W tolerance in the forward."""
    inp, dW, dU, dT = make_inputs(dict(C=C, batch=1, seqlen=128, num_qk_heads=1, num_v_heads=2,
                                       seed=125, dT=True, gate_mu=4.0))
    for c0 in range(0, 128, C):
        inp["k"][0, c0:c0 + C] = inp["k"][0, c0]
    say(f"wy_backward identical keys C={C}")
    out = run_bwd(inp, dW, dU, dT, gpu)
    check(inp, dW, dU, dT, out, "identical keys")


@pytest.mark.parametrize("C", [32, 64, 128])
def test_wy_backward_many_short_sequences(C, gpu):
    """1100 packed sequences of 1..C+1 tokens (a few empty): the work map's search and its empty
    slots, on the key-head units of the backward."""
    rng = np.random.default_rng(126)
    lens = rng.integers(1, C + 2, size=1100)
    lens[rng.random(1100) < 0.05] = 0
    inp, dW, dU, dT = make_inputs(dict(C=C, batch=1, seqlen=0, num_qk_heads=2, num_v_heads=4,
                                       seed=126, gate_mu=4.0, dT=True,
                                       seqlens=[int(x) for x in lens]))
    say(f"wy_backward 1100 short sequences C={C}, tokens={int(lens.sum())}")
    out = run_bwd(inp, dW, dU, dT, gpu)
    check(inp, dW, dU, dT, out, f"1100 short sequences C={C}")


@pytest.mark.parametrize("C", [32, 64, 128])
def test_wy_backward_batch_walk(C, gpu):
    """Batch rows with more units than resident workgroups (432 at C = 64 and 128, 846 at C = 32)
    and 3 key heads, which divides neither grid: each workgroup's division-free walk over its
    units carries the head into the chunk slot and the chunk slot into the next row, on ragged
    rows (T = 1500, 3000 at C = 128), with two value heads per key head summed into dk."""
    inp, dW, dU, dT = make_inputs(dict(C=C, batch=6, seqlen=3000 if C == 128 else 1500,
                                       num_qk_heads=3, num_v_heads=6, seed=130, gate_mu=4.0,
                                       dT=True))
    say(f"wy_backward batch walk C={C}")
    out = run_bwd(inp, dW, dU, dT, gpu)
    check(inp, dW, dU, dT, out, f"batch walk C={C}")


@pytest.mark.parametrize("case", ["packed_gva_mu4_dT", "C128_gva8_mu4_dT"])
def test_wy_backward_deterministic(case, gpu):
    import torch
    inp, dW, dU, dT = make_inputs(CASES[case])
    a = run_bwd(inp, dW, dU, dT, gpu)
    b = run_bwd(inp, dW, dU, dT, gpu)
    assert all(torch.equal(x, y) for x, y in zip(a, b))


@pytest.mark.slow
@pytest.mark.parametrize("mu,C", [(None, 64), (4.0, 64), (None, 32), (4.0, 32), (None, 128),
                                  (4.0, 128)])
def test_wy_backward_full_size(mu, C, gpu):
    """B=1 T=8192 H=16/16, whole tensors against the oracle."""
    import torch
    w = synth.workload(2, chunk_size=C, gate_mu=mu)
    inp = synth.generate(w)
    inp["C"] = C
    rng = np.random.default_rng(7)
    B, T, Hv = inp["beta"].shape
    dW = synth.f32_to_bf16_bits(rng.standard_normal((B, T, Hv, 128)).astype(np.float32))
    dU = synth.f32_to_bf16_bits(rng.standard_normal((B, T, Hv, 128)).astype(np.float32))
    dT = rng.standard_normal((B, T, Hv, C)).astype(np.float32)
    say(f"wy_backward full {w.name} gate_mu={mu}")
    out = run_bwd(inp, dW, dU, dT, gpu)
    check(inp, dW, dU, dT, out, f"full {w.name} mu={mu}")
    del out
    torch.cuda.empty_cache()
