"""Every entry point of the preparation step at full size, whole tensors against the fp64 oracle
(needs a GPU).

Each seeded workload runs at C = 32, 64 and 128, ungated and with the seeded gate recipe
(g = log sigmoid(4 + N(0,1))), through wy_prepare (T, W, U), kkt_solve (T) and wu_prepare (W, U)
in the launch configuration the benchmark times.  Bar, over every stored entry: T within 1e-5
max-abs of the oracle, with its diagonal exactly 1 and strict upper triangle exactly 0; W and U
within 1e-2 relative Frobenius over the whole tensor; every output written (outputs are
pre-filled with NaN).  kkt_solve's T and wu_prepare's W, U must also equal wy_prepare's bit for
bit (one arithmetic).  The oracle runs one range of whole chunks at a time.
"""
import numpy as np
import pytest

from chunkwise_gated_deltanet_amd import synth
from gpu_util import check_structure, compare_all, run_all, say

pytestmark = pytest.mark.gpu


def check_entry_points(inp, gpu, label):
    import torch
    outs = run_all(inp, gpu)
    check_structure(outs["T"], inp)
    assert torch.equal(outs["T"], outs["T_kkt"]), "kkt_solve's T differs from wy_prepare's"
    assert torch.equal(outs["W"], outs["W_wu"]) and torch.equal(outs["U"], outs["U_wu"]), \
        "wu_prepare's W / U differ from wy_prepare's"
    compare_all(inp, outs, label=label)
    del outs
    torch.cuda.empty_cache()


# A mid-size packed-free shape with a ragged end whose unit count is at least three times the
# resident workgroups of every instance (T only: up to 7 per CU), so each persistent workgroup
# runs its loop over several units: 8000 tokens, Hq=12 / Hv=48 -> 12000 / 6000 / 3024 units.
@pytest.mark.parametrize("C", [32, 64, 128])
def test_mid_size_multi_unit(C, gpu):
    inp = synth.custom(1, 8000, 12, 48, C, seed=60 + C)
    say(f"mid size B=1 T=8000 H=12/48 C={C}")
    check_entry_points(inp, gpu, f"mid C={C}")


# Eight value heads per key head with enough units that the W / U instances take groups of two
# key heads (16 consecutive units per workgroup) and the r >= 4 occupancy (three workgroups per
# CU at C = 64, six at C = 32): 98304 packed tokens in 6 sequences, Hq=2 / Hv=16, gated.
@pytest.mark.parametrize("C", [32, 64])
def test_eight_value_heads_per_key_head(C, gpu):
    lens = [30000, 1, 20000, 18303, 0, 30000]
    inp = synth.custom(1, 0, 2, 16, C, seed=70 + C, gate_mu=4.0, seqlens=lens)
    say(f"Hq=2 Hv=16 packed {len(lens)} seqs, {sum(lens)} tokens, C={C}")
    check_entry_points(inp, gpu, f"r=8 C={C}")


def short_lengths(seed, count, C, zero_frac=0.05):
    """Lengths uniform in [1, C + 1], a few of them 0: most sequences are a single short chunk."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(1, C + 2, size=count)
    lens[rng.random(count) < zero_frac] = 0
    return [int(x) for x in lens]


# Many short packed sequences: the work map searches cu_seqlens for every unit (two rounds of the
# search for 1200 sequences, three for 5000) and skips the slots past each sequence's last chunk.
@pytest.mark.parametrize("C", [32, 64, 128])
def test_many_short_sequences(C, gpu):
    lens = short_lengths(90 + C, 1200, C)
    inp = synth.custom(1, 0, 4, 16, C, seed=95 + C, gate_mu=4.0, seqlens=lens)
    say(f"1200 packed sequences, lengths 1..{C + 1}, C={C}, tokens={sum(lens)}")
    check_entry_points(inp, gpu, f"1200 seqs C={C}")


def test_five_thousand_sequences(gpu):
    lens = short_lengths(99, 5000, 32)
    inp = synth.custom(1, 0, 1, 2, 32, seed=98, seqlens=lens)
    say(f"5000 packed sequences, lengths 1..33, C=32, tokens={sum(lens)}")
    check_entry_points(inp, gpu, "5000 seqs C=32")


FULL = [(i, c) for i in (1, 2, 3, 4, 5) for c in (32, 64, 128)]


@pytest.mark.slow
@pytest.mark.parametrize("idx,C", FULL, ids=[f"w{i}_C{c}" for i, c in FULL])
def test_full_size_every_entry(idx, C, gpu):
    """Ungated, then gated: the gates are drawn after k, v and beta, so both runs see the same
    k, v and beta (the ungated run drops g)."""
    w = synth.workload(idx, chunk_size=C, gate_mu=4.0)
    inp = synth.generate(w)
    tokens = inp["batch"] * inp["seqlen"]
    g = inp["g"]
    inp["g"] = None
    say(f"full size {w.name} C={C} ungated tokens={tokens}")
    check_entry_points(inp, gpu, f"{w.name} C={C} ungated")
    inp["g"] = g
    say(f"full size {w.name} C={C} gated (mu=4) tokens={tokens}")
    check_entry_points(inp, gpu, f"{w.name} C={C} gated")
