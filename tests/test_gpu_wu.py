"""wu_prepare: W and U without T in HBM (needs a GPU).

[Inv] section 1 materialises T only because W and U both reuse it; this entry point keeps it
on chip.  Its W and U must equal wy_prepare's bit for bit (same arithmetic) and the oracle's
within the W/U tolerance.
"""
import pytest

from chunkwise_gated_deltanet_amd import synth
from gpu_util import compare_full, gate_of, run_wy, say, to_device

pytestmark = pytest.mark.gpu

CASES = {
    "packed_gva_C32": dict(batch=1, seqlen=0, num_qk_heads=2, num_v_heads=8, chunk_size=32,
                           seed=70, seqlens=[31, 33, 1, 95, 200]),
    "B2_C64": dict(batch=2, seqlen=333, num_qk_heads=4, num_v_heads=4, chunk_size=64, seed=71),
    "packed_C128": dict(batch=1, seqlen=0, num_qk_heads=2, num_v_heads=4, chunk_size=128,
                        seed=72, seqlens=[127, 129, 1, 300, 17]),
    "fp32_C64": dict(batch=1, seqlen=200, num_qk_heads=2, num_v_heads=2, chunk_size=64,
                     dtype="f32", seed=73),
    "fp32_C128": dict(batch=1, seqlen=0, num_qk_heads=1, num_v_heads=2, chunk_size=128,
                      dtype="f32", seed=74, seqlens=[300, 1, 128]),
}


def run_wu(inp, device):
    import torch
    import chunkwise_gated_deltanet_amd as cg
    k, v, beta, cu = to_device(inp, device)
    B, T, _, dk = k.shape
    Hv = beta.shape[2]
    W = torch.full((B, T, Hv, dk), float("nan"), dtype=k.dtype, device=device)
    U = torch.full((B, T, Hv, v.shape[3]), float("nan"), dtype=k.dtype, device=device)
    cg.wu_prepare(k, v, beta, inp["chunk_size"], cu_seqlens=cu, W_out=W, U_out=U,
                  g=gate_of(inp, device))
    torch.cuda.synchronize(device)
    return W, U


@pytest.mark.parametrize("name", sorted(CASES))
def test_wu_prepare_matches_wy_prepare_and_oracle(name, gpu):
    import torch
    inp = synth.custom(**CASES[name])
    say(f"wu_prepare {name}")
    W, U = run_wu(inp, gpu)
    T0, W0, U0 = run_wy(inp, gpu)
    assert torch.equal(W, W0) and torch.equal(U, U0)
    compare_full(inp, T0, W, U, label="wu " + name)
