"""HIP path vs the fp64 oracle, element by element, through the C ABI (needs a GPU).

Bar: T within 1e-5 max-abs (fp32 T); W and U within 1e-2 relative Frobenius (bf16 outputs);
T's diagonal exactly 1 and strict upper triangle exactly 0; every output entry written
(outputs are pre-filled with NaN).
"""
import pytest

from chunkwise_gated_deltanet_amd import synth
from gpu_util import check_structure, compare_full, run_wy, say

pytestmark = pytest.mark.gpu

# Reduced sizes the oracle finishes in seconds; each spans several chunks and ends ragged.
SMALL = {
    "w1_tiny_fp32_C32": dict(idx=1),
    "w2_shape_T700_C64": dict(batch=1, seqlen=700, num_qk_heads=16, num_v_heads=16,
                              chunk_size=64, beta_sigma=1.5, seed=2),
    "w3_shape_B2_T333_C32": dict(batch=2, seqlen=333, num_qk_heads=4, num_v_heads=4,
                                 chunk_size=32, seed=3),
    "w3_shape_B2_T333_C64": dict(batch=2, seqlen=333, num_qk_heads=4, num_v_heads=4,
                                 chunk_size=64, seed=3),
    "w3_shape_B2_T333_C128": dict(batch=2, seqlen=333, num_qk_heads=4, num_v_heads=4,
                                  chunk_size=128, seed=3),
    "w4_shape_T1000_C128": dict(batch=1, seqlen=1000, num_qk_heads=2, num_v_heads=2,
                                chunk_size=128, seed=4),
    "w5_shape_packed_gva_C64": dict(batch=1, seqlen=0, num_qk_heads=4, num_v_heads=16,
                                    chunk_size=64, seed=5,
                                    seqlens=[300, 517, 64, 1, 129, 250, 63, 65]),
    "packed_gva_C32": dict(batch=1, seqlen=0, num_qk_heads=2, num_v_heads=8, chunk_size=32,
                           seed=6, seqlens=[31, 33, 1, 95, 200]),
    "packed_gva_C128": dict(batch=1, seqlen=0, num_qk_heads=2, num_v_heads=4, chunk_size=128,
                            seed=7, seqlens=[127, 129, 1, 300, 17]),
    "fp32_C64": dict(batch=1, seqlen=200, num_qk_heads=2, num_v_heads=2, chunk_size=64,
                     dtype="f32", seed=8),
    "fp32_packed_gva_C128": dict(batch=1, seqlen=0, num_qk_heads=1, num_v_heads=2,
                                 chunk_size=128, dtype="f32", seed=9, seqlens=[300, 1, 128]),
}


def small_inputs(spec):
    spec = dict(spec)
    if "idx" in spec:
        return synth.generate(synth.workload(spec["idx"]))
    return synth.custom(**spec)


@pytest.mark.parametrize("name", sorted(SMALL))
def test_wy_prepare_small(name, gpu):
    inp = small_inputs(SMALL[name])
    say(f"wy_prepare small {name}")
    T, W, U = run_wy(inp, gpu)
    check_structure(T, inp)
    compare_full(inp, T, W, U, label=name)


@pytest.mark.parametrize("name", ["w3_shape_B2_T333_C32", "w3_shape_B2_T333_C64",
                                  "w3_shape_B2_T333_C128", "w5_shape_packed_gva_C64",
                                  "w1_tiny_fp32_C32"])
def test_kkt_solve_small(name, gpu):
    inp = small_inputs(SMALL[name])
    say(f"kkt_solve small {name}")
    T, _, _ = run_wy(inp, gpu, kkt_only=True)
    check_structure(T, inp)
    compare_full(inp, T, None, None, label="kkt " + name)


def test_kkt_solve_matches_wy_prepare(gpu):
    """The T of both entry points is bit-identical."""
    import torch
    inp = small_inputs(SMALL["w5_shape_packed_gva_C64"])
    T1, _, _ = run_wy(inp, gpu)
    T2, _, _ = run_wy(inp, gpu, kkt_only=True)
    assert torch.equal(T1, T2)
