"""The seeded input generator (CPU only)."""
import numpy as np
import torch

from chunkwise_gated_deltanet_amd import synth


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = rng.standard_normal(100000).astype(np.float32) * np.float32(3.0)
    # exact ties: low 16 bits 0x8000 with both parities of the kept bit
    ties = (np.arange(2000, dtype=np.uint32) << np.uint32(16) | np.uint32(0x3F808000)).view(
        np.float32)
    x = np.concatenate([x, ties, np.array([0.0, -0.0, 1e-40, 65504.0], np.float32)])
    ours = synth.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = synth.bf16_bits_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(ours.view(np.int16)).view(torch.bfloat16)
                          .float().numpy())


def test_deterministic_and_shapes():
    a = synth.custom(2, 100, 2, 4, 32, seed=7)
    b = synth.custom(2, 100, 2, 4, 32, seed=7)
    for key in ("k", "v", "beta"):
        assert np.array_equal(a[key], b[key])
    assert a["k"].shape == (2, 100, 2, 128) and a["k"].dtype == np.uint16
    assert a["v"].shape == (2, 100, 4, 128) and a["beta"].shape == (2, 100, 4)
    kf = synth.bf16_bits_to_f32(a["k"]).astype(np.float64)
    assert np.max(np.abs(np.linalg.norm(kf, axis=-1) - 1)) < 1e-2
    assert np.all((a["beta"] > 0) & (a["beta"] < 1))


def test_packed_workload_lengths():
    w = synth.workload(5)
    rng = np.random.default_rng(w.seed)
    lens = synth.draw_seqlens(rng, 300, 16384, 8, 64)
    assert len(lens) == 8 and np.all(lens % 64 != 0)
    assert np.all((lens >= 300) & (lens <= 16384))


def test_workload_table():
    ws = synth.workloads()
    assert ws[2].chunk_size == 64 and ws[2].seqlen == 8192 and ws[2].num_v_heads == 16
    assert ws[2].beta_sigma == 1.5
    assert ws[1].dtype == "f32" and ws[1].chunk_size == 32
    assert ws[5].num_qk_heads == 16 and ws[5].num_v_heads == 64
    assert synth.workload(3, chunk_size=128).chunk_size == 128


def test_short_sequence_workload():
    inp = synth.generate(synth.workload(6))
    lens = np.diff(inp["cu_seqlens"].astype(np.int64))
    assert len(lens) == 1024 and lens.min() >= 1 and lens.max() <= 65 and np.all(lens % 64 != 0)
    assert inp["seqlen"] == int(lens.sum())
