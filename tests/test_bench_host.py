"""Host logic of bench.py: the one-GPU guard, the algorithmic byte counts behind the roofline,
and the profile naming and counter lookup (no GPU, no kernel calls)."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402
from chunkwise_gated_deltanet_amd import synth  # noqa: E402


def test_more_than_one_gpu_is_refused(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err


def test_headline_bytes_from_tensor_sizes():
    # B=1, T=8192, H_q=H_v=16, d_k=d_v=128, C=64, bf16 k/v/W/U, fp32 beta and T.  Counted
    # tensor by tensor: k, v and beta read once; T (C fp32 per row), W and U written once.
    tok, h, d, C = 8192, 16, 128, 64
    reads = tok * h * d * 2 + tok * h * d * 2 + tok * h * 4
    writes = tok * h * C * 4 + tok * h * d * 2 + tok * h * d * 2
    assert reads == 67_633_152 and writes == 100_663_296
    assert bench.algorithmic_bytes(tok, h, h, d, d, C, 2) == reads + writes


@pytest.mark.parametrize("C", [32, 64, 128])
def test_grouped_heads_read_k_once_per_key_head(C):
    # H_v = 4 H_q: k is read once per key head, everything else once per value head.
    tok, hq, hv, d = 1000, 16, 64, 128
    k_bytes = tok * hq * d * 2
    per_v_head = tok * hv * (d * 2 + 4 + 4 * C + d * 2 + d * 2)
    assert bench.algorithmic_bytes(tok, hq, hv, d, d, C, 2) == k_bytes + per_v_head
    # without T (W and U only) and T only
    assert bench.algorithmic_bytes(tok, hq, hv, d, d, C, 2, entry="wu") == \
        k_bytes + tok * hv * (d * 2 + 4 + d * 2 + d * 2)
    assert bench.algorithmic_bytes(tok, hq, hv, d, d, C, 2, entry="kkt") == \
        k_bytes + tok * hv * (4 + 4 * C)
    # log gates: one more fp32 read per token and value head
    assert bench.algorithmic_bytes(tok, hq, hv, d, d, C, 2, gated=True) - \
        bench.algorithmic_bytes(tok, hq, hv, d, d, C, 2) == tok * hv * 4


def test_profile_names():
    w = synth.workload(2)
    assert bench.profile_name("wy", w, 1, 8192, 0) == "wy_prepare_bf16_c64_b1t8192h16"
    g = synth.workload(2, gate_mu=4.0)
    assert bench.profile_name("wy", g, 1, 8192, 0) == "wy_prepare_gated_bf16_c64_b1t8192h16"
    p = synth.workload(5)
    assert bench.profile_name("kkt", p, 1, 1000, 8) == \
        f"kkt_solve_bf16_c{p.chunk_size}_packed8_hq{p.num_qk_heads}hv{p.num_v_heads}"


def test_counter_traffic_is_tied_to_the_source(tmp_path, monkeypatch):
    # a summary taken on another source is ignored; one taken on this source is read
    name = "wy_prepare_bf16_c64_b1t9h1"
    prof = tmp_path / "profiles"
    prof.mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    (prof / (name + "_counters.md")).write_text(
        "traffic_bytes_per_launch: 12345\nkernel_source_sha256: " + "0" * 64 + "\n")
    assert bench.counter_traffic(name) is None
    (prof / (name + "_counters.md")).write_text(
        "traffic_bytes_per_launch: 12345\nkernel_source_sha256: " + bench.kernel_source_sha() + "\n")
    assert bench.counter_traffic(name) == 12345.0
    assert bench.counter_traffic("no_such_profile") is None


def test_committed_headline_counters_are_near_the_algorithmic_bytes():
    # Where the committed headline summary matches the current source, the HBM bytes it
    # measured lie between the algorithmic bytes and 1.1 times them (no large re-reads).
    t = bench.counter_traffic("wy_prepare_bf16_c64_b1t8192h16")
    if t is None:
        pytest.skip("headline counter summary was taken on another kernel source")
    alg = bench.algorithmic_bytes(8192, 16, 16, 128, 128, 64, 2)
    assert 0.99 * alg <= t <= 1.1 * alg


def test_extra_workloads_cover_the_c64_configs_and_the_chunk_study():
    extras = bench.parse_extras(bench.DEFAULT_EXTRAS)
    wy = [(i, c) for e, i, c, seg in extras if e == "wy"]
    assert (3, 64) in wy and (5, 64) in wy
    assert {c for i, c in wy if i == 3} == {32, 64, 128}
    # the backward and the sequence-parallel recurrence on the headline's shape ride along
    assert {c for e, i, c, seg in extras if e == "bwd" and i == 2} == {32, 64, 128}
    assert ("fwd", 2, 64, "auto") in extras
    assert bench.parse_extras("none") == [] and bench.parse_extras("2:32") == [("wy", 2, 32, None)]
    assert bench.parse_extras("2:32", "kkt") == [("kkt", 2, 32, None)]
    assert bench.parse_extras("gdn/2:64/16") == [("gdn", 2, 64, "16")]
    with pytest.raises(ValueError):
        bench.parse_extras("nope/2:64")


def test_cpu_threads_are_capped_and_host_cores_recorded():
    assert 1 <= bench.cpu_threads() <= min(16, bench.host_cores())


def test_solve_bytes():
    # one right-hand side: k once per key head; R, beta read and X written per value head
    tok, hq, hv, d = 1000, 16, 64, 128
    assert bench.algorithmic_bytes(tok, hq, hv, d, d, 64, 2, entry="solve") == \
        tok * (hq * d * 2 + hv * (d * 2 + 4 + d * 2))
    assert bench.profile_name("solve", synth.workload(2), 1, 8192, 0) == "solve_rhs_bf16_c64_b1t8192h16"


def test_split_forward_reads_its_own_profile():
    # the split form's summary covers its three kernels; the unsplit one is another file
    w = synth.workload(2)
    assert bench.profile_name("fwd", w, 1, 8192, 0) == "chunk_fwd_bf16_c64_b1t8192h16"
    assert bench.profile_name("fwd", w, 1, 8192, 0, 16) == "chunk_fwd_cp16_bf16_c64_b1t8192h16"
    assert bench.profile_name("wy", w, 1, 8192, 0, 16) == "wy_prepare_bf16_c64_b1t8192h16"
    t = bench.counter_traffic("chunk_fwd_cp16_bf16_c64_b1t8192h16", "fwd")
    if t is None:
        pytest.skip("split forward counter summary was taken on another kernel source")
    alg = bench.fwd_bytes(8192, 1, 16, 16, 128, 128, 2, False)
    assert 1.5 * alg < t < 2.0 * alg  # two passes over K, W, U and the workspace round trip
