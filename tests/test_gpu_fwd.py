"""The chunked forward (wyp_chunk_fwd, after wu_prepare) against the gated delta rule stepped
token by token in fp64 (oracle.gdn_forward), through the C ABI (needs a GPU).

The FlashQLA usage section returns o and final_state from q, k, v, g, beta, scale and
initial_state; the recurrence is S_t = alpha_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T,
o_t = scale S_t^T q_t.  The chunked path differs from it only by rounding: W, U, o are bf16 and
the state enters its products with W and Q as bf16.  Bar (derived from that arithmetic: bf16
rounding of W, U, the state operand and o gives about 4e-3 relative in a simulation over 8192
tokens, with no growth along the sequence): o and the final state within 1e-2 relative
Frobenius; every output entry written (o is pre-filled with NaN).
"""
import numpy as np
import pytest

import oracle
from chunkwise_gated_deltanet_amd import synth
from gpu_util import gate_of, oracle_threads, rel_fro, say, to_device, to_f64

pytestmark = pytest.mark.gpu

FWD_TOL = 1e-2

CASES = {
    "B2_T333_H4": dict(batch=2, seqlen=333, num_qk_heads=4, num_v_heads=4, seed=100),
    "B2_T333_H4_mu4_h0": dict(batch=2, seqlen=333, num_qk_heads=4, num_v_heads=4, seed=101,
                              gate_mu=4.0, h0=True),
    "packed_gva_mu4": dict(batch=1, seqlen=0, num_qk_heads=4, num_v_heads=16, seed=102,
                           gate_mu=4.0, seqlens=[300, 517, 64, 1, 129, 250, 63, 65]),
    "packed_gva_mu0_h0": dict(batch=1, seqlen=0, num_qk_heads=2, num_v_heads=8, seed=103,
                              gate_mu=0.0, h0=True, seqlens=[31, 33, 1, 95, 200]),
    "T2048_H2_ungated_h0": dict(batch=1, seqlen=2048, num_qk_heads=2, num_v_heads=2, seed=104,
                                h0=True),
    "packed_empty_seq_mu2_h0": dict(batch=1, seqlen=0, num_qk_heads=1, num_v_heads=2, seed=105,
                                    gate_mu=2.0, h0=True, seqlens=[100, 0, 70, 0]),
    # 128 or more (sequence, value head) pairs: the launch takes 64-column slices of the state
    # (two workgroups per pair) instead of 32-column ones once that gives every CU one.
    "wide_B8_T321_H4_16_mu4_h0": dict(batch=8, seqlen=321, num_qk_heads=4, num_v_heads=16,
                                      seed=106, gate_mu=4.0, h0=True),
    "wide_B16_T130_H8_ungated": dict(batch=16, seqlen=130, num_qk_heads=8, num_v_heads=8, seed=107),
    "wide_packed_40_mu0_h0": dict(batch=1, seqlen=0, num_qk_heads=2, num_v_heads=4, seed=108,
                                  gate_mu=0.0, h0=True,
                                  seqlens=[1, 0, 64, 65, 127, 129, 200, 31, 33, 63] * 4),
    # the other chunk sizes the preparation step supports: C = 32 (two waves per workgroup) and
    # C = 128 (eight waves; gates two per lane)
    "C32_B2_T333_H4_mu4_h0": dict(C=32, batch=2, seqlen=333, num_qk_heads=4, num_v_heads=4,
                                  seed=109, gate_mu=4.0, h0=True),
    "C32_packed_gva_ungated": dict(C=32, batch=1, seqlen=0, num_qk_heads=2, num_v_heads=8,
                                   seed=110, seqlens=[31, 32, 33, 1, 0, 95, 200]),
    "C32_wide_B8_T200_H4_16_mu2": dict(C=32, batch=8, seqlen=200, num_qk_heads=4,
                                       num_v_heads=16, seed=111, gate_mu=2.0),
    "C128_B2_T333_H2_4_mu4_h0": dict(C=128, batch=2, seqlen=333, num_qk_heads=2, num_v_heads=4,
                                     seed=112, gate_mu=4.0, h0=True),
    "C128_packed_mu0_h0": dict(C=128, batch=1, seqlen=0, num_qk_heads=1, num_v_heads=2,
                               seed=113, gate_mu=0.0, h0=True,
                               seqlens=[127, 128, 129, 1, 0, 300, 64]),
    "C128_wide_B8_T300_H4_16_ungated": dict(C=128, batch=8, seqlen=300, num_qk_heads=4,
                                            num_v_heads=16, seed=114),
}


def make_inputs(spec):
    spec = dict(spec)
    want_h0 = spec.pop("h0", False)
    C = spec.pop("C", 64)
    inp = synth.custom(chunk_size=C, with_q=True, **spec)
    inp["C"] = C
    N = inp["batch"] if inp["cu_seqlens"] is None else len(inp["cu_seqlens"]) - 1
    Hv = inp["beta"].shape[2]
    h0 = None
    if want_h0:
        rng = np.random.default_rng(spec["seed"] + 1000)
        h0 = (0.1 * rng.standard_normal((N, Hv, 128, 128))).astype(np.float32)
    return inp, h0


def q_of(inp, device):
    import torch
    return torch.from_numpy(inp["q"].view(np.int16)).view(torch.bfloat16).to(device)


def run_fwd(inp, h0, device, in_place=False):
    """wu_prepare then chunk_fwd; o pre-filled with NaN."""
    import torch
    import chunkwise_gated_deltanet_amd as cg
    k, v, beta, cu = to_device(inp, device)
    q = q_of(inp, device)
    g = gate_of(inp, device)
    C = inp.get("C", 64)
    W, U = cg.wu_prepare(k, v, beta, C, cu_seqlens=cu, g=g)
    o = torch.full(v.shape, float("nan"), dtype=v.dtype, device=device)
    h0d = None if h0 is None else torch.from_numpy(h0).to(device)
    if in_place:
        o, hT = cg.chunk_fwd(q, k, W, U, C, g=g, initial_state=h0d, cu_seqlens=cu,
                             o_out=o, final_state=h0d)
    else:
        o, hT = cg.chunk_fwd(q, k, W, U, C, g=g, initial_state=h0d, cu_seqlens=cu,
                             o_out=o, output_final_state=True)
    torch.cuda.synchronize(device)
    return o, hT


def oracle_fwd(inp, h0, pairs=None):
    return oracle.gdn_forward(inp["q"], inp["k"], inp["v"], inp["beta"], g=inp.get("g"), h0=h0,
                              cu_seqlens=inp["cu_seqlens"], pairs=pairs)


@pytest.mark.parametrize("name", sorted(CASES))
def test_chunk_fwd_small(name, gpu):
    import torch
    inp, h0 = make_inputs(CASES[name])
    say(f"chunk_fwd {name}")
    o, hT = run_fwd(inp, h0, gpu)
    assert not torch.isnan(o).any(), "unwritten o entries"
    o_ref, h_ref = oracle_fwd(inp, h0)
    ro, rh = rel_fro(to_f64(o), o_ref), rel_fro(to_f64(hT), h_ref)
    say(f"[{name}] o rel fro {ro:.3e}, final state rel fro {rh:.3e}")
    assert ro <= FWD_TOL and rh <= FWD_TOL, (ro, rh)
    if inp["cu_seqlens"] is not None:
        lens = np.diff(inp["cu_seqlens"])
        for s in np.nonzero(lens == 0)[0]:  # an empty sequence hands its initial state back
            want = np.zeros(hT[s].shape, np.float32) if h0 is None else h0[s]
            assert np.array_equal(hT[s].cpu().numpy(), want)


def test_chunk_fwd_in_place_state(gpu):
    """initial_state and final_state may be one buffer."""
    import torch
    inp, h0 = make_inputs(CASES["B2_T333_H4_mu4_h0"])
    o1, h1 = run_fwd(inp, h0, gpu)
    o2, h2 = run_fwd(inp, h0, gpu, in_place=True)
    assert torch.equal(o1, o2) and torch.equal(h1, h2)


def test_chunk_gated_delta_rule_api(gpu):
    """The one-call API (the FlashQLA usage argument list) equals wu_prepare + chunk_fwd."""
    import torch
    import chunkwise_gated_deltanet_amd as cg
    inp, h0 = make_inputs(CASES["packed_gva_mu0_h0"])
    o1, h1 = run_fwd(inp, h0, gpu)
    k, v, beta, cu = to_device(inp, gpu)
    o2, h2 = cg.chunk_gated_delta_rule(q_of(inp, gpu), k, v, gate_of(inp, gpu), beta,
                                       initial_state=torch.from_numpy(h0).to(gpu),
                                       output_final_state=True, cu_seqlens=cu)
    torch.cuda.synchronize(gpu)
    assert torch.equal(o1, o2) and torch.equal(h1, h2)


# Full sizes: every (sequence, value head) pair against the oracle, whole tensors, with the worst
# pair reported; every output entry written.  C = 64, and the other chunk sizes on one workload
# each.
FULL = [(2, None, 64), (2, 4.0, 64), (3, None, 64), (5, 4.0, 64), (4, None, 128), (2, 4.0, 32)]


def compare_pairs(inp, o, hT, o_ref, h_ref, label):
    """Whole-tensor relative Frobenius of o and the final state, plus the worst single pair."""
    B, T = inp["batch"], inp["seqlen"]
    Hv = inp["beta"].shape[2]
    cu = inp["cu_seqlens"]
    N = B if cu is None else len(cu) - 1
    starts = (np.arange(N) * T if cu is None else cu[:-1]).astype(np.int64)
    ends = (starts + T if cu is None else cu[1:]).astype(np.int64)
    og, rf = to_f64(o).reshape(-1, Hv, 128), o_ref.reshape(-1, Hv, 128)
    hg = to_f64(hT)
    ro, rh = rel_fro(og, rf), rel_fro(hg, h_ref)
    worst = 0.0
    for s in range(N):
        for h in range(Hv):
            if ends[s] > starts[s]:
                worst = max(worst, rel_fro(og[starts[s]:ends[s], h], rf[starts[s]:ends[s], h]))
            worst = max(worst, rel_fro(hg[s, h], h_ref[s, h]))
    say(f"[{label}] o rel fro {ro:.3e}, final state rel fro {rh:.3e}, worst pair {worst:.3e}")
    assert ro <= FWD_TOL and rh <= FWD_TOL, (ro, rh)
    return worst


@pytest.mark.slow
@pytest.mark.parametrize("idx,mu,C", FULL,
                         ids=[f"w{i}_{'mu' + str(m) if m else 'ungated'}_C{c}" for i, m, c in FULL])
def test_chunk_fwd_full_size(idx, mu, C, gpu):
    import torch
    w = synth.workload(idx, chunk_size=C, gate_mu=mu, with_q=True)
    inp = synth.generate(w)
    inp["C"] = C
    say(f"chunk_fwd full {w.name} gate_mu={mu} tokens={inp['batch'] * inp['seqlen']}")
    o, hT = run_fwd(inp, None, gpu)
    assert not torch.isnan(o).any(), "unwritten o entries"
    o_ref, h_ref = oracle.gdn_forward(inp["q"], inp["k"], inp["v"], inp["beta"], g=inp.get("g"),
                                      cu_seqlens=inp["cu_seqlens"], nthreads=oracle_threads())
    compare_pairs(inp, o, hT, o_ref, h_ref, f"full {w.name} mu={mu}")
    del o, hT
    torch.cuda.empty_cache()


# Sequence-parallel forward (wyp_chunk_fwd_cp): per-segment transitions, an fp32 combine, then
# the forward per segment.  Same oracle, same bar; segment lengths cover a single chunk, a
# ragged last segment and a single segment.
CP_CASES = {
    "B1_T1000_H2_seg1": (dict(batch=1, seqlen=1000, num_qk_heads=2, num_v_heads=2, seed=130), 1),
    "B2_T700_H2_mu4_h0_seg3": (dict(batch=2, seqlen=700, num_qk_heads=1, num_v_heads=2, seed=131,
                                    gate_mu=4.0, h0=True), 3),
    "B1_T2048_H4_mu0_seg5": (dict(batch=1, seqlen=2048, num_qk_heads=4, num_v_heads=4, seed=132,
                                  gate_mu=0.0), 5),
    "B1_T2048_H2_ungated_h0_seg8": (dict(batch=1, seqlen=2048, num_qk_heads=2, num_v_heads=2,
                                         seed=133, h0=True), 8),
    "B1_T333_H2_one_segment": (dict(batch=1, seqlen=333, num_qk_heads=2, num_v_heads=2, seed=134), 6),
    # 17 segments x 8 value heads: 64-column slices in both kernel passes
    "wide_B1_T2100_H2_8_mu4_h0_seg2": (dict(batch=1, seqlen=2100, num_qk_heads=2, num_v_heads=8,
                                            seed=136, gate_mu=4.0, h0=True), 2),
    # Packed sequences: segments start at each sequence's first chunk; one-segment, empty and
    # one-token sequences run beside split ones (segment lengths 1 .. 4 chunks, ragged tails)
    "packed_mu4_h0_seg2": (dict(batch=1, seqlen=0, num_qk_heads=2, num_v_heads=4, seed=137,
                                gate_mu=4.0, h0=True,
                                seqlens=[700, 0, 90, 1, 257, 64, 65, 128, 129]), 2),
    "packed_one_long_many_short_mu0_h0_seg4": (dict(batch=1, seqlen=0, num_qk_heads=1,
                                                    num_v_heads=8, seed=138, gate_mu=0.0, h0=True,
                                                    seqlens=[4000] + [5, 63, 64, 65, 0] * 8), 4),
    "packed_ungated_seg1": (dict(batch=1, seqlen=0, num_qk_heads=2, num_v_heads=2, seed=139,
                                 seqlens=[300, 1, 513]), 1),
    # 64-column slices: 14 sequences, Hv = 16
    "wide_packed_mu4_seg3": (dict(batch=1, seqlen=0, num_qk_heads=4, num_v_heads=16, seed=140,
                                  gate_mu=4.0, seqlens=[1000, 333, 64, 0, 1, 2000, 150] * 2), 3),
    # C = 32 and 128: segments of segment_chunks x C tokens
    "C32_B1_T1000_H2_mu4_h0_seg5": (dict(C=32, batch=1, seqlen=1000, num_qk_heads=2,
                                         num_v_heads=2, seed=141, gate_mu=4.0, h0=True), 5),
    "C32_packed_seg3": (dict(C=32, batch=1, seqlen=0, num_qk_heads=1, num_v_heads=4, seed=142,
                             seqlens=[500, 0, 33, 1, 250]), 3),
    "C128_B1_T2100_H2_8_h0_seg3": (dict(C=128, batch=1, seqlen=2100, num_qk_heads=2,
                                        num_v_heads=8, seed=143, h0=True), 3),
    "C128_packed_mu4_seg2": (dict(C=128, batch=1, seqlen=0, num_qk_heads=2, num_v_heads=4,
                                  seed=144, gate_mu=4.0, seqlens=[1300, 1, 0, 256, 257, 90]), 2),
    # 150 sequences: the owner search over cu_seqlens takes two 64-ary levels
    "packed_150_mu2_h0_seg2": (dict(batch=1, seqlen=0, num_qk_heads=1, num_v_heads=2, seed=145,
                                    gate_mu=2.0, h0=True,
                                    seqlens=[int(x) for x in
                                             np.random.default_rng(145).integers(0, 300, 150)]), 2),
}


def run_fwd_cp(inp, h0, device, seg):
    import torch
    import chunkwise_gated_deltanet_amd as cg
    k, v, beta, cu = to_device(inp, device)
    q = q_of(inp, device)
    g = gate_of(inp, device)
    C = inp.get("C", 64)
    W, U = cg.wu_prepare(k, v, beta, C, g=g, cu_seqlens=cu)
    o = torch.full(v.shape, float("nan"), dtype=v.dtype, device=device)
    h0d = None if h0 is None else torch.from_numpy(h0).to(device)
    o, hT = cg.chunk_fwd(q, k, W, U, C, g=g, initial_state=h0d, o_out=o, cu_seqlens=cu,
                         output_final_state=True, segment_chunks=seg)
    torch.cuda.synchronize(device)
    return o, hT


@pytest.mark.parametrize("name", sorted(CP_CASES))
def test_chunk_fwd_cp(name, gpu):
    import torch
    spec, seg = CP_CASES[name]
    inp, h0 = make_inputs(spec)
    say(f"chunk_fwd_cp {name} segment_chunks={seg}")
    o, hT = run_fwd_cp(inp, h0, gpu, seg)
    assert not torch.isnan(o).any(), "unwritten o entries"
    o_ref, h_ref = oracle_fwd(inp, h0)
    ro, rh = rel_fro(to_f64(o), o_ref), rel_fro(to_f64(hT), h_ref)
    say(f"[cp {name}] o rel fro {ro:.3e}, final state rel fro {rh:.3e}")
    assert ro <= FWD_TOL and rh <= FWD_TOL, (ro, rh)
    if inp["cu_seqlens"] is not None:
        worst = compare_pairs(inp, o, hT, o_ref, h_ref, f"cp {name} per pair")
        assert worst <= 2 * FWD_TOL, worst
        for s in np.nonzero(np.diff(inp["cu_seqlens"]) == 0)[0]:  # empty: the initial state back
            want = np.zeros((inp["beta"].shape[2], 128, 128), np.float32) if h0 is None else h0[s]
            assert np.array_equal(hT[s].cpu().numpy(), want)


def test_chunk_fwd_cp_packed_in_place_state(gpu):
    """Packed split forward with final_state = initial_state: the split sequences' segment 0
    reads the combine's copy, the one-segment sequences read and write their own state in one
    workgroup."""
    import torch
    import chunkwise_gated_deltanet_amd as cg
    spec, seg = CP_CASES["packed_mu4_h0_seg2"]
    inp, h0 = make_inputs(spec)
    say("chunk_fwd_cp packed in place, segment_chunks=2")
    k, v, beta, cu = to_device(inp, gpu)
    q = q_of(inp, gpu)
    g = gate_of(inp, gpu)
    W, U = cg.wu_prepare(k, v, beta, 64, g=g, cu_seqlens=cu)
    o1, h1 = cg.chunk_fwd(q, k, W, U, 64, g=g, initial_state=torch.from_numpy(h0).to(gpu),
                          cu_seqlens=cu, output_final_state=True, segment_chunks=seg)
    state = torch.from_numpy(h0).to(gpu)
    o2, h2 = cg.chunk_fwd(q, k, W, U, 64, g=g, initial_state=state, final_state=state,
                          cu_seqlens=cu, segment_chunks=seg)
    torch.cuda.synchronize(gpu)
    assert h2.data_ptr() == state.data_ptr()
    assert torch.equal(o1, o2) and torch.equal(h1, h2)


def test_chunk_fwd_cp_in_place_state(gpu):
    """Split forward with final_state = initial_state: segment 0 starts from the combine's copy
    of the initial state, so the last segment's write cannot reach it.  B=2 T=4096 H=8 with
    4-chunk segments runs 1024 output-pass workgroups, more than one resident round (768), so
    last segments do finish while first segments are still waiting to start."""
    import torch
    import chunkwise_gated_deltanet_amd as cg
    inp, h0 = make_inputs(dict(batch=2, seqlen=4096, num_qk_heads=4, num_v_heads=8, seed=135,
                               gate_mu=4.0, h0=True))
    say("chunk_fwd_cp in place, B=2 T=4096 H=4/8, segment_chunks=4")
    k, v, beta, _ = to_device(inp, gpu)
    q = q_of(inp, gpu)
    g = gate_of(inp, gpu)
    W, U = cg.wu_prepare(k, v, beta, 64, g=g)
    o1, h1 = cg.chunk_fwd(q, k, W, U, 64, g=g, initial_state=torch.from_numpy(h0).to(gpu),
                          output_final_state=True, segment_chunks=4)
    state = torch.from_numpy(h0).to(gpu)
    o2, h2 = cg.chunk_fwd(q, k, W, U, 64, g=g, initial_state=state, final_state=state,
                          segment_chunks=4)
    torch.cuda.synchronize(gpu)
    assert h2.data_ptr() == state.data_ptr()
    assert torch.equal(o1, o2) and torch.equal(h1, h2)
    o_ref, h_ref = oracle_fwd(inp, h0)
    ro, rh = rel_fro(to_f64(o2), o_ref), rel_fro(to_f64(h2), h_ref)
    say(f"[cp in place] o rel fro {ro:.3e}, final state rel fro {rh:.3e}")
    assert ro <= FWD_TOL and rh <= FWD_TOL, (ro, rh)


@pytest.mark.slow
@pytest.mark.parametrize("mu", [None, 4.0])
def test_chunk_fwd_cp_full_size(mu, gpu):
    """B=1 T=8192 H=16/16 C=64 with the automatic segment length, every head."""
    import torch
    import chunkwise_gated_deltanet_amd as cg
    w = synth.workload(2, chunk_size=64, gate_mu=mu, with_q=True)
    inp = synth.generate(w)
    seg = cg.cp_segment_chunks(1, 8192, 16)
    say(f"chunk_fwd_cp full {w.name} gate_mu={mu} segment_chunks={seg}")
    o, hT = run_fwd_cp(inp, None, gpu, seg)
    assert not torch.isnan(o).any()
    o_ref, h_ref = oracle.gdn_forward(inp["q"], inp["k"], inp["v"], inp["beta"], g=inp.get("g"),
                                      nthreads=oracle_threads())
    compare_pairs(inp, o, hT, o_ref, h_ref, f"cp full {w.name} mu={mu} segment_chunks={seg}")
