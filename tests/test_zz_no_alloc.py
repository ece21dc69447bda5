"""wyp_chunk_fwd_cp_noalloc (the split forward on the library's static scratch, for callers that
cannot allocate) against wyp_chunk_fwd_cp with a caller workspace, through the C ABI (needs a
GPU).  Both run the same kernels on the same inputs, so o and the final state must agree bit for
bit; calls in a row, each smaller than the one before (the last one on packed sequences), so
a later call reads nothing an earlier one left behind."""
import ctypes

import numpy as np
import pytest

from chunkwise_gated_deltanet_amd import synth
from gpu_util import say

pytestmark = pytest.mark.gpu


def inputs(batch, seqlen, hq, hv, seed, gate_mu, device, seqlens=None):
    import torch
    import chunkwise_gated_deltanet_amd as cg
    inp = synth.custom(batch, seqlen, hq, hv, 64, seed=seed, gate_mu=gate_mu, with_q=True,
                       seqlens=seqlens)
    batch, seqlen = inp["batch"], inp["seqlen"]
    cu = None if inp["cu_seqlens"] is None else torch.from_numpy(inp["cu_seqlens"]).to(device)
    n = batch if cu is None else cu.numel() - 1
    bf = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
    k, v, q = bf(inp["k"]), bf(inp["v"]), bf(inp["q"])
    beta = torch.from_numpy(inp["beta"]).to(device)
    g = None if inp["g"] is None else torch.from_numpy(inp["g"]).to(device)
    W, U = cg.wu_prepare(k, v, beta, 64, g=g, cu_seqlens=cu)
    rng = np.random.default_rng(seed + 7)
    h0 = torch.from_numpy((0.1 * rng.standard_normal((n, hv, 128, 128))).astype(np.float32)).to(device)
    return dict(q=q, k=k, W=W, U=U, g=g, h0=h0, B=batch, T=seqlen, hq=hq, hv=hv, cu=cu, N=n)


def run(lib, x, seg, noalloc, device):
    import torch
    import chunkwise_gated_deltanet_amd as cg
    p = problem(x)
    o = torch.full((x["B"], x["T"], x["hv"], 128), float("nan"), dtype=torch.bfloat16, device=device)
    hT = torch.full((x["N"], x["hv"], 128, 128), float("nan"), dtype=torch.float32, device=device)
    gp = None if x["g"] is None else x["g"].data_ptr()
    cup = None if x["cu"] is None else x["cu"].data_ptr()
    stream = ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)
    args = (x["q"].data_ptr(), x["k"].data_ptr(), x["W"].data_ptr(), x["U"].data_ptr(), gp,
            x["h0"].data_ptr(), ctypes.c_float(128 ** -0.5), cup, seg)
    if noalloc:
        st = lib.wyp_chunk_fwd_cp_noalloc(ctypes.byref(p), *args, o.data_ptr(), hT.data_ptr(), stream)
    else:
        nbytes = lib.wyp_chunk_fwd_cp_workspace_bytes(ctypes.byref(p), cup, seg)
        ws = torch.empty(max(nbytes, 16) // 4, dtype=torch.float32, device=device)
        st = lib.wyp_chunk_fwd_cp(ctypes.byref(p), *args, ws.data_ptr(), nbytes, o.data_ptr(),
                                  hT.data_ptr(), stream)
    assert st == 0, lib.wyp_last_error().decode()
    torch.cuda.synchronize(device)
    return o, hT


def problem(x):
    import chunkwise_gated_deltanet_amd as cg
    return cg.Problem(x["B"], x["T"], x["hq"], x["hv"], 128, 128, 64,
                      0 if x["cu"] is None else x["N"], 0)


def test_noalloc_matches_workspace_entry_two_calls(gpu):
    import torch
    import chunkwise_gated_deltanet_amd as cg
    lib = cg.load_library()
    big = inputs(1, 8192, 16, 16, 500, 4.0, gpu)      # 8 segments of 16 chunks: 15 MiB of scratch
    small = inputs(2, 1000, 2, 4, 501, None, gpu)      # then 4 segments of 4 chunks, ragged
    packed = inputs(1, 0, 2, 4, 502, 4.0, gpu, seqlens=[700, 0, 90, 1, 257])  # then packed
    for x, seg in ((big, 16), (small, 4), (packed, 2)):
        p = problem(x)
        need = lib.wyp_chunk_fwd_cp_workspace_bytes(ctypes.byref(p), None if x["cu"] is None
                                                    else ctypes.c_void_p(x["cu"].data_ptr()), seg)
        say(f"noalloc B={x['B']} T={x['T']} N={x['N']} Hv={x['hv']} segment_chunks={seg} "
            f"scratch={need}")
        assert 0 < need <= 32 * 1024 * 1024
        o1, h1 = run(lib, x, seg, False, gpu)
        o2, h2 = run(lib, x, seg, True, gpu)
        assert not torch.isnan(o2).any() and not torch.isnan(h2).any()
        assert torch.equal(o1, o2) and torch.equal(h1, h2)
