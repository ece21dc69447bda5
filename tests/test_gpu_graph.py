"""wy_prepare under HIP graph capture (needs a GPU).

The benchmark replays captured launches, so every replay must equal the eager result.  The
graph is replayed several times with eager work and synchronisations in between, and the
outputs are cleared before each replay so a replay that does nothing cannot pass.
"""
import numpy as np
import pytest

from chunkwise_gated_deltanet_amd import synth
from gpu_util import compare_full, say, to_device

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("C", [32, 64, 128])
def test_graph_replays_match_eager(C, gpu):
    import torch
    import chunkwise_gated_deltanet_amd as cg
    inputs = [synth.custom(1, 0, 2, 4, C, seed=90 + C, seqlens=[3 * C + 7, C - 5]),
              synth.custom(2, 2 * C + 9, 2, 2, C, seed=91 + C)]
    dev_in = [to_device(inp, gpu) for inp in inputs]
    outs = []
    for (k, v, beta, cu), inp in zip(dev_in, inputs):
        B, T, _, _ = k.shape
        Hv = beta.shape[2]
        outs.append((torch.empty(B, T, Hv, C, device=gpu),
                     torch.empty(B, T, Hv, 128, dtype=k.dtype, device=gpu),
                     torch.empty(B, T, Hv, 128, dtype=k.dtype, device=gpu)))

    def launch_all():
        for (k, v, beta, cu), (To, Wo, Uo) in zip(dev_in, outs):
            cg.wy_prepare(k, v, beta, C, cu_seqlens=cu, T_out=To, W_out=Wo, U_out=Uo)

    launch_all()  # eager, also fills the library's per-device launch cache
    torch.cuda.synchronize(gpu)
    eager = [tuple(t.clone() for t in o) for o in outs]

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=torch.cuda.Stream(gpu)):
        launch_all()
    torch.cuda.synchronize(gpu)

    for rep in range(4):
        for o in outs:
            for t in o:
                t.fill_(float("nan"))
        # unrelated eager work between replays
        scratch = torch.randn(1 << 20, device=gpu).cumsum(0)
        torch.cuda.synchronize(gpu)
        g.replay()
        torch.cuda.synchronize(gpu)
        say(f"graph C={C} replay {rep} (scratch {float(scratch[-1]):.3f})")
        for o, e in zip(outs, eager):
            for t, te in zip(o, e):
                assert torch.equal(t, te), f"replay {rep} differs from eager"
    for inp, (To, Wo, Uo) in zip(inputs, outs):
        compare_full(inp, To, Wo, Uo, label=f"graph C={C}")
