"""Helpers shared by the GPU parity tests (not collected by pytest)."""
import sys

import numpy as np

import chunkwise_gated_deltanet_amd as cg
import oracle

T_TOL = 1e-5   # max |T_gpu - T_oracle| (fp32 T)
WU_TOL = 1e-2  # ||X_gpu - X_oracle||_F / ||X_oracle||_F for W and U


def say(*args):
    print(*args, flush=True)
    sys.stdout.flush()


def to_device(inp, device):
    import torch
    if inp["dtype"] == "bf16":
        k = torch.from_numpy(inp["k"].view(np.int16)).view(torch.bfloat16)
        v = torch.from_numpy(inp["v"].view(np.int16)).view(torch.bfloat16)
    else:
        k = torch.from_numpy(inp["k"])
        v = torch.from_numpy(inp["v"])
    beta = torch.from_numpy(inp["beta"])
    cu = None if inp["cu_seqlens"] is None else torch.from_numpy(inp["cu_seqlens"]).to(device)
    return k.to(device), v.to(device), beta.to(device), cu


def gate_of(inp, device):
    """The inputs' log gates g on the device, or None (ungated)."""
    import torch
    g = inp.get("g")
    return None if g is None else torch.from_numpy(g).to(device)


def run_wy(inp, device, sentinel=True, kkt_only=False, stream=None):
    """Runs the HIP path on `inp`; outputs are pre-filled with NaN so unwritten entries show."""
    import torch
    k, v, beta, cu = to_device(inp, device)
    g = gate_of(inp, device)
    B, T, Hq, dk = k.shape
    Hv = beta.shape[2]
    C = inp["chunk_size"]
    fill = float("nan") if sentinel else 0.0
    T_out = torch.full((B, T, Hv, C), fill, dtype=torch.float32, device=device)
    if kkt_only:
        with torch.cuda.stream(stream or torch.cuda.current_stream(device)):
            cg.kkt_solve(k, beta, C, cu_seqlens=cu, T_out=T_out, g=g)
        torch.cuda.synchronize(device)
        return T_out, None, None
    W_out = torch.full((B, T, Hv, dk), fill, dtype=k.dtype, device=device)
    U_out = torch.full((B, T, Hv, v.shape[3]), fill, dtype=k.dtype, device=device)
    with torch.cuda.stream(stream or torch.cuda.current_stream(device)):
        cg.wy_prepare(k, v, beta, C, cu_seqlens=cu, T_out=T_out, W_out=W_out, U_out=U_out, g=g)
    torch.cuda.synchronize(device)
    return T_out, W_out, U_out


def chunk_row_index(inp):
    """Per flattened token: its row inside its chunk (numpy int64)."""
    B, T, C = inp["batch"], inp["seqlen"], inp["chunk_size"]
    starts, lens = oracle.list_chunks(B, T, C, inp["cu_seqlens"])
    rows = np.empty(B * T, np.int64)
    for s, n in zip(starts, lens):
        rows[s:s + n] = np.arange(n)
    return rows


def check_structure(T_gpu, inp):
    """Diagonal exactly 1, strictly upper entries (incl. columns >= n) exactly 0, no NaN."""
    import torch
    B, T, Hv, C = T_gpu.shape
    rows = torch.from_numpy(chunk_row_index(inp)).to(T_gpu.device)
    Tf = T_gpu.reshape(B * T, Hv, C)
    assert not torch.isnan(Tf).any(), "unwritten T entries"
    cols = torch.arange(C, device=T_gpu.device)
    upper = cols[None, :] > rows[:, None]          # [BT, C]
    diag = cols[None, :] == rows[:, None]
    assert bool((Tf.masked_select(upper[:, None, :].expand_as(Tf)) == 0).all()), "upper != 0"
    assert bool((Tf.masked_select(diag[:, None, :].expand_as(Tf)) == 1).all()), "diag != 1"


def rel_fro(x, ref):
    ref = np.asarray(ref, np.float64)
    x = np.asarray(x, np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(x - ref) / (den if den > 0 else 1.0))


def to_f64(t):
    import torch
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def compare_full(inp, T_gpu, W_gpu, U_gpu, label=""):
    """Whole-tensor comparison with the oracle; returns the metrics."""
    Tr, Wr, Ur, _ = oracle.wy_prepare(inp["k"], inp["beta"], inp["chunk_size"], v=inp["v"],
                                      cu_seqlens=inp["cu_seqlens"], g=inp.get("g"))
    Tg = to_f64(T_gpu)
    assert not np.isnan(Tg).any(), "unwritten T entries"
    dT = float(np.max(np.abs(Tg - Tr))) if Tg.size else 0.0
    out = {"max_abs_dT": dT}
    if W_gpu is not None:
        Wg, Ug = to_f64(W_gpu), to_f64(U_gpu)
        assert not np.isnan(Wg).any() and not np.isnan(Ug).any(), "unwritten W/U entries"
        out["W_rel_fro"] = rel_fro(Wg, Wr)
        out["U_rel_fro"] = rel_fro(Ug, Ur)
    say(f"[{label}] {out}")
    assert dT <= T_TOL, out
    if W_gpu is not None:
        assert out["W_rel_fro"] <= WU_TOL and out["U_rel_fro"] <= WU_TOL, out
    return out


def sample_units(inp, m, seed=0):
    """m random (chunk, v-head) units plus every short chunk and the first / last chunk."""
    B, T, C = inp["batch"], inp["seqlen"], inp["chunk_size"]
    Hv = inp["beta"].shape[2]
    starts, lens = oracle.list_chunks(B, T, C, inp["cu_seqlens"])
    rng = np.random.default_rng(seed)
    idx = list(rng.integers(0, len(starts), size=m))
    idx += [int(i) for i in np.nonzero(lens < C)[0]] + [0, len(starts) - 1]
    heads = rng.integers(0, Hv, size=len(idx))
    heads[-2:] = [0, Hv - 1]
    return starts[idx], lens[idx], heads.astype(np.int32)


def compare_sampled(inp, T_gpu, W_gpu, U_gpu, m=256, label=""):
    """Compares the oracle's value of sampled units with the rows the GPU wrote for them."""
    import torch
    starts, lens, heads = sample_units(inp, m)
    C = inp["chunk_size"]
    Tr, Wr, Ur = oracle.units(inp["k"], inp["beta"], C, starts, lens, heads,
                              v=inp["v"] if W_gpu is not None else None, g=inp.get("g"))
    B, T = inp["batch"], inp["seqlen"]
    Hv = inp["beta"].shape[2]
    Tf = T_gpu.reshape(B * T, Hv, C)
    rows = torch.from_numpy(np.concatenate([np.arange(s, s + n) for s, n in zip(starts, lens)])).to(T_gpu.device)
    hsel = torch.from_numpy(np.concatenate([np.full(n, h) for n, h in zip(lens, heads)])).to(T_gpu.device)
    Tg = to_f64(Tf[rows, hsel])
    Tref = np.concatenate([Tr[u, :n] for u, n in enumerate(lens)])
    out = {"units": int(len(starts)), "max_abs_dT": float(np.max(np.abs(Tg - Tref)))}
    if W_gpu is not None:
        dk = W_gpu.shape[-1]
        Wg = to_f64(W_gpu.reshape(B * T, Hv, dk)[rows, hsel])
        Ug = to_f64(U_gpu.reshape(B * T, Hv, -1)[rows, hsel])
        Wref = np.concatenate([Wr[u, :n] for u, n in enumerate(lens)])
        Uref = np.concatenate([Ur[u, :n] for u, n in enumerate(lens)])
        out["W_rel_fro"] = rel_fro(Wg, Wref)
        out["U_rel_fro"] = rel_fro(Ug, Uref)
        worst = 0.0
        off = 0
        for n in lens:
            worst = max(worst, rel_fro(Wg[off:off + n], Wref[off:off + n]),
                        rel_fro(Ug[off:off + n], Uref[off:off + n]))
            off += n
        out["worst_unit_rel_fro"] = worst
    say(f"[{label}] sampled {out}")
    assert out["max_abs_dT"] <= T_TOL, out
    if W_gpu is not None:
        assert out["W_rel_fro"] <= WU_TOL and out["U_rel_fro"] <= WU_TOL, out
    return out
