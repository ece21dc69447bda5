"""Helpers shared by the GPU parity tests (not collected by pytest)."""
import os
import sys

import numpy as np

import chunkwise_gated_deltanet_amd as cg
import oracle

T_TOL = 1e-5   # max |T_gpu - T_oracle| (fp32 T)
WU_TOL = 1e-2  # ||X_gpu - X_oracle||_F / ||X_oracle||_F for W and U


def oracle_threads():
    """Threads for the oracle: the usable host cores, at most 16 (a GPU machine's CPU share)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


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


def run_all(inp, device):
    """wy_prepare (T, W, U), kkt_solve (T) and wu_prepare (W, U) on the same inputs, every output
    pre-filled with NaN; returns {"T", "W", "U", "T_kkt", "W_wu", "U_wu"}."""
    import torch
    T, W, U = run_wy(inp, device)
    T_kkt, _, _ = run_wy(inp, device, kkt_only=True)
    k, v, beta, cu = to_device(inp, device)
    B, Tn, _, dk = k.shape
    Hv = beta.shape[2]
    W_wu = torch.full((B, Tn, Hv, dk), float("nan"), dtype=k.dtype, device=device)
    U_wu = torch.full((B, Tn, Hv, v.shape[3]), float("nan"), dtype=k.dtype, device=device)
    cg.wu_prepare(k, v, beta, inp["chunk_size"], cu_seqlens=cu, W_out=W_wu, U_out=U_wu,
                  g=gate_of(inp, device))
    torch.cuda.synchronize(device)
    return {"T": T, "W": W, "U": U, "T_kkt": T_kkt, "W_wu": W_wu, "U_wu": U_wu}


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


# Oracle units held at once by compare_all: T, W, U of this many units take about 512 MB (fp64).
ORACLE_BATCH_BYTES = 512 << 20


def compare_all(inp, outs, label=""):
    """Every stored entry of the GPU outputs against the oracle, one range of whole chunks at a
    time (so the largest workloads fit in host memory).

    outs maps a name to a GPU tensor: names starting with "T" are [B,T,Hv,C] float32 T tensors,
    "W..." and "U..." are W / U tensors of k's dtype.  Bar: max |T_gpu - T_oracle| <= 1e-5 over
    every entry of each T; relative Frobenius <= 1e-2 over the whole of each W and U.  Returns
    the metrics, with the worst single unit's W / U relative Frobenius as a diagnostic."""
    import torch
    B, T, C = inp["batch"], inp["seqlen"], inp["chunk_size"]
    Hv = inp["beta"].shape[2]
    dk = inp["k"].shape[3]
    dv = inp["v"].shape[3]
    starts, lens = oracle.list_chunks(B, T, C, inp["cu_seqlens"])
    want_wu = any(n[0] in "WU" for n in outs)
    per_unit = 8 * C * (C + (dk + dv if want_wu else 0))
    step = max(1, ORACLE_BATCH_BYTES // (per_unit * Hv))
    flat = {n: t.reshape(B * T, Hv, t.shape[-1]) for n, t in outs.items()}
    max_dT = {n: 0.0 for n in outs if n[0] == "T"}
    sq_err = {n: 0.0 for n in outs if n[0] in "WU"}
    sq_ref = {n: 0.0 for n in outs if n[0] in "WU"}
    worst_unit = 0.0
    threads = oracle_threads()
    for c0 in range(0, len(starts), step):
        cs, cl = starts[c0:c0 + step], lens[c0:c0 + step]
        nch = len(cs)
        t_lo, t_hi = int(cs[0]), int(cs[-1] + cl[-1])
        # chunks tile the flattened token range, so this batch is rows t_lo .. t_hi - 1
        ci = np.repeat(np.arange(nch), cl)
        row = np.concatenate([np.arange(n) for n in cl])
        Tr, Wr, Ur = oracle.units(inp["k"], inp["beta"], C, np.repeat(cs, Hv),
                                  np.repeat(cl, Hv), np.tile(np.arange(Hv, dtype=np.int32), nch),
                                  v=inp["v"] if want_wu else None, g=inp.get("g"),
                                  nthreads=threads)
        ref = {"T": Tr.reshape(nch, Hv, C, C)[ci, :, row, :]}
        if want_wu:
            ref["W"] = Wr.reshape(nch, Hv, C, dk)[ci, :, row, :]
            ref["U"] = Ur.reshape(nch, Hv, C, dv)[ci, :, row, :]
        del Tr, Wr, Ur
        for n, t in flat.items():
            got = to_f64(t[t_lo:t_hi])
            assert not np.isnan(got).any(), f"{n}: unwritten entries in rows {t_lo}..{t_hi - 1}"
            r = ref[n[0]]
            if n[0] == "T":
                max_dT[n] = max(max_dT[n], float(np.max(np.abs(got - r))))
            else:
                d2 = (got - r) ** 2
                sq_err[n] += float(d2.sum())
                sq_ref[n] += float((r * r).sum())
                # per unit: (chunk, head) sums of the rows of that chunk
                e_u = np.add.reduceat(d2.sum(axis=2), np.r_[0, np.cumsum(cl)[:-1]], axis=0)
                r_u = np.add.reduceat((r * r).sum(axis=2), np.r_[0, np.cumsum(cl)[:-1]], axis=0)
                ok = r_u > 0
                if ok.any():
                    worst_unit = max(worst_unit, float(np.sqrt(np.max(e_u[ok] / r_u[ok]))))
    out = {"units": int(len(starts) * Hv)}
    out.update({f"max_abs_d{n}": v for n, v in max_dT.items()})
    for n in sq_err:
        out[f"{n}_rel_fro"] = float(np.sqrt(sq_err[n] / sq_ref[n])) if sq_ref[n] > 0 else \
            float(np.sqrt(sq_err[n]))
    if sq_err:
        out["worst_unit_rel_fro"] = worst_unit
    say(f"[{label}] whole tensors {out}")
    for n, v in max_dT.items():
        assert v <= T_TOL, (n, out)
    for n in sq_err:
        assert out[f"{n}_rel_fro"] <= WU_TOL, (n, out)
    return out
