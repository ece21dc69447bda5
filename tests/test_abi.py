"""The C-ABI library on the CPU: it loads, exports every declared symbol, and rejects bad
arguments before any HIP call (no GPU is touched by these tests)."""
import ctypes
import os
import re

import numpy as np
import pytest

import chunkwise_gated_deltanet_amd as cg
from chunkwise_gated_deltanet_amd import build

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include",
                      "wyprep.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(cg.LIB_PATH):
        build.build_library()
    return cg.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(wyp_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == {"wyp_abi_version", "wyp_status_string", "wyp_last_error",
                          "wyp_kkt_solve", "wyp_wy_prepare", "wyp_wu_prepare", "wyp_solve_rhs",
                          "wyp_chunk_fwd",
                          "wyp_wy_backward", "wyp_chunk_fwd_cp", "wyp_chunk_fwd_cp_noalloc",
                          "wyp_chunk_fwd_cp_workspace_bytes"}
    for name in names:
        assert hasattr(lib, name), name


def test_version_and_strings(lib):
    assert lib.wyp_abi_version() == 8 == cg.ABI_VERSION
    assert lib.wyp_status_string(0) == b"WYP_OK"
    assert lib.wyp_status_string(3) == b"WYP_ERR_HIP"
    assert lib.wyp_status_string(99) == b"WYP_ERR_UNKNOWN"


FAKE = 0x10000  # never dereferenced: every case below fails validation or is empty


def good(**kw):
    d = dict(batch=1, seqlen=128, num_qk_heads=2, num_v_heads=4, head_dim_k=128,
             head_dim_v=128, chunk_size=64, num_seqs=0, kv_dtype=0)
    d.update(kw)
    return cg.Problem(*[d[n] for n, _ in cg.Problem._fields_])


def call_wy(lib, p, k=FAKE, v=FAKE, beta=FAKE, cu=None, T=FAKE, W=FAKE, U=FAKE, g=None):
    return lib.wyp_wy_prepare(ctypes.byref(p) if p is not None else None, k, v, g, beta, cu, T,
                              W, U, None)


@pytest.mark.parametrize("kw,code,needle", [
    (dict(chunk_size=48), 2, "chunk_size"),
    (dict(chunk_size=16), 2, "chunk_size"),
    (dict(head_dim_k=64), 2, "head_dim"),
    (dict(head_dim_v=256), 2, "head_dim"),
    (dict(num_v_heads=3), 1, "multiple"),
    (dict(num_qk_heads=0), 1, "head counts"),
    (dict(batch=0), 1, "batch"),
    (dict(seqlen=-1), 1, "seqlen"),
    (dict(kv_dtype=7), 1, "kv_dtype"),
    (dict(kv_dtype=1, chunk_size=96), 2, "chunk_size"),
])
def test_rejects_bad_problem(lib, kw, code, needle):
    assert call_wy(lib, good(**kw)) == code
    assert needle in lib.wyp_last_error().decode()


def test_rejects_null_and_misaligned(lib):
    assert call_wy(lib, None) == 1
    assert call_wy(lib, good(), k=None) == 1
    assert call_wy(lib, good(), U=None) == 1
    assert call_wy(lib, good(), T=FAKE + 4) == 1
    assert "16-byte" in lib.wyp_last_error().decode()
    assert call_wy(lib, good(), beta=FAKE + 2) == 1
    assert call_wy(lib, good(), g=FAKE + 2) == 1
    assert "g is not 4-byte" in lib.wyp_last_error().decode()
    assert lib.wyp_kkt_solve(ctypes.byref(good()), FAKE, None, FAKE, None, None, None) == 1
    assert lib.wyp_kkt_solve(ctypes.byref(good()), FAKE, FAKE + 1, FAKE, None, FAKE, None) == 1
    # wu_prepare takes no T_out, but needs W_out and U_out
    assert lib.wyp_wu_prepare(ctypes.byref(good()), FAKE, FAKE, None, FAKE, None, FAKE, None,
                              None) == 1
    assert lib.wyp_wu_prepare(ctypes.byref(good()), FAKE, FAKE, None, FAKE, None, FAKE + 8, FAKE,
                              None) == 1
    assert "16-byte" in lib.wyp_last_error().decode()


def test_rejects_bad_packing(lib):
    assert call_wy(lib, good(batch=2, num_seqs=2), cu=FAKE) == 1
    assert "batch" in lib.wyp_last_error().decode()
    assert call_wy(lib, good(num_seqs=-1), cu=FAKE) == 1
    assert call_wy(lib, good(num_seqs=0, seqlen=5), cu=FAKE) == 1
    assert call_wy(lib, good(num_seqs=2), cu=FAKE + 2) == 1


def test_empty_problem_is_a_noop(lib):
    assert call_wy(lib, good(seqlen=0)) == 0
    assert lib.wyp_last_error() == b""
    assert call_wy(lib, good(seqlen=0, num_seqs=0), cu=FAKE) == 0
    assert lib.wyp_kkt_solve(ctypes.byref(good(seqlen=0)), FAKE, None, FAKE, None, FAKE,
                             None) == 0
    assert lib.wyp_wu_prepare(ctypes.byref(good(seqlen=0)), None, None, None, None, None, None,
                              None, None) == 0


def test_error_text_is_per_call(lib):
    assert call_wy(lib, good(chunk_size=3)) == 2
    assert lib.wyp_last_error() != b""
    assert call_wy(lib, good(seqlen=0)) == 0
    assert lib.wyp_last_error() == b""


def test_binding_rejects_cpu_tensors(lib):
    import torch
    k = torch.zeros(1, 4, 1, 128, dtype=torch.bfloat16)
    beta = torch.zeros(1, 4, 1)
    with pytest.raises(ValueError):
        cg.kkt_solve(k, beta, 64)
    with pytest.raises(ValueError):
        cg.kkt_solve(k, beta, 64, g=torch.zeros(1, 4, 1))


def call_fwd(lib, p, q=FAKE, k=FAKE, w=FAKE, u=FAKE, g=None, h0=None, scale=0.5, cu=None,
             o=FAKE, hT=None):
    return lib.wyp_chunk_fwd(ctypes.byref(p) if p is not None else None, q, k, w, u, g, h0,
                             scale, cu, o, hT, None)


@pytest.mark.parametrize("kw,code,needle", [
    (dict(chunk_size=48), 2, "chunk_size"),
    (dict(chunk_size=256), 2, "chunk_size"),
    (dict(kv_dtype=1), 2, "bf16"),
    (dict(head_dim_v=64), 2, "head_dim"),
    (dict(num_v_heads=3), 1, "multiple"),
    (dict(batch=0), 1, "batch"),
])
def test_chunk_fwd_rejects_bad_problem(lib, kw, code, needle):
    assert call_fwd(lib, good(**kw)) == code
    assert needle in lib.wyp_last_error().decode()


def test_chunk_fwd_rejects_bad_arguments(lib):
    assert call_fwd(lib, None) == 1
    assert call_fwd(lib, good(), q=None) == 1
    assert call_fwd(lib, good(), o=None) == 1
    assert call_fwd(lib, good(), w=FAKE + 8) == 1
    assert "16-byte" in lib.wyp_last_error().decode()
    assert call_fwd(lib, good(), hT=FAKE + 2) == 1
    assert call_fwd(lib, good(), scale=float("nan")) == 1
    assert "scale" in lib.wyp_last_error().decode()
    assert call_fwd(lib, good(), scale=float("inf")) == 1
    assert call_fwd(lib, good(batch=2, num_seqs=2), cu=FAKE) == 1


def test_chunk_fwd_empty_is_a_noop(lib):
    # no tokens and no final state requested: nothing to do, no pointer is touched
    assert call_fwd(lib, good(seqlen=0), q=None, k=None, w=None, u=None, o=None) == 0
    assert call_fwd(lib, good(seqlen=0, num_seqs=0), cu=FAKE, q=None, k=None, w=None, u=None,
                    o=None, hT=FAKE) == 0


def call_bwd(lib, p, k=FAKE, v=FAKE, g=None, beta=FAKE, cu=None, dT=None, dW=FAKE, dU=FAKE,
             dk=FAKE, dv=FAKE, db=FAKE, dg=None):
    return lib.wyp_wy_backward(ctypes.byref(p) if p is not None else None, k, v, g, beta, cu, dT,
                               dW, dU, dk, dv, db, dg, None)


def test_wy_backward_rejects(lib):
    assert call_bwd(lib, good(kv_dtype=1)) == 2        # the backward is built for bf16 only
    assert call_bwd(lib, good(chunk_size=48)) == 2
    assert "chunk_size" in lib.wyp_last_error().decode()
    assert call_bwd(lib, good(chunk_size=256)) == 2
    assert call_bwd(lib, good(), dW=None) == 1
    assert call_bwd(lib, good(), dk=None) == 1
    assert call_bwd(lib, good(), g=FAKE) == 1          # gates given, dg missing
    assert "dg" in lib.wyp_last_error().decode()
    assert call_bwd(lib, good(), dv=FAKE + 4) == 1
    assert call_bwd(lib, good(), dT=FAKE + 2) == 1
    assert call_bwd(lib, good(seqlen=0), k=None, v=None, beta=None, dW=None, dU=None, dk=None,
                    dv=None, db=None) == 0


def test_chunk_fwd_cp_workspace_and_rejects(lib):
    p = good(batch=2, seqlen=1000, num_v_heads=4)       # 16 chunks per row
    ws = lib.wyp_chunk_fwd_cp_workspace_bytes
    assert ws(ctypes.byref(p), None, 16) == 0   # one segment
    # four segments: A and M of three, plus the initial-state copy, per (row, value head)
    assert ws(ctypes.byref(p), None, 5) == 2 * 4 * 7 * 128 * 128 * 4
    assert ws(ctypes.byref(p), None, 0) == -1
    assert ws(ctypes.byref(good(chunk_size=48)), None, 4) == -1
    # C = 32 and 128: segments of segment_chunks x C tokens
    assert ws(ctypes.byref(good(batch=2, seqlen=1000, num_v_heads=4, chunk_size=32)), None, 8) == \
        2 * 4 * (2 * 4 - 1) * 128 * 128 * 4   # 32 chunks of 32 per row: 4 segments
    assert ws(ctypes.byref(good(batch=2, seqlen=1000, num_v_heads=4, chunk_size=128)), None, 8) == 0
    need = ws(ctypes.byref(p), None, 4)

    def call(seg=4, ws=FAKE, nbytes=need, **kw):
        return lib.wyp_chunk_fwd_cp(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, None, None, 0.5, None,
                                    seg, ws, nbytes, FAKE, None, None)
    assert call(ws=None) == 1
    assert "workspace" in lib.wyp_last_error().decode()
    assert call(nbytes=need - 1) == 1
    assert call(ws=FAKE + 4) == 1
    assert call(seg=0) == 1


def test_chunk_fwd_cp_packed_workspace(lib):
    """Packed sequences: floor(T / X) + N a-slots and floor(T / X) m-slots per value head, X = 64
    segment_chunks tokens; the pointer is only tested for NULL, never read."""
    ws = lib.wyp_chunk_fwd_cp_workspace_bytes
    slot = 128 * 128 * 4
    p = good(batch=1, seqlen=5000, num_v_heads=8, num_seqs=7)
    cu = ctypes.c_void_p(FAKE)
    assert ws(ctypes.byref(p), cu, 4) == (2 * (5000 // 256) + 7) * 8 * slot
    assert ws(ctypes.byref(p), cu, 78) == (2 * 1 + 7) * 8 * slot     # X = 4992 <= T
    assert ws(ctypes.byref(p), cu, 79) == 0                          # X > T: never split
    assert ws(ctypes.byref(p), cu, 0) == -1
    assert ws(ctypes.byref(good(batch=2, seqlen=5000, num_seqs=7)), cu, 4) == -1
    # the bound holds for any length mix: brute force over a few, counting the slots the
    # kernel uses (a-slots floor(cu[n] / X) + n + s, m-slots floor(cu[n] / X) + s)
    rng = np.random.default_rng(3)
    for trial in range(200):
        lens = rng.integers(0, 3000, size=int(rng.integers(1, 12)))
        lens[rng.random(lens.size) < 0.2] = 0
        T, X = int(lens.sum()), 64 * int(rng.integers(1, 20))
        cu_h = np.concatenate([[0], np.cumsum(lens)])
        a_used, m_used = set(), set()
        for n, ln in enumerate(lens):
            nseg = max(1, -(-int(ln) // X))
            for s in range(nseg):
                a = cu_h[n] // X + n + s
                assert a not in a_used
                a_used.add(a)
            for s in range(nseg - 1):
                m = cu_h[n] // X + s
                assert m not in m_used
                m_used.add(m)
        assert max(a_used) < T // X + lens.size
        assert not m_used or max(m_used) < T // X


def test_chunk_fwd_cp_noalloc_rejects_before_any_hip_call(lib):
    """The scratch limit and argument checks are host-side: nothing is launched."""
    lim = 32 * 1024 * 1024
    p = good(batch=1, seqlen=64 * 128, num_qk_heads=16, num_v_heads=16)   # 128 chunks

    def call(prob, seg, **kw):
        return lib.wyp_chunk_fwd_cp_noalloc(ctypes.byref(prob), FAKE, FAKE, FAKE, FAKE, None, None,
                                            0.5, None, seg, FAKE, None, None)
    assert lib.wyp_chunk_fwd_cp_workspace_bytes(ctypes.byref(p), None, 16) <= lim      # 8 segments
    big = good(batch=4, seqlen=64 * 128, num_qk_heads=32, num_v_heads=32)
    assert lib.wyp_chunk_fwd_cp_workspace_bytes(ctypes.byref(big), None, 16) > lim
    assert call(big, 16) == 2
    assert "scratch" in lib.wyp_last_error().decode()
    assert call(p, 0) == 1
    assert call(good(chunk_size=48), 4) == 2
    assert call(good(seqlen=0), 4) == 0          # no tokens, no final state: a no-op


def test_solve_rhs_rejects_before_any_hip_call(lib):
    def call(p, k=FAKE, rhs=FAKE, beta=FAKE, X=FAKE, g=None, cu=None):
        return lib.wyp_solve_rhs(ctypes.byref(p) if p is not None else None, k, rhs, g, beta, cu,
                                 X, None)
    assert call(None) == 1
    assert call(good(), rhs=None) == 1
    assert call(good(), X=None) == 1
    assert call(good(), X=FAKE + 8) == 1
    assert call(good(), rhs=FAKE + 8) == 1
    assert call(good(chunk_size=48)) == 2
    assert call(good(head_dim_v=64)) == 2
    assert call(good(num_v_heads=3)) == 1
    assert call(good(seqlen=0), k=None, rhs=None, beta=None, X=None) == 0


def test_segment_length_choice():
    """cp_segment_chunks / auto_segment_chunks: no split once the 32-column workgroups of every
    (sequence, value head) give each of the 256 CUs one; otherwise segments of at least 4 chunks
    for about 512 such workgroups.  A packed batch counts as num_seqs rows of its mean length,
    and a choice that would not split comes back as None, so no sequence of a packed batch is
    cut when the rule says the batch needs no split."""
    assert cg.cp_segment_chunks(1, 8192, 16) == 16          # 64 items: 8 segments of 16 chunks
    assert cg.cp_segment_chunks(1, 32768, 8) == 32          # 32 items: 16 segments
    assert cg.cp_segment_chunks(4, 4096, 32) == 64          # 512 items: no split (all 64 chunks)
    assert cg.cp_segment_chunks(1, 1024, 2) == 4            # capped at 4 chunks per segment
    assert cg.auto_segment_chunks(1, 8192, 16) == 16
    assert cg.auto_segment_chunks(4, 4096, 32) is None
    assert cg.auto_segment_chunks(1, 100, 16) is None        # two chunks: nothing to split
    # packed: 2 sequences of 16384 tokens in all are two rows of 8192
    assert cg.auto_segment_chunks(1, 16384, 16, num_seqs=2) == cg.cp_segment_chunks(2, 8192, 16)
    # packed, many sequences x heads: no split at all
    assert cg.auto_segment_chunks(1, 70000, 64, num_seqs=8) is None
    # the chunk size enters through the chunk count
    assert cg.auto_segment_chunks(1, 8192, 16, chunk_size=128) == cg.cp_segment_chunks(1, 8192, 16, 128)
