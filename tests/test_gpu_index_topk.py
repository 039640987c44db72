"""GPU parity of csa_index_topk, the MXFP4 decode scan fused with the top-k ("DeepSeek-V4
混合注意力" §4.2: FP4 index scores of every compressed entry, then each query's k best).

Two references: the oracle (MXFP4 decoded exactly, scores in fp64, top-k with the near-tie
rule of the top-k tests), and the unfused GPU path (csa_index_scores, then csa_topk), which
computes the same fp32 scores and must therefore give the same indices and values bit for
bit. Shapes span one chunk (4,096 entries: the chunk's winners are the output), several
chunks with a ragged last one (the winners then go through the csa_topk selection, in one
or two levels), k of a whole chunk, heavy ties, queries with no visible entry, N = 0, a
workspace reused across calls, and the Pro 1M decode shape.
"""
import numpy as np
import pytest
import torch

import workloads as W
from tests.helpers import check_topk_sets, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def csa():
    import long_context_compressed_amd as m
    m.lib()
    return m


def say(*a):
    print(*a, flush=True)


def _inputs(T, N, B, seed, zero_keys=False):
    q32 = W.normal((T, 64, 128), seed, "q", device=DEV)
    qc, qs = W.quantize_mxfp4(q32)
    if zero_keys:
        kc = torch.zeros((B, N, 64, 64), dtype=torch.uint8, device=DEV)
        ks = torch.full((B, N, 64, 4), 127, dtype=torch.uint8, device=DEV)
    else:
        kc, ks = W.normal_mxfp4((B, N, 64, 128), seed, "k", device=DEV, chunk_rows=1 << 20)
    w = W.normal((T, 64), seed, "w", device=DEV)
    return qc, qs, kc, ks, w


def _unfused(csa, qc, qs, w, kc, ks, q_seq, q_pos, k):
    sc = csa.index_scores(qc, w, kc, q_seq, q_pos, q_I_scale=qs, k_I_scale=ks, mxfp4=True)
    idx, vals = csa.topk(sc, k, with_vals=True)
    return sc, idx, vals


def _oracle_scores(orc, qc, qs, w, kc, ks, q_seq, q_pos, rows=None, chunk=4096):
    """Oracle scores [T][N] (fp64) with the keys decoded a chunk of entries at a time, so the
    fp64 keys never exceed chunk x 64 x 128 values; `rows` limits it to some queries."""
    T, N = qc.shape[0], kc.shape[1]
    rows = range(T) if rows is None else rows
    out = np.full((len(rows), N), -np.inf)
    qd = orc.mxfp4_decode(qc, qs)
    seq, pos, wn = to_np(q_seq), to_np(q_pos), to_np(w)
    for r, t in enumerate(rows):
        s0 = int(seq[t])
        if s0 < 0:
            continue
        for c0 in range(0, N, chunk):
            c1 = min(N, c0 + chunk)
            kd = orc.mxfp4_decode(kc[s0, c0:c1], ks[s0, c0:c1])[None]
            out[r, c0:c1] = orc.index_scores(qd[t:t + 1], wn[t:t + 1], kd, np.zeros(1, dtype=np.int32),
                                             pos[t:t + 1], entry_ids=np.arange(c0, c1, dtype=np.int64))[0]
    return out


def _check_exact(idx, vals, ridx, rvals, what):
    np.testing.assert_array_equal(to_np(idx), to_np(ridx), err_msg=f"{what}: indices")
    a, b = to_np(vals), to_np(rvals)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), f"{what}: values differ"


@pytest.mark.parametrize("T,N,B,k,pos", [
    (3, 3000, 2, 64, [4 * 2500, 4 * 3000, 4 * 37]),    # one chunk, cut at several points
    (2, 40000, 1, 2048, [4 * 40000, 4 * 33333]),       # 10 chunks, the last ragged; 20,480 winners
    (2, 30000, 2, 4096, [4 * 30000, 4 * 29000]),       # k = a whole chunk; 32,768 winners
    (4, 20000, 2, 333, [4 * 20000, 4 * 16383, 4 * 8193, 4 * 4096]),  # odd k, chunk edges
    (1, 4096, 1, 1024, [4 * 4096]),                    # exactly one chunk
    (2, 300000, 1, 1024, [4 * 300000, 4 * 299999]),    # 74 chunks: 75,776 winners
])
def test_index_topk(csa, orc, T, N, B, k, pos):
    say("index_topk", T, N, B, k)
    s = 9100 + N + k
    qc, qs, kc, ks, w = _inputs(T, N, B, s)
    q_seq = (torch.arange(T, dtype=torch.int32, device=DEV) % B)
    q_pos = torch.tensor(pos, dtype=torch.int64, device=DEV)
    idx, vals = csa.index_topk(qc, w, kc, q_seq, q_pos, k, qs, ks, with_vals=True)
    sc, ridx, rvals = _unfused(csa, qc, qs, w, kc, ks, q_seq, q_pos, k)
    torch.cuda.synchronize()
    _check_exact(idx, vals, ridx, rvals, "fused vs csa_index_scores + csa_topk")
    ref = _oracle_scores(orc, qc, qs, w, kc, ks, q_seq, q_pos)
    nd = check_topk_sets(idx, ref, k)
    say("  rows with near-tie differences from the oracle:", nd)


def test_index_topk_ties_empty_and_reuse(csa, orc):
    """All keys zero: every visible entry scores 0 (ReLU of 0), so the top-k is the first k
    visible entries (ties go to the lower index, also across chunks); a query of no sequence
    and a query at position 0 see nothing (all -1); one workspace serves three calls."""
    T, N, B, k = 4, 20000, 2, 700
    qc, qs, kc, ks, w = _inputs(T, N, B, 77, zero_keys=True)
    q_seq = torch.tensor([0, 1, -1, 0], dtype=torch.int32, device=DEV)
    q_pos = torch.tensor([4 * 20000, 4 * 650, 4 * 20000, 0], dtype=torch.int64, device=DEV)
    ws = csa.index_topk_workspace(T, N, k, DEV)
    outs = [csa.index_topk(qc, w, kc, q_seq, q_pos, k, qs, ks, workspace=ws, with_vals=True) for _ in range(3)]
    torch.cuda.synchronize()
    i0 = to_np(outs[0][0])
    np.testing.assert_array_equal(i0[0], np.arange(k))
    np.testing.assert_array_equal(i0[1, :650], np.arange(650))
    assert np.all(i0[1, 650:] == -1) and np.all(i0[2] == -1) and np.all(i0[3] == -1)
    v0 = to_np(outs[0][1])
    assert np.all(v0[0] == 0.0) and np.all(np.isneginf(v0[2]))
    for idx, vals in outs[1:]:
        _check_exact(idx, vals, outs[0][0], outs[0][1], "workspace reuse")


def test_index_topk_no_entries(csa):
    qc, qs, _, _, w = _inputs(2, 1, 1, 5)
    kc = torch.zeros((1, 0, 64, 64), dtype=torch.uint8, device=DEV)
    ks = torch.zeros((1, 0, 64, 4), dtype=torch.uint8, device=DEV)
    q_seq = torch.zeros(2, dtype=torch.int32, device=DEV)
    q_pos = torch.tensor([100, 200], dtype=torch.int64, device=DEV)
    idx, vals = csa.index_topk(qc, w, kc, q_seq, q_pos, 16, qs, ks, with_vals=True)
    torch.cuda.synchronize()
    assert np.all(to_np(idx) == -1) and np.all(np.isneginf(to_np(vals)))


def test_index_topk_pro_decode_full_size(csa, orc):
    """Pro 1M decode: 4 queries x 262,144 MXFP4 entries (64 chunks per query: 65,536
    winners), k = 1,024. Bit-exact against the unfused GPU path, and
    the oracle's scores of every entry of query 0 decide its top-k set."""
    cfg = W.PRO
    B, T, N, k = cfg.B, cfg.T, cfg.N, cfg.k
    say("index_topk Pro 1M decode")
    inp = W.decode_inputs(cfg, DEV, mxfp4=True)
    kc, ks = inp["k_I"], inp["k_I_scale"]
    qc, qs = W.quantize_mxfp4(inp["q_I"])
    w, q_seq, q_pos = inp["w"], inp["q_seq"], inp["q_pos"]
    idx, vals = csa.index_topk(qc, w, kc, q_seq, q_pos, k, qs, ks, with_vals=True)
    sc, ridx, rvals = _unfused(csa, qc, qs, w, kc, ks, q_seq, q_pos, k)
    torch.cuda.synchronize()
    _check_exact(idx, vals, ridx, rvals, "Pro decode: fused vs unfused")
    ref = _oracle_scores(orc, qc, qs, w, kc, ks, q_seq, q_pos, rows=[0], chunk=8192)
    check_topk_sets(idx[0:1], ref, k)
