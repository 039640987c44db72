"""Parity at the full configuration sizes, in the launch configuration bench.py times.

Each test builds the configuration's inputs on the GPU, runs the same pipeline object
bench.py times (long_context_compressed_amd.pipeline) and checks sampled outputs against
the fp64 oracle, stage by stage and fed: every stage's oracle call gets the same inputs as
the GPU stage (the GPU's upstream outputs, once those have passed). The oracle sees only
the sampled rows, gathered on the GPU, so no full-size tensor is widened on the host.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads as W
from tests.helpers import TOL_BF16, TOL_F32, assert_rel

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def csa():
    import long_context_compressed_amd as m
    m.lib()
    return m


def say(*a):
    print(*a, flush=True)


def _free():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _check_index_sample(orc, scores, q_I, w, k_I, q_seq, q_pos, ids, mxfp4_scales=None):
    """Oracle scores of the sampled entries `ids` (shared by every sequence) for every query."""
    idt = torch.from_numpy(ids).to(k_I.device)
    if mxfp4_scales is None:
        k_s = k_I.index_select(1, idt)
        q_o = q_I
    else:
        qs, ks = mxfp4_scales
        k_s = orc.mxfp4_decode(k_I.index_select(1, idt), ks.index_select(1, idt))
        q_o = orc.mxfp4_decode(q_I, qs)
    ref = orc.index_scores(q_o, w, k_s, q_seq, q_pos, entry_ids=ids)
    gpu = scores.index_select(1, idt).cpu().double().numpy()
    fin = np.isfinite(ref)
    assert np.array_equal(fin, np.isfinite(gpu)), "masked (causal) entries differ"
    assert np.all(gpu[~fin] == -np.inf)
    assert_rel(gpu[fin], ref[fin], TOL_F32, "index scores (sampled entries)")


def _check_topk_fed(orc, scores, idx, k):
    """Top-k of the GPU scores: identical fp32 inputs give identical sets."""
    ridx, _ = orc.topk(scores.cpu(), k)
    gi = idx.cpu().numpy()
    for t in range(gi.shape[0]):
        g = gi[t][gi[t] >= 0]
        r = ridx[t][ridx[t] >= 0]
        assert sorted(g.tolist()) == sorted(r.tolist()), f"top-k set of query {t}"
        assert np.all(gi[t, len(g):] == -1)


def _gathered_rows(kv, seqs, idx):
    """kv rows each query selected, as [1][T*k][D] with the matching slot indices."""
    T, k = idx.shape
    rows = []
    for t in range(T):
        rows.append(kv[int(seqs[t])].index_select(0, idx[t].clamp(min=0).long()))
    kv_c = torch.cat(rows, 0)[None]
    slot = torch.arange(T * k, dtype=torch.int32, device=idx.device).view(T, k)
    idx_c = torch.where(idx >= 0, slot, torch.full_like(slot, -1))
    return kv_c, idx_c


@pytest.mark.parametrize("name,keys", [("flash_decode_128k", "bf16"), ("pro_decode_1m", "bf16"),
                                       ("pro_decode_1m", "shared"), ("pro_decode_1m", "mxfp4")])
def test_decode_step_full_size(csa, orc, name, keys):
    """keys="shared": the side line with one 128-dim index key per entry for all heads;
    keys="mxfp4": MXFP4 index keys, with the step's q_I and new key Hadamard-rotated and
    encoded on the GPU (checked bit-exact against the oracle's encoder, fed the same
    values) and the scan checked on the decoded codes."""
    from long_context_compressed_amd import pipeline

    cfg = W.CONFIGS[name]
    shared, fp4 = keys == "shared", keys == "mxfp4"
    say("full-size decode step", name, keys)
    inp = W.decode_step_inputs(cfg, DEV, shared_keys=shared, mxfp4=fp4)
    step = pipeline.DecodeStep(inp, cfg.k, cfg.window, cfg.rope_dim, cfg.scale)
    step()
    torch.cuda.synchronize()
    B, T, N = cfg.B, cfg.T, cfg.N

    # compressors: the completing block of every sequence (KV entry, index key, summary)
    b, c, ib, ic, hb = inp["blk"], inp["carry"], inp["iblk"], inp["icarry"], inp["hblk"]
    assert_rel(step.kv_new, orc.compress(b["Ca"], b["Za"], b["Cb"], b["Zb"], c["C"], c["Z"]), TOL_BF16,
               "new KV entry")
    assert_rel(step.kI_new, orc.compress(ib["Ca"], ib["Za"], ib["Cb"], ib["Zb"], ic["C"], ic["Z"]), TOL_BF16,
               "new index key")
    assert_rel(step.summ_new, orc.compress(hb["C"], hb["Z"], ratio=128, overlap=0), TOL_BF16, "new summary")

    # index scores: 4,096 sampled entries (both ends included) of every sequence
    ids = np.unique(np.concatenate([[0, 1, N - 2, N - 1], W.distinct_sample(4092, N, cfg.seed, "fullsize_ids")]))
    if fp4:
        rc, rs = orc.mxfp4_encode(step.kI_new.view(B, 64, 128), hadamard=True)
        np.testing.assert_array_equal(inp["k_I"][:, N - 1].cpu().numpy(), rc)
        np.testing.assert_array_equal(inp["k_I_scale"][:, N - 1].cpu().numpy(), rs)
        rc, rs = orc.mxfp4_encode(inp["q_I"], hadamard=True)
        np.testing.assert_array_equal(step.qc.cpu().numpy(), rc)
        np.testing.assert_array_equal(step.qs.cpu().numpy(), rs)
        # the step's scan is fused with the top-k (no score array): the same scores from the
        # plain scan must select exactly the step's indices
        scores = csa.index_scores(step.qc, inp["w"], inp["k_I"], inp["q_seq"], inp["q_pos"], q_I_scale=step.qs,
                                  k_I_scale=inp["k_I_scale"], mxfp4=True)
        ridx, _ = csa.topk(scores, cfg.k)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(step.idx.cpu().numpy(), ridx.cpu().numpy())
        _check_index_sample(orc, scores, step.qc, inp["w"], inp["k_I"], inp["q_seq"], inp["q_pos"], ids,
                            mxfp4_scales=(step.qs, inp["k_I_scale"]))
    else:
        scores = step.scores
        _check_index_sample(orc, scores, inp["q_I"], inp["w"], inp["k_I"], inp["q_seq"], inp["q_pos"], ids)

    # top-k over the full 262,144 / 32,768 scores of every query
    _check_topk_fed(orc, scores, step.idx, cfg.k)

    # sparse attention of every query over its selected rows + SWA
    kv_c, idx_c = _gathered_rows(inp["kv"], inp["q_seq"].cpu().numpy(), step.idx)
    seq = torch.zeros(T, dtype=torch.int32)
    swa = inp["swa"].index_select(0, inp["q_seq"].long())
    p0 = inp["swa_pos0"].index_select(0, inp["q_seq"].long())
    outs = []
    for t in range(T):  # one sequence per call: the query's own SWA rows
        outs.append(orc.sparse_attn(inp["q"][t:t + 1], kv_c, inp["sink"], idx_c[t:t + 1], cfg.scale,
                                    swa[t:t + 1], p0[t:t + 1], cfg.window, seq[:1], inp["q_pos"][t:t + 1],
                                    inp["rope_cs"][t:t + 1], cfg.rope_dim))
    assert_rel(step.out, np.concatenate([o for o, _ in outs]), TOL_BF16, "sparse attention out")
    assert_rel(step.lse, np.concatenate([l for _, l in outs]), 2e-3, "sparse attention lse")

    # HCA attention of every query over all its visible summaries + SWA
    ref, rlse = orc.hca_attn(inp["q"], inp["summ"], inp["sink_h"], 128, cfg.scale, inp["swa"], inp["swa_pos0"],
                             cfg.window, inp["q_seq"], inp["q_pos"], inp["rope_cs"], cfg.rope_dim)
    assert_rel(step.out_h, ref, TOL_BF16, "hca attention out")
    assert_rel(step.lse_h, rlse, 2e-3, "hca attention lse")
    del inp, step, kv_c
    _free()


def test_pro_decode_fp4_candidates_rerank(csa, orc):
    """Pro 1M decode shape: the bf16 index keys and queries are Hadamard-rotated and MXFP4-
    encoded on the GPU (sampled rows bit-exact with the oracle's encoder); the FP4 scan picks
    2k = 2,048 candidates per query, csa_index_rescore scores them exactly (bf16 keys) and
    csa_topk_ids keeps the best k = 1,024, which must be the oracle's top-k of the candidates
    by those scores. Prints the recall of the exact bf16 top-k by the 2k candidates (the
    quantity the pages report as 99.7% for the trained indexer; here on N(0,1) data)."""
    cfg = W.PRO
    B, T, N, k = cfg.B, cfg.T, cfg.N, cfg.k
    say("FP4 candidates + exact re-rank, Pro 1M decode")
    inp = W.decode_inputs(cfg, DEV)
    q_I, w, k_I, q_seq, q_pos = inp["q_I"], inp["w"], inp["k_I"], inp["q_seq"], inp["q_pos"]
    kc, ks = csa.quantize_mxfp4(k_I, hadamard=True)
    qc, qs = csa.quantize_mxfp4(q_I, hadamard=True)
    torch.cuda.synchronize()
    rows = torch.from_numpy(W.distinct_sample(256, N, cfg.seed, "fp4_rows")).to(DEV)
    rc, rs = orc.mxfp4_encode(k_I[1].index_select(0, rows), hadamard=True)
    np.testing.assert_array_equal(kc[1].index_select(0, rows).cpu().numpy(), rc)
    np.testing.assert_array_equal(ks[1].index_select(0, rows).cpu().numpy(), rs)
    rc, rs = orc.mxfp4_encode(q_I, hadamard=True)
    np.testing.assert_array_equal(qc.cpu().numpy(), rc)
    np.testing.assert_array_equal(qs.cpu().numpy(), rs)

    s4 = csa.index_scores(qc, w, kc, q_seq, q_pos, q_I_scale=qs, k_I_scale=ks, mxfp4=True)
    cand, _ = csa.topk(s4, 2 * k)
    exact = csa.index_rescore(q_I, w, k_I, cand, q_seq, q_pos)
    final, _ = csa.topk_ids(exact, cand, k)
    full = csa.index_scores(q_I, w, k_I, q_seq, q_pos)
    ref_top, _ = csa.topk(full, k)
    torch.cuda.synchronize()
    del kc, ks, s4
    _free()

    # re-rank: the kept entries are the oracle's top-k of the candidates by the exact scores
    ex = exact.cpu().double().numpy()
    c_np, f_np = cand.cpu().numpy(), final.cpu().numpy()
    for t in range(T):
        sub = orc.index_scores(q_I[t:t + 1], w[t:t + 1], k_I[int(q_seq[t])].index_select(
            0, torch.from_numpy(c_np[t].astype(np.int64)).to(DEV))[None], np.zeros(1, dtype=np.int32),
            q_pos[t:t + 1].cpu().numpy(), entry_ids=c_np[t].astype(np.int64))
        assert_rel(ex[t], sub[0], TOL_F32, "exact scores of the candidates")
        pos, _ = orc.topk(ex[t:t + 1], k)
        assert sorted(f_np[t].tolist()) == sorted(c_np[t][pos[0]].tolist()), f"re-ranked set of query {t}"
    recall_c = np.mean([len(set(c_np[t]) & set(ref_top[t].cpu().numpy())) / k for t in range(T)])
    recall_f = np.mean([len(set(f_np[t]) & set(ref_top[t].cpu().numpy())) / k for t in range(T)])
    say(f"recall of the exact top-{k} by the FP4 2k candidates: {recall_c:.4f}; after the re-rank: {recall_f:.4f}")
    assert recall_f >= recall_c - 1e-12
    del inp, cand, exact, final, full, ref_top
    _free()


def test_pro_prefill_chunk_full_size(csa, orc):
    from long_context_compressed_amd import pipeline

    say("full-size Pro prefill chunk")
    inp = W.prefill_inputs("pro_prefill_chunk", DEV)
    cfg, T, N, k = inp["cfg"], inp["T"], inp["N"], inp["k"]
    ch = pipeline.ProPrefillChunk(inp, k, cfg.window, cfg.rope_dim, cfg.scale)
    for f in ch.stages().values():
        f()
    torch.cuda.synchronize()

    # compressor over the whole chunk (with the carry of the block before it)
    C, cr = inp["C"], inp["carry"]
    assert_rel(ch.kv_new, orc.compress(C["Ca"], C["Za"], C["Cb"], C["Zb"], cr["C"], cr["Z"]), TOL_BF16,
               "chunk KV entries")

    # every 64th query plus the first and last 16 (160 queries)
    sel = np.unique(np.concatenate([np.arange(16), np.arange(T - 16, T), np.arange(0, T, 64)]))
    st = torch.from_numpy(sel).to(DEV)
    pos = inp["q_pos"].index_select(0, st)
    # index scores: 2,048 sampled entries, including each sampled query's causal boundary
    edge = np.concatenate([[p // 4 - 1, p // 4, p // 4 + 1] for p in pos.cpu().numpy()])
    ids = np.unique(np.clip(np.concatenate([[0, N - 1], edge, W.distinct_sample(1980, N, cfg.seed, "fs_e")]),
                            0, N - 1))
    _check_index_sample(orc, ch.scores.index_select(0, st), inp["q_I"].index_select(0, st),
                        inp["w"].index_select(0, st), inp["k_I"], inp["q_seq"].index_select(0, st), pos, ids,
                        mxfp4_scales=(inp["q_I_scale"].index_select(0, st), inp["k_I_scale"]))
    # top-k of the sampled queries' full score rows
    _check_topk_fed(orc, ch.scores.index_select(0, st), ch.idx.index_select(0, st), k)
    # sparse attention of the sampled queries
    idx_s = ch.idx.index_select(0, st)
    kv_c, idx_c = _gathered_rows(inp["kv"], np.zeros(len(sel), np.int64), idx_s)
    ref, rlse = orc.sparse_attn(inp["q"].index_select(0, st), kv_c, inp["sink"], idx_c, cfg.scale, inp["swa"],
                                inp["swa_pos0"], cfg.window, inp["q_seq"].index_select(0, st), pos,
                                inp["rope_cs"].index_select(0, st), cfg.rope_dim)
    assert_rel(ch.out.index_select(0, st), ref, TOL_BF16, "prefill sparse attention out")
    assert_rel(ch.lse.index_select(0, st), rlse, 2e-3, "prefill sparse attention lse")
    del inp, ch, kv_c
    _free()


def test_hca_prefill_chunk_full_size(csa, orc):
    from long_context_compressed_amd import pipeline

    say("full-size HCA prefill chunk")
    inp = W.prefill_inputs("hca_prefill_4k", DEV)
    cfg, T = inp["cfg"], inp["T"]
    ch = pipeline.HcaPrefillChunk(inp, cfg.window, cfg.rope_dim, cfg.scale)
    for f in ch.stages().values():
        f()
    torch.cuda.synchronize()
    assert_rel(ch.summ_new, orc.compress(inp["C"], inp["Z"], ratio=128, overlap=0), TOL_BF16, "chunk summaries")
    # every 64th query plus the first and last 16 (96 queries; 127 / 128 straddle a summary edge)
    sel = np.unique(np.concatenate([np.arange(16), np.arange(T - 16, T), np.arange(0, T, 64), [127, 128]]))
    st = torch.from_numpy(sel).to(DEV)
    ref, rlse = orc.hca_attn(inp["q"].index_select(0, st), inp["summ"], inp["sink"], 128, cfg.scale, inp["swa"],
                             inp["swa_pos0"], cfg.window, inp["q_seq"].index_select(0, st),
                             inp["q_pos"].index_select(0, st), inp["rope_cs"].index_select(0, st), cfg.rope_dim)
    assert_rel(ch.out.index_select(0, st), ref, TOL_BF16, "HCA prefill attention out")
    assert_rel(ch.lse.index_select(0, st), rlse, 2e-3, "HCA prefill attention lse")
    del inp, ch
    _free()


def test_pro_prefill_q_norm_rope_full_size(csa, orc):
    """RMSNorm + RoPE of the Pro prefill chunk's queries as bench.py times it (8,192 x 128
    rows of 512 bf16, one angle row per token): 2,000 sampled rows against the oracle; and
    at every row, with unit gains, eps = 0 and fp32 output, a mean square of 1 (the
    normalisation's invariant, which the rotation keeps)."""
    cfg = W.PRO_PREFILL
    T, H, D, R, s = cfg.T, cfg.H, cfg.c, cfg.rope_dim, cfg.seed
    say("q_norm_rope full size", T, H, D)
    q = W.normal((T, H, D), s, "q", dtype=torch.bfloat16, device=DEV)
    g = W.uniform((D,), s, "q_norm_gain", lo=0.5, hi=1.5, device=DEV)
    cs = W.rope_table(torch.arange(cfg.n, cfg.n + T, dtype=torch.int64), R).to(DEV)
    out = csa.rmsnorm_rope(q, g, 1e-6, rope_cs=cs, rope_group=H)
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(7).choice(T * H, 2000, replace=False))
    rt = torch.from_numpy(rows).to(DEV)
    ref = orc.rmsnorm_rope(q.view(T * H, D)[rt], g, 1e-6, rope_cs=cs[torch.from_numpy(rows // H).to(DEV)],
                           rope_dim=R)
    assert_rel(out.view(T * H, D)[rt], ref, TOL_BF16, "q_norm_rope sample")
    del out
    y = csa.rmsnorm_rope(q, torch.ones(D, device=DEV), 0.0, rope_cs=cs, rope_group=H, out_dtype=torch.float32)
    ms = (y.view(T * H, D).double() ** 2).mean(-1)
    assert float((ms - 1.0).abs().max()) < 1e-5
    del y, ms
    _free()
