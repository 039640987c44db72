"""The hot path strung together: a decode step and the two prefill chunks.

Each object allocates its outputs and workspaces once and then only launches the
library's calls (every step runs in libcsa.so), on torch's current stream. The call
chain is the one of "DeepSeek-V4 混合注意力" §7 (CSA: compress -> indexer -> top-k ->
sparse attention; HCA: compress -> dense attention over the summaries).
"""
from __future__ import annotations

import torch

from . import (attn_workspace_bytes, compress, compress_batch, hca_attn, index_scores, index_topk,
               index_topk_workspace, quantize_kv8, quantize_mxfp4, sparse_attn, topk, topk_workspace_bytes)


def _ws(nbytes, dev):
    return torch.empty(max(1, nbytes), dtype=torch.uint8, device=dev)


class DecodeStep:
    """One decode step of a CSA layer and an HCA layer for B sequences, one query each.

    `inp` holds: q [T][H][D], kv [B][N][D], swa [B][window][D], swa_pos0 [B], sink [H],
    q_seq [T], q_pos [T], rope_cs [T][R/2][2], q_I [T][64][128], w [T][64],
    k_I [B][N][64][128], summ [B][n/128][D], sink_h [H], and the completing blocks:
    blk / carry (KV compressor, ratio 4), iblk / icarry (index-key compressor, ratio 4),
    hblk (HCA compressor, ratio 128). The step writes the block's new KV row, index key
    and summary into the last row of kv, k_I and summ, then scores, selects and attends.
    With MXFP4 index keys (k_I codes [B][N][64][64] and k_I_scale [B][N][64][4] in `inp`)
    the new index key is compressed to bf16, rotated by the Hadamard transform and encoded
    into the last entry, and each step's q_I is rotated and encoded before the scan; the scan
    and the top-k are then one csa_index_topk call (the scores stay on chip), unless
    `fused_topk` is False.
    With FP8-format caches (kv [B][N][592] and summ [B][n/128][592] uint8) the new KV entry
    and summary are compressed to bf16 and encoded (csa_quantize_kv8) into the last rows,
    and both attention calls read the FP8 rows.
    """

    def __init__(self, inp: dict, k: int, window: int, rope_dim: int, scale: float, fused_topk: bool = True):
        self.inp, self.k, self.window, self.rope_dim, self.scale = inp, k, window, rope_dim, scale
        q, kv, k_I, summ = inp["q"], inp["kv"], inp["k_I"], inp["summ"]
        T, H, D = q.shape
        B, N = kv.shape[0], kv.shape[1]
        NH = summ.shape[1]
        dev = q.device
        # FP8-format caches (uint8 rows): the step compresses into bf16 staging rows and
        # encodes them into the last row of each sequence's cache
        self.kv8 = kv.dtype == torch.uint8
        if self.kv8:
            self.kv_new = torch.empty((B, 1, D), dtype=torch.bfloat16, device=dev)
            self.summ_new_bf = torch.empty((B, 1, D), dtype=torch.bfloat16, device=dev)
        else:
            self.kv_new = kv[:, N - 1:N, :]
        self.mxfp4 = inp.get("k_I_scale") is not None
        if self.mxfp4:
            qI = inp["q_I"]
            self.kI_new = torch.empty((B, 1, 64 * 128), dtype=torch.bfloat16, device=dev)
            self.qc = torch.empty(qI.shape[:-1] + (qI.shape[-1] // 2,), dtype=torch.uint8, device=dev)
            self.qs = torch.empty(qI.shape[:-1] + (qI.shape[-1] // 32,), dtype=torch.uint8, device=dev)
        else:
            self.kI_new = k_I.view(B, N, -1)[:, N - 1:N, :]
        self.summ_new = self.summ_new_bf if self.kv8 else summ[:, NH - 1:NH, :]
        self.fused = self.mxfp4 and fused_topk
        self.scores = None if self.fused else torch.empty((T, N), dtype=torch.float32, device=dev)
        self.idx = torch.empty((T, k), dtype=torch.int32, device=dev)
        self.topk_ws = index_topk_workspace(T, N, k, dev) if self.fused else _ws(topk_workspace_bytes(T, N, k), dev)
        self.attn_ws = _ws(attn_workspace_bytes(T, H, D, k + window), dev)
        self.hca_ws = _ws(attn_workspace_bytes(T, H, D, NH + window), dev)
        self.out = torch.empty((T, H, D), dtype=q.dtype, device=dev)
        self.lse = torch.empty((T, H), dtype=torch.float32, device=dev)
        self.out_h = torch.empty((T, H, D), dtype=q.dtype, device=dev)
        self.lse_h = torch.empty((T, H), dtype=torch.float32, device=dev)

    def compress(self):
        """The block completing with the step, pooled three ways in one launch: the new KV
        entry and index key (ratio 4, with their carries) and the new HCA summary (ratio
        128); then the encodings of the FP8 caches / the MXFP4 index key, if any."""
        i = self.inp
        b, c, ib, ic, h = i["blk"], i["carry"], i["iblk"], i["icarry"], i["hblk"]
        compress_batch([
            dict(C_a=b["Ca"], Z_a=b["Za"], C_b=b["Cb"], Z_b=b["Zb"], carry_C_b=c["C"], carry_Z_b=c["Z"], ratio=4,
                 out=self.kv_new),
            dict(C_a=ib["Ca"], Z_a=ib["Za"], C_b=ib["Cb"], Z_b=ib["Zb"], carry_C_b=ic["C"], carry_Z_b=ic["Z"],
                 ratio=4, out=self.kI_new),
            dict(C_a=h["C"], Z_a=h["Z"], ratio=128, out=self.summ_new),
        ])
        if self.kv8:  # the new entry and summary of every sequence into the last rows of the FP8 caches
            N, NH = i["kv"].shape[1], i["summ"].shape[1]
            quantize_kv8(self.kv_new, out=i["kv"][0, N - 1], group_rows=1, group_stride=N)
            quantize_kv8(self.summ_new, out=i["summ"][0, NH - 1], group_rows=1, group_stride=NH)
        if self.mxfp4:  # rotate and encode the new key into the last entry of every sequence
            kI, ks = i["k_I"], i["k_I_scale"]
            N = kI.shape[1]
            quantize_mxfp4(self.kI_new.view(-1, 64, 128), hadamard=True, codes=kI[0, N - 1], scales=ks[0, N - 1],
                           group_rows=64, group_stride=64 * N)

    def index_prep(self):
        """MXFP4 keys: the query's index vectors rotated and encoded (nothing otherwise)."""
        if self.mxfp4:
            quantize_mxfp4(self.inp["q_I"], hadamard=True, codes=self.qc, scales=self.qs)

    def index(self):
        """The index scan (fused: the scan and the top-k)."""
        i = self.inp
        if self.fused:
            index_topk(self.qc, i["w"], i["k_I"], i["q_seq"], i["q_pos"], self.k, self.qs, i["k_I_scale"],
                       idx=self.idx, workspace=self.topk_ws)
        elif self.mxfp4:
            index_scores(self.qc, i["w"], i["k_I"], i["q_seq"], i["q_pos"], q_I_scale=self.qs,
                         k_I_scale=i["k_I_scale"], mxfp4=True, scores=self.scores)
        else:
            index_scores(i["q_I"], i["w"], i["k_I"], i["q_seq"], i["q_pos"], scores=self.scores)

    def select(self):
        """The top-k over the scores (done inside index() when fused)."""
        if not self.fused:
            topk(self.scores, self.k, idx=self.idx, workspace=self.topk_ws)

    def attend(self):
        i = self.inp
        sparse_attn(i["q"], i["kv"], i["sink"], self.idx, self.scale, i["swa"], i["swa_pos0"], self.window,
                    i["q_seq"], i["q_pos"], i["rope_cs"], self.rope_dim, out=self.out, lse=self.lse,
                    workspace=self.attn_ws)

    def hca(self):
        i = self.inp
        hca_attn(i["q"], i["summ"], i["sink_h"], 128, self.scale, i["swa"], i["swa_pos0"], self.window,
                 i["q_seq"], i["q_pos"], i["rope_cs"], self.rope_dim, out=self.out_h, lse=self.lse_h,
                 workspace=self.hca_ws)

    def __call__(self, index_events=None):
        """The whole step; `index_events` = (start, end) events recorded around the scan."""
        if self.graphs is not None:
            return self.replay(index_events)
        self.compress()
        self.index_prep()
        if index_events is not None:
            index_events[0].record()
        self.index()
        if index_events is not None:
            index_events[1].record()
        self.select()
        self.attend()
        self.hca()

    graphs = None

    def capture(self):
        """Record the small calls around the index scan as two HIP graphs (before it: the
        compressors and the query encoding; after it: top-k, sparse attention, the HCA
        compressor and attention), so a step is two graph launches and one scan launch
        instead of a dozen library calls from the host. The scan itself is launched directly
        between the events that time it (a graph launch adds latency a single long kernel
        does not need). Every buffer the step touches is allocated in __init__, so the
        graphs stay valid for the object's life; the library records no memset, only
        kernels."""
        parts = ((self.compress, self.index_prep), (self.select, self.attend, self.hca))
        graphs = []
        torch.cuda.synchronize()
        for fns in parts:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for f in fns:
                    f()
            graphs.append(g)
        torch.cuda.synchronize()
        self.graphs = graphs

    def replay(self, index_events=None):
        pre, post = self.graphs
        pre.replay()
        if index_events is not None:
            index_events[0].record()
        self.index()
        if index_events is not None:
            index_events[1].record()
        post.replay()


class ProPrefillChunk:
    """A CSA prefill chunk: compress the chunk's blocks into the KV cache, MXFP4 index scores
    of every query against every entry (causal), top-k, sparse attention.

    `inp`: kv [1][N][D] (rows from `old` on are rewritten), C = {Ca, Cb, Za, Zb} [1][T][D],
    carry = {C, Z} [1][4][D], q_I / q_I_scale, k_I / k_I_scale (MXFP4), w [T][64],
    q [T][H][D], swa, swa_pos0, sink, q_pos, q_seq, rope_cs.
    """

    def __init__(self, inp: dict, k: int, window: int, rope_dim: int, scale: float):
        self.inp, self.k, self.window, self.rope_dim, self.scale = inp, k, window, rope_dim, scale
        q, kv = inp["q"], inp["kv"]
        T, H, D = q.shape
        N = kv.shape[1]
        dev = q.device
        self.kv_new = kv[:, inp["old"]:, :]
        self.scores = torch.empty((T, N), dtype=torch.float32, device=dev)
        self.idx = torch.empty((T, k), dtype=torch.int32, device=dev)
        self.topk_ws = _ws(topk_workspace_bytes(T, N, k), dev)
        self.attn_ws = _ws(attn_workspace_bytes(T, H, D, k + window), dev)
        self.out = torch.empty_like(q)
        self.lse = torch.empty((T, H), dtype=torch.float32, device=dev)

    def compress(self):
        C, c = self.inp["C"], self.inp["carry"]
        compress(C["Ca"], C["Za"], C["Cb"], C["Zb"], c["C"], c["Z"], out=self.kv_new)

    def index(self):
        i = self.inp
        index_scores(i["q_I"], i["w"], i["k_I"], i["q_seq"], i["q_pos"], q_I_scale=i["q_I_scale"],
                     k_I_scale=i["k_I_scale"], mxfp4=True, scores=self.scores)

    def select(self):
        topk(self.scores, self.k, idx=self.idx, workspace=self.topk_ws)

    def attend(self):
        i = self.inp
        sparse_attn(i["q"], i["kv"], i["sink"], self.idx, self.scale, i["swa"], i["swa_pos0"], self.window,
                    i["q_seq"], i["q_pos"], i["rope_cs"], self.rope_dim, out=self.out, lse=self.lse,
                    workspace=self.attn_ws)

    def stages(self):
        return {"compress": self.compress, "index_scores_mxfp4": self.index, "topk": self.select,
                "sparse_attn": self.attend}


class HcaPrefillChunk:
    """An HCA prefill chunk: compress the chunk's 128-token blocks into the last summaries,
    then dense attention of every query over its visible summaries and SWA rows.

    `inp`: summ [1][NH][D] (the last T/128 rows are rewritten), C, Z [1][T][D], q, swa,
    swa_pos0, sink, q_pos, q_seq, rope_cs.
    """

    def __init__(self, inp: dict, window: int, rope_dim: int, scale: float):
        self.inp, self.window, self.rope_dim, self.scale = inp, window, rope_dim, scale
        q, summ = inp["q"], inp["summ"]
        T, H, D = q.shape
        NH = summ.shape[1]
        self.summ_new = summ[:, NH - T // 128:, :]
        self.attn_ws = _ws(attn_workspace_bytes(T, H, D, NH + window), q.device)
        self.out = torch.empty_like(q)
        self.lse = torch.empty((T, H), dtype=torch.float32, device=q.device)

    def compress(self):
        compress(self.inp["C"], self.inp["Z"], ratio=128, overlap=0, out=self.summ_new)

    def attend(self):
        i = self.inp
        hca_attn(i["q"], i["summ"], i["sink"], 128, self.scale, i["swa"], i["swa_pos0"], self.window,
                 i["q_seq"], i["q_pos"], i["rope_cs"], self.rope_dim, out=self.out, lse=self.lse,
                 workspace=self.attn_ws)

    def stages(self):
        return {"compress_hca": self.compress, "hca_attn": self.attend}
