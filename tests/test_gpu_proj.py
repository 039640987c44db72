"""GPU parity of the projections around the attention path against the fp64 oracle:
csa_compress_hidden (hidden rows -> the four projections -> compressor pooling, one
kernel) and csa_out_proj (grouped output projection). Shapes are ragged against the
128 x 128 GEMM tile, the 124-token step of the overlapped compressor and the 32-wide K
slices; the Pro-width cases use the model's hidden width 7,168 ("DeepSeek-V4 混合注意力" §2
table) on a sub-chunk, or sample rows of the full-size output.
"""
import numpy as np
import pytest
import torch

import workloads as W
from tests.helpers import TOL_BF16, TOL_F32, assert_rel, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def csa():
    import long_context_compressed_amd as m
    m.lib()
    return m


def say(*a):
    print(*a, flush=True)


def _weights(shape, seed, name):
    # projection weights are 0.05 * N(0, 1), as the Tiny configuration's
    return W.normal(shape, seed, name, scale=0.05, dtype=torch.bfloat16, device=DEV)


@pytest.mark.parametrize("ratio,B,n,d,c,carry,odt,bias", [
    (4, 2, 1030, 256, 200, True, torch.float32, False),     # 9 token steps, ragged channels, carry
    (4, 1, 1030, 256, 200, False, torch.bfloat16, False),   # entry 0 pools its own block alone
    (4, 1, 500, 96, 64, True, torch.bfloat16, True),        # positional logit bias, d = 3 K slices
    (128, 2, 128 * 5 + 17, 256, 96, False, torch.float32, False),  # HCA: a trailing partial block
    (128, 1, 128 * 3, 160, 130, False, torch.bfloat16, True),
    (4, 1, 248, 7168, 512, True, torch.bfloat16, False),    # Pro hidden width, two token steps
])
def test_compress_hidden(csa, orc, ratio, B, n, d, c, carry, odt, bias):
    say("compress_hidden", ratio, B, n, d, c, carry, odt, bias)
    s = 5150 + n + d
    ov = 1 if ratio == 4 else 0
    H = W.normal((B, n, d), s, "H", dtype=torch.bfloat16, device=DEV)
    Wt = _weights((2 * (1 + ov), c, d), s, "W")
    cH = W.normal((B, 4, d), s, "cH", dtype=torch.bfloat16, device=DEV) if carry else None
    lb = W.normal(((1 + ov) * ratio, c), s, "bias", device=DEV) if bias else None
    out = csa.compress_hidden(H, Wt, cH, lb, ratio=ratio, overlap=ov, out_dtype=odt)
    torch.cuda.synchronize()
    ref = orc.compress_hidden(H, Wt, cH, lb, ratio=ratio, overlap=ov)
    assert out.shape == ref.shape == (B, n // ratio, c)
    assert_rel(out, ref, TOL_F32 if odt == torch.float32 else TOL_BF16, "compress_hidden")


def test_compress_hidden_into_cache_and_full_size_sample(csa, orc):
    """The Pro prefill chunk's KV compressor at full size (8,192 tokens x 7,168 hidden ->
    2,048 entries x 512 written into rows 16,384.. of an 18,432-row cache, with the carry of
    block 16,383), checked on sampled entries: entry e needs hidden rows 4e-4 .. 4e+3, so
    the oracle recomputes it from those 8 rows (4 of them as its carry)."""
    B, n, d, c, N, old = 1, 8192, 7168, 512, 18432, 16384
    s = 7171
    H = W.normal((B, n, d), s, "H", dtype=torch.bfloat16, device=DEV)
    Wt = _weights((4, c, d), s, "W")
    cH = W.normal((B, 4, d), s, "cH", dtype=torch.bfloat16, device=DEV)
    cache = torch.zeros((B, N, c), dtype=torch.bfloat16, device=DEV)
    csa.compress_hidden(H, Wt, cH, out=cache[:, old:, :])
    torch.cuda.synchronize()
    assert torch.count_nonzero(cache[:, :old]) == 0
    ents = [0, 1, 30, 31, 32, 123, 124, 1000, 2046, 2047]
    got, ref = [], []
    for e in ents:
        rows = H[:, 4 * e:4 * e + 4]
        prev = cH if e == 0 else H[:, 4 * e - 4:4 * e]
        ref.append(orc.compress_hidden(rows, Wt, prev)[:, 0])
        got.append(cache[:, old + e])
    assert_rel(torch.stack(got, 1), np.stack(ref, 1), TOL_BF16, "compress_hidden full-size sample")


@pytest.mark.parametrize("T,H,D,G,d_g,dm,odt", [
    (300, 128, 512, 16, 96, 320, torch.bfloat16),   # ragged rows, group width and model width
    (130, 64, 512, 1, 200, 0, torch.float32),       # one group, the grouped stage alone (fp32 y)
    (77, 8, 128, 4, 64, 96, torch.float32),
    (70, 6, 32, 2, 80, 160, torch.bfloat16),        # K of both maps an odd multiple of 32
    (1, 8, 64, 2, 32, 32, torch.bfloat16),          # one token, one tile far from full
    (513, 4, 128, 1, 257, 0, torch.float32),        # 256-row and 256-column tiles plus one of each
    (4096, 8, 64, 2, 64, 5000, torch.bfloat16),     # W_b: 320 tiles, the columns past one round in half-size tiles
])
def test_out_proj(csa, orc, T, H, D, G, d_g, dm, odt):
    say("out_proj", T, H, D, G, d_g, dm, odt)
    s = 6000 + T
    o = W.normal((T, H, D), s, "o", dtype=torch.bfloat16, device=DEV)
    Wa = _weights((G, d_g, (H // G) * D), s, "Wa")
    Wb = _weights((dm, G * d_g), s, "Wb") if dm else None
    out = csa.out_proj(o, Wa, Wb, out_dtype=odt)
    torch.cuda.synchronize()
    ref = orc.out_proj(o, Wa, Wb)
    # the grouped stage alone is one bf16 GEMM with fp32 sums; with W_b the group results
    # pass through bf16 (as activations between two projections), so the bf16 bar applies
    tol = TOL_F32 if (odt == torch.float32 and Wb is None) else TOL_BF16
    assert_rel(out, ref, tol, "out_proj")


def test_out_proj_full_size_sample(csa, orc):
    """Pro prefill chunk width: 8,192 tokens x 128 heads x 512 -> 16 groups of 1,024 ->
    the model width 7,168 (group count and width are arguments: the pages give neither);
    rows are independent, so sampled rows are checked against the oracle."""
    T, H, D, G, d_g, dm = 8192, 128, 512, 16, 1024, 7168
    s = 8123
    o = W.normal((T, H, D), s, "o", dtype=torch.bfloat16, device=DEV)
    Wa = _weights((G, d_g, (H // G) * D), s, "Wa")
    Wb = _weights((dm, G * d_g), s, "Wb")
    out = csa.out_proj(o, Wa, Wb)
    torch.cuda.synchronize()
    rows = torch.tensor([0, 1, 127, 128, 129, 4095, 4096, 8190, 8191], device=DEV)
    ref = orc.out_proj(o.index_select(0, rows), Wa, Wb)
    assert_rel(out.index_select(0, rows), ref, TOL_BF16, "out_proj full-size sample")


def test_query_norm_attention_out_proj_chain(csa, orc):
    """The query side of one layer, §6 and §7: RMSNorm of each head's query row (no rotation
    there: the attention call rotates q by rope_cs and rotates its output back), sparse
    attention, then the grouped output projection, against the oracle's chain."""
    T, H, D, B, N, k, R = 6, 128, 512, 1, 700, 64, 64
    s = 9090
    x = W.normal((T, H, D), s, "x", dtype=torch.bfloat16, device=DEV)
    g = W.uniform((D,), s, "g", lo=0.5, hi=1.5, device=DEV)
    kv = W.normal((B, N, D), s, "kv", dtype=torch.bfloat16, device=DEV)
    swa = W.normal((B, 128, D), s, "swa", dtype=torch.bfloat16, device=DEV)
    sink = W.normal((H,), s, "sink", device=DEV)
    pos = torch.tensor([2900, 2901, 2902, 2903, 2904, 2905], dtype=torch.int64, device=DEV)
    seq = torch.zeros(T, dtype=torch.int32, device=DEV)
    p0 = torch.tensor([2905 - 127], dtype=torch.int64, device=DEV)
    idx = torch.stack([torch.from_numpy(W.distinct_sample(k, N, s, f"i{t}")) for t in range(T)]).to(torch.int32).to(DEV)
    cs = W.rope_table(pos.cpu(), R).to(DEV)
    Wa = _weights((16, 64, 8 * D), s, "Wa")
    Wb = _weights((128, 16 * 64), s, "Wb")
    scale = D ** -0.5
    qn = csa.rmsnorm_rope(x, g, 1e-6)
    o, _ = csa.sparse_attn(qn, kv, sink, idx, scale, swa, p0, 128, seq, pos, cs, R)
    out = csa.out_proj(o, Wa, Wb)
    torch.cuda.synchronize()
    rq = orc.rmsnorm_rope(x.reshape(T * H, D), g, 1e-6).reshape(T, H, D)
    ro, _ = orc.sparse_attn(rq, kv, sink, idx, scale, swa, p0, 128, seq, pos, cs, R)
    rout = orc.out_proj(ro, Wa, Wb)
    assert_rel(qn, rq, TOL_BF16, "chain: rmsnorm")
    assert_rel(out, rout, TOL_BF16, "chain: norm -> attention -> out_proj")
