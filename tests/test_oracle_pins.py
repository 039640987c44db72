"""Pins of the CPU oracle against facts fixed by the pages and by mathematics.

Each test names the passage of "DeepSeek-V4 混合注意力：从压缩记忆到百万上下文"
(the brenchcc technical note) that fixes the value, or the closed form /
library routine the special case reduces to. None of these runs the GPU.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import workloads

GOLD = os.path.join(os.path.dirname(__file__), "golden")
rng = np.random.default_rng(12345)


def _rand(*shape, scale=1.0):
    return rng.standard_normal(shape) * scale


# ------------------------------------------------------------------------------------
# Compressor: §4.1 (ratio 4, overlapped) and §5 (ratio 128)
# ------------------------------------------------------------------------------------

def _one_entry_overlap(orc, zb, za, cb, ca):
    """Entry 1 of a 2-block sequence: b-slots from block 0, a-slots from block 1."""
    n, c = 8, len(zb[0]) if np.ndim(zb) > 1 else 1
    Zb = np.zeros((1, n, c)); Za = np.zeros((1, n, c))
    Cb = np.zeros((1, n, c)); Ca = np.zeros((1, n, c))
    Zb[0, 0:4, :] = np.reshape(zb, (4, c)); Cb[0, 0:4, :] = np.reshape(cb, (4, c))
    Za[0, 4:8, :] = np.reshape(za, (4, c)); Ca[0, 4:8, :] = np.reshape(ca, (4, c))
    # rows of the other branch carry arbitrary junk that must not enter entry 1
    Zb[0, 4:8, :] = 50.0; Cb[0, 4:8, :] = -1e3
    Za[0, 0:4, :] = 50.0; Ca[0, 0:4, :] = -1e3
    out = orc.compress(Ca, Za, Cb, Zb, ratio=4, overlap=1)
    return out[0, 1]


def test_worked_channel_example(orc):
    """§4.1 worked example: weights [1,2,1,2,4,2,1,3] normalise to /16, slot 5 dominates."""
    g = json.load(open(os.path.join(GOLD, "compress_worked_example.json")))
    w = np.array(g["unnormalised_weights"], dtype=np.float64)
    logits = np.log(w) + 0.37  # any constant shift
    contents = np.array(g["contents_for_output_check"], dtype=np.float64)
    out = _one_entry_overlap(orc, logits[:4], logits[4:], contents[:4], contents[4:])
    assert out[0] == pytest.approx(g["output_with_those_contents"], abs=1e-14)
    # out is linear in the contents: unit vectors recover alpha slot by slot
    alpha = []
    for r in range(8):
        e = np.zeros(8); e[r] = 1.0
        alpha.append(_one_entry_overlap(orc, logits[:4], logits[4:], e[:4], e[4:])[0])
    alpha = np.array(alpha)
    np.testing.assert_allclose(alpha * g["alpha_denominator"], g["alpha_numerators_over_16"],
                               atol=1e-13)
    assert int(np.argmax(alpha)) + 1 == g["argmax_slot_1_based"]


def test_output_lengths_n_over_ratio(orc):
    """§3 / §4.1 / §5: n/4 = 262,144 entries and n/128 = 8,192 summaries at n = 2^20."""
    n = 1 << 20
    z = np.zeros((1, n, 1))
    assert orc.compress(z, z, z, z, ratio=4, overlap=1).shape == (1, 262144, 1)
    assert orc.compress(z, z, ratio=128, overlap=0).shape == (1, 8192, 1)
    # a trailing partial block is not compressed
    z2 = np.zeros((1, 1030, 1))
    assert orc.compress(z2, z2, z2, z2, ratio=4, overlap=1).shape == (1, 257, 1)


def test_compress_invariants(orc):
    """§4.1: per-channel softmax over the 8-slot receptive field (convex weights)."""
    B, n, c = 2, 32, 5
    Ca, Cb, Za, Zb = (_rand(B, n, c) for _ in range(4))
    cCb, cZb = _rand(B, 4, c), _rand(B, 4, c)
    base = orc.compress(Ca, Za, Cb, Zb, cCb, cZb)
    assert base.shape == (B, n // 4, c)
    # constant content in the field gives that constant
    const = np.full((B, n, c), 2.5)
    out = orc.compress(const, Za, const, Zb, np.full((B, 4, c), 2.5), cZb)
    np.testing.assert_allclose(out, 2.5, atol=1e-14)
    # output lies between min and max of the 8 contents it pools
    for i in range(1, n // 4):
        lo = np.minimum(Cb[:, 4 * (i - 1):4 * i].min(1), Ca[:, 4 * i:4 * i + 4].min(1))
        hi = np.maximum(Cb[:, 4 * (i - 1):4 * i].max(1), Ca[:, 4 * i:4 * i + 4].max(1))
        assert np.all(base[:, i] >= lo - 1e-12) and np.all(base[:, i] <= hi + 1e-12)
    # a per-channel constant added to every logit changes nothing
    shift = _rand(1, 1, c) * 10
    out = orc.compress(Ca, Za + shift, Cb, Zb + shift, cCb, cZb + shift)
    np.testing.assert_allclose(out, base, atol=1e-12)
    # uniform logits give the mean of the 8 pooled rows (numpy mean)
    zero = np.zeros((B, n, c))
    out = orc.compress(Ca, zero, Cb, zero, cCb, np.zeros((B, 4, c)))
    for i in range(1, n // 4):
        ref = np.concatenate([Cb[:, 4 * (i - 1):4 * i], Ca[:, 4 * i:4 * i + 4]], axis=1).mean(1)
        np.testing.assert_allclose(out[:, i], ref, atol=1e-13)
    ref0 = np.concatenate([cCb, Ca[:, 0:4]], axis=1).mean(1)
    np.testing.assert_allclose(out[:, 0], ref0, atol=1e-13)


def test_compress_overlap_locality(orc):
    """§4.1: a block's a-branch feeds entry i, its b-branch feeds entry i+1 ("overlap")."""
    B, n, c = 1, 24, 3
    Ca, Cb, Za, Zb = (_rand(B, n, c) for _ in range(4))
    base = orc.compress(Ca, Za, Cb, Zb)
    i, j = 2, 1
    Ca2 = Ca.copy(); Ca2[0, 4 * i + 1, j] += 1.0
    d = orc.compress(Ca2, Za, Cb, Zb) - base
    assert np.count_nonzero(np.abs(d) > 0) == 1 and abs(d[0, i, j]) > 0
    Cb2 = Cb.copy(); Cb2[0, 4 * i + 3, j] += 1.0
    d = orc.compress(Ca, Za, Cb2, Zb) - base
    assert np.count_nonzero(np.abs(d) > 0) == 1 and abs(d[0, i + 1, j]) > 0
    Zb2 = Zb.copy(); Zb2[0, 4 * i, j] += 1.0
    d = orc.compress(Ca, Za, Cb, Zb2) - base
    nz = np.argwhere(np.abs(d) > 0)
    assert len(nz) == 1 and tuple(nz[0]) == (0, i + 1, j)


def test_compress_first_entry_without_carry(orc):
    """Entry 0 without a carry pools only block 0's a-branch (4-way softmax)."""
    B, n, c = 1, 8, 4
    Ca, Cb, Za, Zb = (_rand(B, n, c) for _ in range(4))
    out = orc.compress(Ca, Za, Cb, Zb)
    z = torch.tensor(Za[0, 0:4])
    ref = (torch.softmax(z, dim=0) * torch.tensor(Ca[0, 0:4])).sum(0).numpy()
    np.testing.assert_allclose(out[0, 0], ref, atol=1e-13)
    # with a carry, entry 0 equals entry 1 of the sequence that has the carry prepended
    cCb, cZb = _rand(B, 4, c), _rand(B, 4, c)
    out_c = orc.compress(Ca, Za, Cb, Zb, cCb, cZb)
    pad = lambda x, y: np.concatenate([y, x], axis=1)
    full = orc.compress(pad(Ca, _rand(B, 4, c)), pad(Za, _rand(B, 4, c)), pad(Cb, cCb), pad(Zb, cZb))
    np.testing.assert_allclose(out_c[0], full[0, 1:], atol=1e-13)


def test_hca_compress_softmax_pool(orc):
    """§5: C^hca_i = sum over the 128 rows of block i of softmax(Z)_r C_r (torch.softmax)."""
    B, n, c = 2, 3 * 128 + 17, 3
    Cz, Zz = _rand(B, n, c), _rand(B, n, c, scale=2.0)
    out = orc.compress(Cz, Zz, ratio=128, overlap=0)
    assert out.shape == (B, 3, c)
    for i in range(3):
        blk = slice(128 * i, 128 * i + 128)
        ref = (torch.softmax(torch.tensor(Zz[:, blk]), dim=1) * torch.tensor(Cz[:, blk])).sum(1)
        np.testing.assert_allclose(out[:, i], ref.numpy(), atol=1e-13)
    # a dominant logit selects its row
    Z2 = np.zeros((1, 128, 1)); Z2[0, 77, 0] = 800.0
    C2 = np.arange(128, dtype=np.float64).reshape(1, 128, 1)
    assert orc.compress(C2, Z2, ratio=128, overlap=0)[0, 0, 0] == pytest.approx(77.0, abs=1e-12)


def test_compress_bias_is_added_to_logits(orc):
    """Positional logit bias (the CSA two-step description: softmax weights with a
    positional bias) is equivalent to shifting the logits of the matching slot."""
    B, n, c = 1, 16, 2
    Ca, Cb, Za, Zb = (_rand(B, n, c) for _ in range(4))
    bias = _rand(8, c)
    out = orc.compress(Ca, Za, Cb, Zb, bias=bias)
    Zb2 = Zb + np.tile(bias[:4], (n // 4, 1))[None]
    Za2 = Za + np.tile(bias[4:], (n // 4, 1))[None]
    ref = orc.compress(Ca, Za2, Cb, Zb2)
    np.testing.assert_allclose(out[0, 1:], ref[0, 1:], atol=1e-13)


# ------------------------------------------------------------------------------------
# Indexer: §4.2 s_{t,i} = sum_h w_{t,h} ReLU(<q^I_{t,h}, k^I_{i,h}>)
# ------------------------------------------------------------------------------------

def test_index_single_head_is_gemv(orc):
    """H=1, w=1, q,k >= 0: the score is a plain dot product (numpy matmul)."""
    T, N, Dh = 3, 40, 16
    q = np.abs(_rand(T, 1, Dh)); k = np.abs(_rand(1, N, 1, Dh))
    s = orc.index_scores(q, np.ones((T, 1)), k, np.zeros(T), np.full(T, 4 * N))
    np.testing.assert_allclose(s, q[:, 0] @ k[0, :, 0].T, rtol=1e-14)


def test_index_head_selection_and_relu(orc):
    """w picks one head: the score is ReLU of that head's own dot (key head h' = h)."""
    T, N, H, Dh = 2, 30, 4, 8
    q, k = _rand(T, H, Dh), _rand(1, N, H, Dh)
    for h in range(H):
        w = np.zeros((T, H)); w[:, h] = 2.0
        s = orc.index_scores(q, w, k, np.zeros(T), np.full(T, 10 ** 6))
        dot = q[:, h] @ k[0, :, h].T
        np.testing.assert_allclose(s, 2.0 * np.maximum(dot, 0.0), rtol=1e-13, atol=1e-15)
    # all dots negative: score exactly 0 whatever w
    s = orc.index_scores(np.abs(q), _rand(T, H), -np.abs(k), np.zeros(T), np.full(T, 10 ** 6))
    assert np.all(s == 0.0)


def test_index_head_sum_and_homogeneity(orc):
    """The head sum splits over disjoint head sets; s is linear in w and 1-homogeneous in q."""
    T, N, H, Dh = 3, 50, 64, 128
    q, k, w = _rand(T, H, Dh), _rand(1, N, H, Dh), _rand(T, H)
    qs, qp = np.zeros(T), np.full(T, 4 * N)
    full = orc.index_scores(q, w, k, qs, qp)
    a = orc.index_scores(q[:, :32], w[:, :32], k[:, :, :32], qs, qp)
    b = orc.index_scores(q[:, 32:], w[:, 32:], k[:, :, 32:], qs, qp)
    np.testing.assert_allclose(full, a + b, rtol=1e-12, atol=1e-12)
    tol = 1e-13 * np.abs(full).max()  # sums of mixed signs: compare against the row scale
    np.testing.assert_allclose(orc.index_scores(q, -3 * w, k, qs, qp), -3 * full, rtol=0, atol=3 * tol)
    np.testing.assert_allclose(orc.index_scores(2.5 * q, w, k, qs, qp), 2.5 * full, rtol=0, atol=3 * tol)
    assert np.all(orc.index_scores(q, np.abs(w), k, qs, qp) >= 0)


def test_index_causal_visibility(orc):
    """Entry i (block [4i, 4i+4)) is visible to a query at t iff 4(i+1) <= t:
    floor(t/4) finite scores per query (tiny prefill: t = 0..1023, 256 entries)."""
    T, N = 1024, 256
    q, k = _rand(T, 2, 4), _rand(1, N, 2, 4)
    s = orc.index_scores(q, np.ones((T, 2)), k, np.zeros(T), np.arange(T))
    fin = np.isfinite(s)
    assert np.array_equal(fin.sum(1), np.arange(T) // 4)
    assert np.all(fin[:, :1].sum(1) == (np.arange(T) >= 4))
    # entry_ids re-indexes a sampled key store
    ids = np.array([3, 100, 255])
    s2 = orc.index_scores(q, np.ones((T, 2)), k[:, ids], np.zeros(T), np.arange(T), entry_ids=ids)
    np.testing.assert_array_equal(s2, s[:, ids])


def test_index_shared_keys(orc):
    """A single shared key head (kh = 1) equals per-head keys that repeat it."""
    T, N, H, Dh = 2, 20, 8, 16
    q, k1, w = _rand(T, H, Dh), _rand(1, N, 1, Dh), _rand(T, H)
    a = orc.index_scores(q, w, k1, np.zeros(T), np.full(T, 999))
    b = orc.index_scores(q, w, np.repeat(k1, H, axis=2), np.zeros(T), np.full(T, 999))
    np.testing.assert_allclose(a, b, rtol=1e-14)


# ------------------------------------------------------------------------------------
# MXFP4 (E2M1 values, one E8M0 scale per 32 elements)
# ------------------------------------------------------------------------------------

def test_mxfp4_decode_table(orc):
    """All 16 E2M1 codes decode to sign x {0,.5,1,1.5,2,3,4,6}; E8M0 s means 2^(s-127)."""
    mags = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    nib = np.arange(32) % 16
    codes = (nib[0::2] | (nib[1::2] << 4)).astype(np.uint8)
    for sc, f in ((127, 1.0), (128, 2.0), (126, 0.5), (120, 2.0 ** -7)):
        out = orc.mxfp4_decode(codes, np.array([sc], dtype=np.uint8))
        ref = np.array([(-1 if v >= 8 else 1) * mags[v & 7] * f for v in nib])
        np.testing.assert_array_equal(out, ref)


def test_mxfp4_quantiser_roundtrip(orc):
    """Values on the E2M1 grid times 2^e encode exactly; a general block stays within
    half a grid step of the scaled value and its scale is 2^(floor(log2 amax) - 2)."""
    grid = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    vals = np.concatenate([grid, -grid[1:], grid[:8], -grid[1:8], [6.0, -4.0]])[:32] * 2.0 ** -3
    x = torch.tensor(vals, dtype=torch.float32).reshape(1, 32)
    codes, scales = workloads.quantize_mxfp4(x)
    np.testing.assert_array_equal(orc.mxfp4_decode(codes, scales)[0], vals)
    y = torch.randn(64, 128, generator=torch.Generator().manual_seed(7))
    codes, scales = workloads.quantize_mxfp4(y)
    dec = orc.mxfp4_decode(codes, scales)
    amax = y.double().reshape(64, 4, 32).abs().amax(-1)
    expo = torch.floor(torch.log2(amax)) - 2
    assert np.array_equal(scales.numpy().astype(np.int64), (expo + 127).numpy().astype(np.int64))
    scale = torch.pow(2.0, expo).repeat_interleave(32, dim=1).numpy()
    m = np.abs(y.double().numpy()) / scale
    # nearest E2M1 point: half the local grid spacing (0.5 / 1 / 2), saturation above 6
    bound = scale * np.where(m < 2, 0.25, np.where(m < 4, 0.5, np.where(m <= 6, 1.0, m - 6.0)))
    err = np.abs(dec - y.double().numpy())
    assert np.all(err <= bound + 1e-12)
    assert np.all(np.abs(dec) <= 6.0 * scale)


# ------------------------------------------------------------------------------------
# Hadamard rotation and MXFP4 encoding (the DeepSeek-V4-Pro-MXFP4 page, Indexer: the
# query is rotated by a Hadamard transform before the FP4 dot products; OCP MX v1.0)
# ------------------------------------------------------------------------------------

def _popcount(v):
    return bin(int(v)).count("1")


@pytest.mark.parametrize("D", [32, 128, 512])
def test_hadamard_closed_form(orc, D):
    """The rotation of unit vector e_i is column i of the Sylvester matrix over sqrt(D):
    H[j][i] = (-1)^popcount(i & j) / sqrt(D), exactly (one nonzero term per output)."""
    out = orc.hadamard(np.eye(D, dtype=np.float32))  # row i = H e_i
    norm = np.float32(1.0 / np.sqrt(D))
    ref = np.array([[(-1.0) ** _popcount(i & j) for j in range(D)] for i in range(D)], dtype=np.float32) * norm
    np.testing.assert_array_equal(out, ref)


def test_hadamard_orthonormal(orc):
    """H H^T = I, H (H x) = x, and dot products survive the rotation (fp32 rounding)."""
    D = 128
    Hm = orc.hadamard(np.eye(D, dtype=np.float32)).astype(np.float64)
    np.testing.assert_allclose(Hm @ Hm.T, np.eye(D), atol=1e-6)
    rng = np.random.default_rng(11)
    x = rng.standard_normal((16, D)).astype(np.float32)
    y = rng.standard_normal((16, D)).astype(np.float32)
    np.testing.assert_allclose(orc.hadamard(orc.hadamard(x)), x, atol=2e-6)
    hx, hy = orc.hadamard(x).astype(np.float64), orc.hadamard(y).astype(np.float64)
    np.testing.assert_allclose((hx * hy).sum(-1), (x.astype(np.float64) * y).sum(-1), rtol=1e-5, atol=1e-4)


def test_mxfp4_encode_worked_block(orc):
    """A hand-encoded block (tests/golden/mxfp4_encode_block.json): every midpoint of the
    E2M1 grid (ties to the even code), saturation above 6, -0 and small negatives, and
    the block exponent floor(log2(amax)) - 2."""
    g = json.load(open(os.path.join(GOLD, "mxfp4_encode_block.json")))
    x = np.array(g["x"], dtype=np.float32).reshape(1, 32)
    codes, scales = orc.mxfp4_encode(x)
    nib = np.stack([codes[0] & 15, codes[0] >> 4], axis=-1).reshape(-1)
    assert scales[0].tolist() == [g["scale"]]
    assert nib.tolist() == g["nibbles"]


def test_mxfp4_encode_exact_and_zero(orc):
    """Blocks of grid values whose largest code is 6 or 7 encode exactly (decode gives them
    back); an all-zero block gets scale 2^-127 and zero codes."""
    grid = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    rng = np.random.default_rng(5)
    rows = []
    for e in (-3, 0, 5):
        v = rng.choice(grid, size=32) * rng.choice([-1.0, 1.0], size=32)
        v[rng.integers(32)] = rng.choice([4.0, 6.0])
        rows.append(v * 2.0 ** e)
    x = np.array(rows, dtype=np.float32)
    codes, scales = orc.mxfp4_encode(x)
    np.testing.assert_array_equal(orc.mxfp4_decode(codes, scales), x.astype(np.float64))
    c0, s0 = orc.mxfp4_encode(np.zeros((1, 64), dtype=np.float32))
    assert s0.tolist() == [[0, 0]] and not c0.any()


def test_mxfp4_encode_matches_generator(orc):
    """The oracle's encoder and the input generator's (written separately, in torch)
    agree code for code on random blocks."""
    y = torch.randn(200, 128, generator=torch.Generator().manual_seed(3)) * 3.0
    c1, s1 = orc.mxfp4_encode(y)
    c2, s2 = workloads.quantize_mxfp4(y)
    np.testing.assert_array_equal(c1, c2.numpy())
    np.testing.assert_array_equal(s1, s2.numpy())


def test_mxfp4_encode_hadamard_composes(orc):
    """Encoding with the rotation is encoding of the rotated rows."""
    x = np.random.default_rng(9).standard_normal((8, 256)).astype(np.float32)
    a = orc.mxfp4_encode(x, hadamard=True)
    b = orc.mxfp4_encode(orc.hadamard(x))
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


# ------------------------------------------------------------------------------------
# Top-k
# ------------------------------------------------------------------------------------

def test_topk_matches_full_sort(orc):
    """k largest finite scores, ties to the lower index (numpy lexsort), -1 padding."""
    T, N, k = 5, 300, 37
    s = np.round(_rand(T, N), 1)  # many exact ties
    s[1, ::3] = -np.inf
    s[4, :] = -np.inf
    s[4, [5, 9]] = [1.0, 1.0]
    idx, vals = orc.topk(s, k)
    for t in range(T):
        fin = np.flatnonzero(np.isfinite(s[t]))
        order = fin[np.lexsort((fin, -s[t, fin]))]
        m = min(k, len(order))
        np.testing.assert_array_equal(idx[t, :m], order[:m])
        assert np.all(idx[t, m:] == -1) and np.all(np.isneginf(vals[t, m:]))
    assert list(idx[4, :2]) == [5, 9]


def test_topk_distinct_matches_torch(orc):
    T, N, k = 4, 1000, 64
    s = np.stack([rng.permutation(N).astype(np.float64) * 0.25 - 50 for _ in range(T)])
    idx, _ = orc.topk(s, k)
    ref = torch.topk(torch.tensor(s), k, dim=1).indices.numpy()
    for t in range(T):
        assert set(idx[t]) == set(ref[t])


# ------------------------------------------------------------------------------------
# Attention with a sink: §6 p_i = e^{z_i} / (e^{z_s} + sum_j e^{z_j}); §3 working sets
# ------------------------------------------------------------------------------------

def _attn_case(T, H, D, N, k, B=1, swa_rows=0, window=0, seed=0):
    r = np.random.default_rng(seed)
    return dict(q=r.standard_normal((T, H, D)), kv=r.standard_normal((B, N, D)),
                sink=r.standard_normal(H), swa=r.standard_normal((B, max(swa_rows, 1), D)),
                idx=np.stack([r.choice(N, size=k, replace=False) for _ in range(T)]).astype(np.int32))


@pytest.mark.parametrize("k,expect", [(512, 640), (1024, 1152)])
def test_working_set_size_csa(orc, k, expect):
    """§3: the CSA core attention reads top-k + 128 SWA rows: 640 (Flash) / 1,152 (Pro).
    With q = 0 every logit is 0, so lse = log(L + e^sink) recovers L exactly."""
    T, H, D, n = 2, 3, 8, 1 << 20
    N = 4096
    c = _attn_case(T, H, D, N, k, swa_rows=128)
    q = np.zeros((T, H, D))
    out, lse = orc.sparse_attn(q, c["kv"], c["sink"], c["idx"], 0.1, c["swa"][:, :128] * 0 + _rand(1, 128, D),
                               np.array([n - 127]), 128, np.zeros(T), np.full(T, n))
    L = np.exp(lse) - np.exp(c["sink"])[None]
    np.testing.assert_allclose(L, expect, rtol=1e-12)


def test_working_set_size_hca(orc):
    """§3: HCA reads 8,192 summaries + 128 SWA = 8,320 rows at n = 2^20."""
    n, N, D, H = 1 << 20, 8192, 4, 2
    summ = _rand(1, N, D); swa = _rand(1, 128, D); sink = _rand(H)
    out, lse = orc.hca_attn(np.zeros((1, H, D)), summ, sink, 128, 0.5, swa, np.array([n - 127]), 128,
                            np.zeros(1), np.array([n]))
    np.testing.assert_allclose(np.exp(lse) - np.exp(sink), 8320, rtol=1e-12)
    # causal: a query at t sees floor(t/128) summaries and min(128, t+1) SWA rows
    for t in (0, 127, 128, 1000, 5000):
        _, lse = orc.hca_attn(np.zeros((1, H, D)), summ[:, :64], sink, 128, 0.5, _rand(1, 5200, D),
                              np.array([0]), 128, np.zeros(1), np.array([t]))
        L = min(t // 128, 64) + min(128, t + 1)
        np.testing.assert_allclose(np.exp(lse) - np.exp(sink), L, rtol=1e-12)


def test_sink_mass_below_one(orc):
    """§6: with a sink the row weights sum to 1 - e^{sink - lse} < 1; sink -> -inf gives 1,
    a large sink drives the output to 0."""
    T, H, D, N, k = 2, 4, 16, 64, 10
    c = _attn_case(T, H, D, N, k)
    const = np.full((1, N, D), 3.0)  # every row the same vector: o = (sum p) * row
    for sink, check in ((c["sink"], None), (np.full(H, -1e30), 1.0), (np.full(H, 60.0), 0.0)):
        out, lse = orc.sparse_attn(c["q"], const, sink, c["idx"], 0.2, None, np.zeros(1), 0,
                                   np.zeros(T), np.full(T, 10 ** 6))
        mass = out[..., 0] / 3.0
        np.testing.assert_allclose(mass, 1.0 - np.exp(sink[None] - lse), rtol=1e-12, atol=1e-15)
        assert np.all(mass <= 1.0)
        if check is not None:
            np.testing.assert_allclose(mass, check, atol=1e-12)
        else:
            assert np.all(mass < 1.0)


def test_no_sink_is_textbook_attention(orc):
    """§3: with the sink at -inf the sparse MQA is softmax(q K^T scale) K over the same
    rows (torch scaled_dot_product_attention, fp64, K = V shared)."""
    T, H, D, N, k, n = 3, 4, 32, 200, 24, 900
    c = _attn_case(T, H, D, N, k, swa_rows=300, seed=3)
    swa_pos0 = np.array([n - 250])
    out, _ = orc.sparse_attn(c["q"], c["kv"], np.full(H, -np.inf), c["idx"], 0.125, c["swa"],
                             swa_pos0, 128, np.zeros(T), np.full(T, n))
    for t in range(T):
        rows = [c["kv"][0, i] for i in c["idx"][t]]
        rows += [c["swa"][0, p - swa_pos0[0]] for p in range(n - 127, n + 1) if p - swa_pos0[0] < 300]
        K = torch.tensor(np.stack(rows))
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.tensor(c["q"][t])[None], K[None], K[None], scale=0.125)[0]
        np.testing.assert_allclose(out[t], ref.numpy(), rtol=1e-11, atol=1e-12)


def test_single_row_closed_form(orc):
    """One row: o = sigma(z - sink) row, z = scale <q, row> (the §6 formula with L = 1)."""
    H, D = 3, 16
    q, kv, sink = _rand(1, H, D), _rand(1, 5, D), _rand(H)
    out, lse = orc.sparse_attn(q, kv, sink, np.array([[2]]), 0.3, None, np.zeros(1), 0,
                               np.zeros(1), np.array([100]))
    z = 0.3 * q[0] @ kv[0, 2]
    sig = 1.0 / (1.0 + np.exp(sink - z))
    np.testing.assert_allclose(out[0], sig[:, None] * kv[0, 2][None], rtol=1e-13)
    np.testing.assert_allclose(lse[0], np.logaddexp(sink, z), rtol=1e-13)


def test_rope_rotation(orc):
    """§6 partial RoPE on the last R dims of q and inverse RoPE of o.
    (a) identity table = no RoPE; (b) keys stored rotated by the query's own angles give the
    unrotated result (rotations preserve dot products and the inverse undoes the rows'
    rotation); (c) D = R = 2 closed form with an explicit rotation matrix."""
    T, H, D, N, k, R = 2, 3, 16, 30, 8, 8
    c = _attn_case(T, H, D, N, k, seed=5)
    qs, qp = np.zeros(T), np.full(T, 999)
    base, lb = orc.sparse_attn(c["q"], c["kv"], c["sink"], c["idx"], 0.2, None, np.zeros(1), 0, qs, qp)
    ident = np.zeros((T, R // 2, 2)); ident[..., 0] = 1.0
    o1, _ = orc.sparse_attn(c["q"], c["kv"], c["sink"], c["idx"], 0.2, None, np.zeros(1), 0, qs, qp,
                            rope_cs=ident, rope_dim=R)
    np.testing.assert_allclose(o1, base, rtol=1e-14)
    # both queries use the same angle table so that one rotated key store serves both
    ang = rng.uniform(-3, 3, size=(R // 2))
    cs = np.stack([np.cos(ang), np.sin(ang)], -1)[None].repeat(T, 0)
    kv_rot = c["kv"].copy()
    x0, x1 = kv_rot[..., D - R::2].copy(), kv_rot[..., D - R + 1::2].copy()
    kv_rot[..., D - R::2] = x0 * np.cos(ang) - x1 * np.sin(ang)
    kv_rot[..., D - R + 1::2] = x0 * np.sin(ang) + x1 * np.cos(ang)
    o2, l2 = orc.sparse_attn(c["q"], kv_rot, c["sink"], c["idx"], 0.2, None, np.zeros(1), 0, qs, qp,
                             rope_cs=cs, rope_dim=R)
    np.testing.assert_allclose(o2, base, rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(l2, lb, rtol=1e-12)
    # closed form in 2-D: rotation matrix Rot(a) = [[cos, -sin], [sin, cos]]
    a = 0.7
    Rot = np.array([[np.cos(a), -np.sin(a)], [np.sin(a), np.cos(a)]])
    q2, v2 = np.array([[[1.0, 2.0]]]), np.array([[[0.5, -1.5]]])
    o3, _ = orc.sparse_attn(q2, v2, np.array([0.1]), np.array([[0]]), 1.0, None, np.zeros(1), 0,
                            np.zeros(1), np.array([5]), rope_cs=np.array([[[np.cos(a), np.sin(a)]]]),
                            rope_dim=2)
    z = (Rot @ q2[0, 0]) @ v2[0, 0]
    np.testing.assert_allclose(o3[0, 0], Rot.T @ v2[0, 0] / (1 + np.exp(0.1 - z)), rtol=1e-13)


def test_index_handling(orc):
    """Permuting topk_idxs leaves o unchanged; a -1 or out-of-range entry is dropped."""
    T, H, D, N, k = 3, 2, 8, 50, 12
    c = _attn_case(T, H, D, N, k, seed=9)
    qs, qp = np.zeros(T), np.full(T, 10 ** 5)
    base, lb = orc.sparse_attn(c["q"], c["kv"], c["sink"], c["idx"], 0.3, None, np.zeros(1), 0, qs, qp)
    perm = c["idx"][:, ::-1].copy()
    o, l = orc.sparse_attn(c["q"], c["kv"], c["sink"], perm, 0.3, None, np.zeros(1), 0, qs, qp)
    np.testing.assert_allclose(o, base, rtol=1e-12); np.testing.assert_allclose(l, lb, rtol=1e-13)
    pad = np.concatenate([c["idx"], np.full((T, 3), -1, np.int32), np.full((T, 1), N + 7, np.int32)], 1)
    o, l = orc.sparse_attn(c["q"], c["kv"], c["sink"], pad, 0.3, None, np.zeros(1), 0, qs, qp)
    np.testing.assert_allclose(o, base, rtol=1e-14)


def test_dense_special_case_matches_hca(orc):
    """When top-k covers every visible entry, CSA sparse attention equals the dense MQA of
    HCA run at ratio 4 over the same entries (the two oracle paths cross-check)."""
    T, H, D, N, n = 4, 3, 8, 40, 160
    r = np.random.default_rng(2)
    q, kv, sink = r.standard_normal((T, H, D)), r.standard_normal((2, N, D)), r.standard_normal(H)
    swa = r.standard_normal((2, 200, D))
    q_pos = np.array([3, 17, 100, 160]); q_seq = np.array([0, 1, 1, 0])
    idx = np.full((T, N), -1, np.int32)
    for t in range(T):
        vis = np.arange(q_pos[t] // 4)
        idx[t, :len(vis)] = r.permutation(vis)
    pos0 = np.array([0, 0])
    a, la = orc.sparse_attn(q, kv, sink, idx, 0.35, swa, pos0, 128, q_seq, q_pos)
    b, lb = orc.hca_attn(q, kv, sink, 4, 0.35, swa, pos0, 128, q_seq, q_pos)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(la, lb, rtol=1e-13)


def test_swa_window_rows(orc):
    """§6 SWA: a query at t reads raw positions max(0, t-127)..t (min(128, t+1) rows),
    and a position is read only if the caller's SWA buffer holds it."""
    H, D = 2, 4
    q = np.zeros((6, H, D)); sink = np.zeros(H)
    ts = np.array([0, 5, 126, 127, 128, 4000])
    swa = _rand(1, 4200, D)
    _, lse = orc.sparse_attn(q, _rand(1, 4, D), sink, np.full((6, 1), -1, np.int32), 1.0, swa,
                             np.array([0]), 128, np.zeros(6), ts)
    np.testing.assert_allclose(np.exp(lse) - 1.0, np.minimum(128, ts + 1)[:, None].repeat(H, 1), rtol=1e-12)
    _, lse = orc.sparse_attn(q[:1], _rand(1, 4, D), sink, np.full((1, 1), -1, np.int32), 1.0, swa[:, :50],
                             np.array([3970]), 128, np.zeros(1), np.array([4000]))
    np.testing.assert_allclose(np.exp(lse) - 1.0, 31, rtol=1e-12)  # positions 3970..4000


# ---- RMSNorm + RoPE of a row ("DeepSeek-V4 混合注意力" §6) ------------------------------

def test_rmsnorm_worked_rows(orc):
    """Closed forms: a constant row 3 with eps = 16 has rms 5, so y = 0.6 g; the row (3, 4)
    with eps = 0 has mean square 12.5, so y = (3, 4) * sqrt(2) / 5 * g."""
    g = np.array([1.0, -2.0, 0.5, 4.0])
    y = orc.rmsnorm_rope(np.full((1, 4), 3.0), g, 16.0)
    np.testing.assert_allclose(y[0], 0.6 * g, rtol=1e-15)
    y2 = orc.rmsnorm_rope(np.array([[3.0, 4.0]]), np.array([1.0, 2.0]), 0.0)
    np.testing.assert_allclose(y2[0], [3 * math.sqrt(2) / 5, 2 * 4 * math.sqrt(2) / 5], rtol=1e-15)


def test_rmsnorm_unit_mean_square_and_scale_invariance(orc):
    """With g = 1 and eps = 0 every output row has mean square 1 (before and after RoPE,
    a rotation), and positive scaling of a row does not change its output."""
    rng = np.random.default_rng(21)
    x = rng.standard_normal((7, 128)) * rng.uniform(0.1, 10, size=(7, 1))
    ang = rng.uniform(-3, 3, size=(7, 32))
    cs = np.stack([np.cos(ang), np.sin(ang)], -1)
    for c, R in ((None, 0), (cs, 64)):
        y = orc.rmsnorm_rope(x, np.ones(128), 0.0, rope_cs=c, rope_dim=R)
        np.testing.assert_allclose((y ** 2).mean(-1), 1.0, rtol=1e-13)
        np.testing.assert_allclose(orc.rmsnorm_rope(x * 37.5, np.ones(128), 0.0, rope_cs=c, rope_dim=R), y,
                                   rtol=1e-13, atol=1e-15)


def test_rmsnorm_matches_torch_rms_norm(orc):
    """Without RoPE it is torch's rms_norm over the last dim with the same weight and eps."""
    rng = np.random.default_rng(22)
    x = rng.standard_normal((33, 512))
    g = rng.uniform(0.5, 1.5, size=512)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (512,), weight=torch.from_numpy(g), eps=1e-6)
    np.testing.assert_allclose(orc.rmsnorm_rope(x, g, 1e-6), ref.numpy(), rtol=1e-13, atol=1e-15)


def test_rmsnorm_rope_special_angles_and_groups(orc):
    """Only the last R dims rotate, pair (D-R+2p, D-R+2p+1) by its own table entry: angle
    pi/2 maps (a, b) to (-b, a), angle pi to (-a, -b), angle 0 is the identity; row r takes
    table row r // group."""
    rng = np.random.default_rng(23)
    D, R, rows, group = 16, 8, 6, 2
    x = rng.standard_normal((rows, D))
    g = rng.uniform(0.5, 1.5, size=D)
    plain = orc.rmsnorm_rope(x, g, 1e-3)
    angles = np.array([np.pi / 2, np.pi, 0.0])  # table row j: every pair turns by angles[j]
    cs = np.zeros((rows // group, R // 2, 2))
    cs[..., 0] = np.round(np.cos(angles))[:, None]
    cs[..., 1] = np.round(np.sin(angles))[:, None]
    y = orc.rmsnorm_rope(x, g, 1e-3, rope_cs=cs, rope_dim=R, group=group)
    np.testing.assert_array_equal(y[:, :D - R], plain[:, :D - R])
    a, b = plain[:, D - R::2], plain[:, D - R + 1::2]
    for r in range(rows):
        j = r // group
        exp_a, exp_b = [(-b[r], a[r]), (-a[r], -b[r]), (a[r], b[r])][j]
        np.testing.assert_array_equal(y[r, D - R::2], exp_a)
        np.testing.assert_array_equal(y[r, D - R + 1::2], exp_b)


def test_rmsnorm_zero_row(orc):
    """A zero row stays zero, with eps > 0 (0 / sqrt(eps)) and with eps = 0 (the reading
    of 0 / 0)."""
    for eps in (0.0, 1e-6):
        np.testing.assert_array_equal(orc.rmsnorm_rope(np.zeros((2, 64)), np.ones(64), eps), 0.0)


# ------------------------------------------------------------------------------------
# Projections: §4.1 / §7 (the compressor's inputs formed from hidden rows) and §4.2 / §7
# (grouped output projection back to the model width)
# ------------------------------------------------------------------------------------

def test_matmul_nt_is_numpy_matmul(orc):
    X, Wm = _rand(7, 13), _rand(5, 13)
    np.testing.assert_allclose(orc.matmul_nt(X, Wm), X @ Wm.T, rtol=1e-13, atol=1e-13)
    # a zero-width contraction gives zeros
    assert np.all(orc.matmul_nt(np.zeros((3, 0)), np.zeros((4, 0))) == 0)


def test_compress_hidden_wiring(orc):
    """The four projections (numpy matmul) feed the compressor in the order W_Ca, W_Za,
    W_Cb, W_Zb, and the carry rows' b-projections become entry 0's previous block."""
    B, n, d, c = 2, 14, 6, 3
    H, W, cH = _rand(B, n, d), _rand(4, c, d, scale=0.5), _rand(B, 4, d)
    P = [H @ W[p].T for p in range(4)]
    ref = orc.compress(P[0], P[1], P[2], P[3], cH @ W[2].T, cH @ W[3].T, ratio=4, overlap=1)
    np.testing.assert_allclose(orc.compress_hidden(H, W, cH), ref, rtol=1e-12, atol=1e-12)
    ref0 = orc.compress(P[0], P[1], P[2], P[3], ratio=4, overlap=1)
    np.testing.assert_allclose(orc.compress_hidden(H, W), ref0, rtol=1e-12, atol=1e-12)
    assert orc.compress_hidden(H, W).shape == (B, n // 4, c)


@pytest.mark.parametrize("ratio,overlap,carry", [(4, 1, True), (4, 1, False), (128, 0, False)])
def test_compress_hidden_uniform_logits_is_mean_pooling(orc, ratio, overlap, carry):
    """Closed form: W_C = identity on the first c hidden dims and W_Z = 0 make every logit
    0, so each entry is the plain mean of its receptive field's hidden values: 8 rows (the
    previous block's and its own) for ratio 4, 4 for entry 0 without a carry, 128 for HCA."""
    B, c = 1, 5
    n = 3 * ratio + 1
    d = 8
    H = _rand(B, n, d)
    cH = _rand(B, 4, d) if carry else None
    npj = 2 * (1 + overlap)
    W = np.zeros((npj, c, d))
    for p in range(0, npj, 2):
        W[p, :, :c] = np.eye(c)
    got = orc.compress_hidden(H, W, cH, ratio=ratio, overlap=overlap)
    for i in range(n // ratio):
        rows = H[0, i * ratio:(i + 1) * ratio, :c]
        if overlap:
            prev = H[0, (i - 1) * ratio:i * ratio, :c] if i >= 1 else (cH[0, :, :c] if carry else None)
            if prev is not None:
                rows = np.concatenate([prev, rows])
        np.testing.assert_allclose(got[0, i], rows.mean(axis=0), rtol=1e-12, atol=1e-12)


def test_out_proj_groups(orc):
    """Each group's heads, side by side, through its own matrix (numpy per group); W_b maps
    the G results to the model width; G = 1 is a plain two-layer projection; a change to
    the heads of group g moves only group g's results."""
    T, H, D, G, d_g, dm = 3, 6, 4, 3, 5, 7
    o, Wa, Wb = _rand(T, H, D), _rand(G, d_g, (H // G) * D), _rand(dm, G * d_g)
    y_ref = np.concatenate([o[:, g * (H // G):(g + 1) * (H // G)].reshape(T, -1) @ Wa[g].T for g in range(G)], axis=1)
    y = orc.out_proj(o, Wa)
    np.testing.assert_allclose(y, y_ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(orc.out_proj(o, Wa, Wb), y_ref @ Wb.T, rtol=1e-12, atol=1e-12)
    Wa1 = _rand(1, d_g, H * D)
    np.testing.assert_allclose(orc.out_proj(o, Wa1, Wb[:, :d_g]), (o.reshape(T, -1) @ Wa1[0].T) @ Wb[:, :d_g].T,
                               rtol=1e-12, atol=1e-12)
    o2 = o.copy()
    o2[:, H // G:2 * (H // G)] += 1.0  # the heads of group 1
    d = orc.out_proj(o2, Wa) - y
    assert np.all(d[:, :d_g] == 0) and np.all(d[:, 2 * d_g:] == 0) and np.abs(d[:, d_g:2 * d_g]).max() > 0


# ------------------------------------------------------------------------------------
# Compressed-KV storage, §4.2 last paragraph (RoPE dims BF16, the rest FP8), read as
# OCP MX v1.0 MXFP8: E4M3 elements with one E8M0 scale per 32
# ------------------------------------------------------------------------------------

def test_e4m3_all_codes_against_torch_and_spec(orc):
    """All 256 codes: torch's own float8_e4m3fn (an independent implementation of the OCP
    format) gives the same values; the spec's extremes: 448 largest finite, 2^-6 smallest
    normal, 2^-9 smallest subnormal, S.1111.111 NaN."""
    t = orc.e4m3_table()
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(t), np.isnan(ref)) and np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    fin = ~np.isnan(ref)
    assert np.array_equal(t[fin], ref[fin])
    assert t[0x7E] == 448.0 and t[0x08] == 2.0 ** -6 and t[0x01] == 2.0 ** -9 and t[0x80] == 0.0


def test_kv8_layout_and_roundtrip(orc):
    assert orc.kv8_row_bytes(512, 64) == 592  # 448 codes + 128 bytes of bf16 + 14 scales + 2 pad
    rng2 = np.random.default_rng(7)
    # values on the grid: codes times a per-block power of two come back exactly when the
    # block's largest code is 448 (code 126), so that the block exponent picked by the
    # floor(log2 amax) - 8 rule is that power of two (with a smaller maximum, an amax whose
    # mantissa exceeds 1.75 would saturate: the MX rule clips there)
    codes = rng2.integers(0, 127, size=(3, 448))
    codes[:, ::32] = 126
    sign = rng2.choice([-1.0, 1.0], size=(3, 448))
    exps = rng2.integers(-20, 10, size=(3, 14))
    tab = orc.e4m3_table()
    x = np.zeros((3, 512), np.float32)
    x[:, :448] = (sign * tab[codes] * np.repeat(2.0 ** exps, 32, axis=1)).astype(np.float32)
    x[:, 448:] = torch.randn(3, 64).to(torch.bfloat16).float().numpy()  # bf16-exact rope dims
    y = orc.kv8_decode(orc.kv8_encode(x))
    np.testing.assert_array_equal(y, x.astype(np.float64))


def test_kv8_block_scale_rule_saturation_and_rne(orc):
    """Scale exponent floor(log2 amax) - 8 per block of 32; values beyond 448 * scale
    saturate; in-range elements round to nearest even exactly as torch's float8 cast; the
    RoPE dims are the bf16 round-to-nearest-even of the input."""
    x = np.zeros((1, 512), np.float32)
    x[0, 0] = 500.0                      # block 0: amax 500 -> e = 8 - 8 = 0 -> saturates to 448
    x[0, 1] = 0.75
    x[0, 32] = 3.0e-3                    # block 1: amax 0.003 -> e = -9 - 8 = -17
    x[0, 33] = -1.0e-3
    blk = np.random.default_rng(8).standard_normal(32).astype(np.float32) * 7
    x[0, 64:96] = blk                    # block 2: random values
    x[0, 448:] = np.linspace(-3, 3, 64, dtype=np.float32) + np.float32(1e-3)
    enc = orc.kv8_encode(x)
    sc = enc[0, 576:590].astype(int) - 127
    assert sc[0] == 0 and sc[1] == -17 and sc[2] == int(np.floor(np.log2(np.abs(blk).max()))) - 8
    assert sc[3] == -127                 # an all-zero block
    dec = orc.kv8_decode(enc)
    assert dec[0, 0] == 448.0 and dec[0, 1] == 0.75
    for b, lo in ((1, 32), (2, 64)):
        xs = torch.from_numpy(x[0, lo:lo + 32].astype(np.float64) / 2.0 ** sc[b]).to(torch.float32)
        ref = xs.to(torch.float8_e4m3fn).to(torch.float64).numpy() * 2.0 ** sc[b]
        np.testing.assert_array_equal(dec[0, lo:lo + 32], ref)
    ref_rope = torch.from_numpy(x[0, 448:]).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(dec[0, 448:], ref_rope)
