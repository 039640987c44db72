"""GPU parity: every library call against the fp64 oracle on the same seeded inputs.

Sizes are small enough for the oracle to finish in seconds but span several tiles of
each kernel and end on ragged tails. Each stage is fed generated inputs (never another
GPU stage's output), so a mismatch points at one kernel.
"""
import numpy as np
import pytest
import torch

import workloads as W
from tests.helpers import TOL_BF16, TOL_F32, assert_rel, check_topk_sets, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def csa():
    import long_context_compressed_amd as m
    m.lib()
    return m


def say(*a):
    print(*a, flush=True)


# ------------------------------------------------------------------------------------
# compressor
# ------------------------------------------------------------------------------------

@pytest.mark.parametrize("dt,B,n,c,carry", [
    (torch.float32, 1, 1024, 128, False),   # tiny prefill compressor
    (torch.bfloat16, 2, 1030, 200, True),   # ragged channels and a partial trailing block
    (torch.bfloat16, 1, 8192, 512, True),   # Pro prefill chunk shape
])
def test_compress_overlap4(csa, orc, dt, B, n, c, carry):
    say("compress4", dt, B, n, c, carry)
    s = 11 + n
    Ca, Cb, Za, Zb = (W.normal((B, n, c), s, nm, dtype=dt, device=DEV) for nm in ("Ca", "Cb", "Za", "Zb"))
    cC = W.normal((B, 4, c), s, "cC", dtype=dt, device=DEV) if carry else None
    cZ = W.normal((B, 4, c), s, "cZ", dtype=dt, device=DEV) if carry else None
    out = csa.compress(Ca, Za, Cb, Zb, cC, cZ, ratio=4, overlap=1)
    torch.cuda.synchronize()
    ref = orc.compress(Ca, Za, Cb, Zb, cC, cZ, ratio=4, overlap=1)
    assert out.shape == ref.shape == (B, n // 4, c)
    assert_rel(out, ref, TOL_F32 if dt == torch.float32 else TOL_BF16, "compress ratio 4")


def test_compress_bias_and_cache_stride(csa, orc):
    """Logit bias, and writing one new entry per sequence into a [B][N][c] cache."""
    B, n, c, N = 3, 4, 512, 10
    s = 77
    Ca, Cb, Za, Zb = (W.normal((B, n, c), s, nm, dtype=torch.bfloat16, device=DEV) for nm in ("a", "b", "c", "d"))
    cC, cZ = (W.normal((B, 4, c), s, nm, dtype=torch.bfloat16, device=DEV) for nm in ("e", "f"))
    bias = W.normal((8, c), s, "bias", device=DEV)
    cache = torch.zeros((B, N, c), dtype=torch.bfloat16, device=DEV)
    csa.compress(Ca, Za, Cb, Zb, cC, cZ, bias, ratio=4, overlap=1, out=cache[:, N - 1:N, :])
    torch.cuda.synchronize()
    ref = orc.compress(Ca, Za, Cb, Zb, cC, cZ, bias, ratio=4, overlap=1)
    assert_rel(cache[:, N - 1:N], ref, TOL_BF16, "compress into cache")
    assert torch.count_nonzero(cache[:, :N - 1]) == 0


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32])
def test_compress_batch(csa, orc, dt):
    """csa_compress_batch: a decode step's three poolings (two ratio-4 jobs with carries, one
    ratio-128 job into a strided cache view) in one launch equal the separate calls bit for
    bit and the oracle; with a job whose channel count rules out 16-byte rows the batch runs
    job by job and still matches."""
    say("compress_batch", dt)
    s = 4321
    B = 3
    jobs, refs = [], []
    for name, n, c, ratio in (("kv", 4, 512, 4), ("key", 4, 1024, 4), ("summ", 128, 256, 128), ("odd", 8, 200, 4)):
        t = {k: W.normal((B, n, c), s, name + k, dtype=dt, device=DEV) for k in ("Ca", "Za", "Cb", "Zb")}
        ov = 1 if ratio == 4 else 0
        carry = {k: W.normal((B, 4, c), s, name + "carry" + k, dtype=dt, device=DEV) for k in ("C", "Z")}
        cache = torch.zeros((B, 7, c), dtype=dt, device=DEV)
        out = cache[:, 5:5 + n // ratio, :]
        j = dict(C_a=t["Ca"], Z_a=t["Za"], ratio=ratio, out=out)
        if ov:
            j.update(C_b=t["Cb"], Z_b=t["Zb"], carry_C_b=carry["C"], carry_Z_b=carry["Z"])
        jobs.append(j)
        sep = csa.compress(t["Ca"], t["Za"], j.get("C_b"), j.get("Z_b"), j.get("carry_C_b"), j.get("carry_Z_b"),
                           ratio=ratio, overlap=ov)
        ref = orc.compress(t["Ca"], t["Za"], j.get("C_b"), j.get("Z_b"), j.get("carry_C_b"), j.get("carry_Z_b"),
                           ratio=ratio, overlap=ov)
        refs.append((name, cache, out, sep, ref))
    tol = TOL_F32 if dt == torch.float32 else TOL_BF16
    for sub in (jobs[:3], jobs):  # all 16-byte rows: one kernel; with the odd job: one launch per job
        for _, cache, *_ in refs:
            cache.zero_()
        csa.compress_batch(sub)
        torch.cuda.synchronize()
        for (name, cache, out, sep, ref) in refs[:len(sub)]:
            assert torch.equal(out, sep), f"{name}: batch vs separate call"
            assert_rel(out, ref, tol, f"compress_batch {name}")
            assert torch.count_nonzero(cache[:, :5]) == 0, f"{name}: wrote outside its rows"


@pytest.mark.parametrize("dt,B,n,c", [(torch.float32, 1, 128 * 5 + 17, 64), (torch.bfloat16, 2, 4096, 512)])
def test_compress_hca128(csa, orc, dt, B, n, c):
    say("compress128", dt, B, n, c)
    s = 5 + n
    Cz = W.normal((B, n, c), s, "C", dtype=dt, device=DEV)
    Zz = W.normal((B, n, c), s, "Z", dtype=dt, device=DEV)
    out = csa.compress(Cz, Zz, ratio=128, overlap=0)
    torch.cuda.synchronize()
    ref = orc.compress(Cz, Zz, ratio=128, overlap=0)
    assert_rel(out, ref, TOL_F32 if dt == torch.float32 else TOL_BF16, "compress ratio 128")


# ------------------------------------------------------------------------------------
# indexer
# ------------------------------------------------------------------------------------

def test_index_tiny_fp32(csa, orc):
    """Tiny prefill indexer: 1024 causal queries x 256 entries, fp32, w ~ U(0,1)."""
    inp = W.tiny_inputs(DEV)
    sc = csa.index_scores(inp["q_I"], inp["w"], inp["k_I"], inp["q_seq"], inp["q_pos"])
    torch.cuda.synchronize()
    ref = orc.index_scores(inp["q_I"], inp["w"], inp["k_I"], inp["q_seq"], inp["q_pos"])
    assert_rel(sc, ref, TOL_F32, "index tiny")


@pytest.mark.parametrize("T,B,N", [(3, 3, 1000), (5, 2, 700)])
def test_index_bf16_decode(csa, orc, T, B, N):
    """bf16 per-head keys; N ragged against the 256-entry workgroup span; some queries
    see only part of the store, one sees nothing."""
    s = 900 + N
    qI = W.normal((T, 64, 128), s, "q", dtype=torch.bfloat16, device=DEV)
    w = W.normal((T, 64), s, "w", device=DEV)
    kI = W.normal((B, N, 64, 128), s, "k", dtype=torch.bfloat16, device=DEV)
    q_seq = torch.tensor([t % B for t in range(T)], dtype=torch.int32, device=DEV)
    pos = [4 * N, 4 * N + 3, 1501, 2, 4 * N - 1][:T]
    q_pos = torch.tensor(pos, dtype=torch.int64, device=DEV)
    sc = csa.index_scores(qI, w, kI, q_seq, q_pos)
    torch.cuda.synchronize()
    ref = orc.index_scores(qI, w, kI, q_seq, q_pos)
    assert_rel(sc, ref, TOL_F32, "index bf16")


@pytest.mark.parametrize("T,B,N", [(3, 3, 1000), (6, 2, 4133), (40, 1, 257)])
def test_index_bf16_shared_keys(csa, orc, T, B, N):
    """One 128-dim key per entry shared by all 64 heads (matrix-core path): N ragged against
    the 16-entry tile and the 128-entry wavefront span, partly and fully masked queries."""
    say("index shared keys", T, B, N)
    s = 700 + N
    qI = W.normal((T, 64, 128), s, "q", dtype=torch.bfloat16, device=DEV)
    w = W.normal((T, 64), s, "w", device=DEV)
    kI = W.normal((B, N, 1, 128), s, "k", dtype=torch.bfloat16, device=DEV)
    q_seq = torch.tensor([t % B for t in range(T)], dtype=torch.int32, device=DEV)
    pos = [4 * N, 4 * N + 3, 1501, 2, 4 * N - 1, 61]
    q_pos = torch.tensor([pos[t % len(pos)] + (t // len(pos)) * 97 for t in range(T)], dtype=torch.int64,
                         device=DEV)
    sc = csa.index_scores(qI, w, kI, q_seq, q_pos)
    torch.cuda.synchronize()
    ref = orc.index_scores(qI, w, kI, q_seq, q_pos)
    assert_rel(sc, ref, TOL_F32, "index shared keys")


@pytest.mark.parametrize("T,N,B,p_lo,p_hi", [
    (70, 300, 1, 600, 669),      # one workgroup tile, ragged in both directions (matrix cores)
    (520, 650, 1, 1000, 3000),   # 3 x 6 tiles, causal: partly and fully masked tiles
    (1100, 1200, 1, 3000, 4800), # 9 x 10 tiles: two query tiles per XCD, a ragged entry group
    (10, 90, 2, 100, 400),       # two key stores: the per-query key stream
    (4, 1000, 4, 4001, 4001),    # decode shape: one query per store, every entry visible
    (6, 333, 1, 500, 1400),      # few queries on one store: the key stream, causal, ragged run
])
def test_index_mxfp4(csa, orc, T, N, B, p_lo, p_hi):
    """MXFP4 operands (E2M1 + one E8M0 scale per 32), causal prefill positions."""
    say("index_mxfp4", T, N, B)
    s = 4242 + T
    q32 = W.normal((T, 64, 128), s, "q", device=DEV)
    k32 = W.normal((B, N, 64, 128), s, "k", device=DEV)
    qc, qs = W.quantize_mxfp4(q32)
    kc, ks = W.quantize_mxfp4(k32)
    w = W.normal((T, 64), s, "w", device=DEV)
    q_seq = (torch.arange(T, dtype=torch.int32, device=DEV) % B)
    q_pos = torch.linspace(p_lo, p_hi, T, device=DEV).to(torch.int64)
    sc = csa.index_scores(qc, w, kc, q_seq, q_pos, q_I_scale=qs, k_I_scale=ks, mxfp4=True)
    torch.cuda.synchronize()
    qd = orc.mxfp4_decode(qc, qs)
    kd = orc.mxfp4_decode(kc, ks)
    ref = orc.index_scores(qd, w, kd, q_seq, q_pos)
    assert_rel(sc, ref, TOL_F32, "index mxfp4")


def _oracle_rescore(orc, q_I, w, k_I, cand, q_seq, q_pos, ratio=4):
    """Oracle scores [T][M] of per-query candidate lists (-inf for -1 / out-of-range slots)."""
    T, M = cand.shape
    N = k_I.shape[1]
    c = cand.cpu().numpy()
    out = np.full((T, M), -np.inf)
    for t in range(T):
        ok = (c[t] >= 0) & (c[t] < N)
        ids = c[t][ok].astype(np.int64)
        if len(ids) == 0:
            continue
        s_t = int(q_seq[t])
        kg = k_I[s_t].index_select(0, torch.from_numpy(ids).to(k_I.device))[None]
        ref = orc.index_scores(q_I[t:t + 1], w[t:t + 1], kg, np.zeros(1, dtype=np.int32),
                               q_pos[t:t + 1].cpu().numpy(), ratio=ratio, entry_ids=ids)
        out[t, ok] = ref[0]
    return out


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32])
def test_index_rescore(csa, orc, dt):
    """Scores of per-query candidate lists: valid, -1, past-N and not-yet-visible slots;
    a ragged list length (M = 150, three wavefronts' runs)."""
    say("index_rescore", dt)
    T, B, N, M = 5, 2, 3000, 150
    s = 515
    q = W.normal((T, 64, 128), s, "q", dtype=dt, device=DEV)
    k = W.normal((B, N, 64, 128), s, "k", dtype=dt, device=DEV)
    w = W.normal((T, 64), s, "w", device=DEV)
    q_seq = (torch.arange(T, dtype=torch.int32, device=DEV) % B)
    q_pos = torch.tensor([4 * N, 4 * N, 2000, 4 * N, 40], dtype=torch.int64, device=DEV)
    cand = torch.stack([torch.from_numpy(np.sort(W.distinct_sample(M, N, s, f"c{t}"))) for t in range(T)])
    cand = cand.to(torch.int32)
    cand[0, 7] = -1
    cand[1, 9] = N + 5
    cand = cand.to(DEV)
    sc = csa.index_rescore(q, w, k, cand, q_seq, q_pos)
    torch.cuda.synchronize()
    ref = _oracle_rescore(orc, q, w, k, cand, q_seq, q_pos)
    gpu = sc.cpu().double().numpy()
    fin = np.isfinite(ref)
    assert np.array_equal(fin, np.isfinite(gpu))
    assert np.all(gpu[~fin] == -np.inf)
    assert_rel(gpu[fin], ref[fin], TOL_F32, "rescore")


@pytest.mark.parametrize("T,M,k", [(6, 3000, 256), (3, 40000, 1024)])
def test_topk_ids(csa, orc, T, M, k):
    """Top-k over candidate lists: the chosen entries are the ids of the oracle's top-k
    positions (ties to the earlier position), in list order, -1 padded; M = 40,000 takes
    two reduction levels, the first reading the ids."""
    say("topk_ids", T, M, k)
    sc = torch.round(W.normal((T, M), 61 + M, "s", device=DEV) * 16) / 16  # ties
    sc[2, 100:] = -float("inf")                                          # fewer than k finite
    ids = torch.stack([torch.from_numpy(np.sort(W.distinct_sample(M, 200000, 61 + M, f"i{t}"))) for t in range(T)])
    ids = ids.to(torch.int32).to(DEV)
    idx, vals = csa.topk_ids(sc, ids, k, with_vals=True)
    torch.cuda.synchronize()
    rpos, _ = orc.topk(sc.cpu(), k)
    gi, ii = idx.cpu().numpy(), ids.cpu().numpy()
    for t in range(T):
        rp = rpos[t][rpos[t] >= 0]
        expect = sorted(ii[t][rp].tolist())
        got = gi[t][gi[t] >= 0]
        assert got.tolist() == expect, f"row {t}"
        assert np.all(gi[t, len(got):] == -1)


@pytest.mark.parametrize("D,dt,had", [(128, torch.float32, False), (128, torch.float32, True),
                                      (128, torch.bfloat16, True), (256, torch.float32, True),
                                      (512, torch.bfloat16, False), (512, torch.float32, True)])
def test_quantize_mxfp4(csa, orc, D, dt, had):
    """MXFP4 encoding with and without the Hadamard rotation: codes and scales bit-exact
    against the oracle (1,001 rows: random rows at block exponents from -40 to 40, a zero
    row, rows of grid midpoints, an outlier row)."""
    say("quantize_mxfp4", D, dt, had)
    rows = 1001
    x = W.normal((rows, D), 777 + D, "x", device=DEV)
    x = x * torch.pow(2.0, torch.linspace(-40, 40, rows, device=DEV)).unsqueeze(1)
    x[0] = 0.0
    mids = torch.tensor([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0], device=DEV)
    x[1] = mids.repeat(D // 8) * torch.where(torch.arange(D, device=DEV) % 3 == 0, -1.0, 1.0)
    x[2, :] = 0.01
    x[2, 5] = 1.0e4
    x = x.to(dt)
    codes, scales = csa.quantize_mxfp4(x, hadamard=had)
    torch.cuda.synchronize()
    rc, rs = orc.mxfp4_encode(x, hadamard=had)
    np.testing.assert_array_equal(scales.cpu().numpy(), rs)
    np.testing.assert_array_equal(codes.cpu().numpy(), rc)


@pytest.mark.parametrize("rows,D,dti,dto,R,group,inplace",
                         [(1, 512, torch.bfloat16, torch.bfloat16, 64, 1, False),
                          (1001, 512, torch.bfloat16, torch.bfloat16, 64, 128, False),
                          (333, 128, torch.float32, torch.float32, 0, 1, False),
                          (4097, 256, torch.float32, torch.bfloat16, 64, 1, False),
                          (2048, 512, torch.bfloat16, torch.bfloat16, 64, 1, True),
                          (777, 512, torch.float32, torch.float32, 512, 3, True),
                          (300000, 128, torch.bfloat16, torch.float32, 128, 7, False)])
def test_rmsnorm_rope(csa, orc, rows, D, dti, dto, R, group, inplace):
    """RMSNorm (gain, eps) + RoPE of the last R dims against the oracle, element by element:
    rows at scales 2^-20 .. 2^20, a zero row, a constant row, per-table-row angles shared by
    `group` consecutive rows, in place and out of place; the 300,000-row case runs past the
    grid cap (a grid-stride loop)."""
    say("rmsnorm_rope", rows, D, dti, dto, R, group, inplace)
    x = W.normal((rows, D), 4242 + D, "x", device=DEV)
    x = x * torch.pow(2.0, torch.linspace(-20, 20, rows, device=DEV)).unsqueeze(1)
    x[0] = 0.0 if rows > 1 else x[0]
    if rows > 2:
        x[1] = 3.0
    x = x.to(dti)
    g = W.uniform((D,), 4242 + D, "g", lo=-1.5, hi=1.5, device=DEV)
    nt = (rows + group - 1) // group
    cs = None
    if R > 0:
        cs = W.rope_table(torch.arange(nt, dtype=torch.int64) * 977 + 5, R).to(DEV)
    ref = orc.rmsnorm_rope(x, g, 1e-6, rope_cs=cs, rope_dim=R, group=group)
    xin = x.clone()
    out = csa.rmsnorm_rope(xin, g, 1e-6, rope_cs=cs, rope_group=group, out=xin if inplace else None,
                           out_dtype=dto)
    torch.cuda.synchronize()
    assert out.dtype == dto
    tol = TOL_F32 if dto == torch.float32 else TOL_BF16
    assert_rel(out, ref, tol, "rmsnorm_rope")
    if rows > 1:
        assert torch.all(out[0] == 0)


# ------------------------------------------------------------------------------------
# top-k
# ------------------------------------------------------------------------------------

@pytest.mark.parametrize("T,N,k", [(7, 256, 64), (5, 5000, 512), (3, 40000, 1024), (4, 262144, 1024),
                                   (6, 18432, 1024), (2, 100, 1024),
                                   # grids of >= 4 workgroups per compute unit (the 256-lane kernel)
                                   (1100, 5000, 512), (1030, 40000, 1024)])
def test_topk(csa, orc, T, N, k):
    say("topk", T, N, k)
    s = 31 + N
    sc = W.normal((T, N), s, "s", device=DEV)
    sc = torch.round(sc * 64) / 64  # many exact ties
    mask = W.uniform((T, N), s, "m", device=DEV) < 0.2
    sc[mask] = -float("inf")
    sc[0, :] = -float("inf")
    sc[0, : min(N, 10)] = 1.0       # fewer finite than k on row 0
    idx, vals = csa.topk(sc, k, with_vals=True)
    torch.cuda.synchronize()
    ref_idx, ref_vals = orc.topk(sc, k)
    gi = idx.cpu().numpy()
    # identical fp32 inputs on both sides: the sets agree exactly (ties to lower index)
    for t in range(T):
        assert sorted(gi[t][gi[t] >= 0].tolist()) == sorted(ref_idx[t][ref_idx[t] >= 0].tolist()), f"row {t}"
        m = int((ref_idx[t] >= 0).sum())
        assert np.all(gi[t, m:] == -1)
        assert np.all(np.diff(gi[t, :m]) > 0)  # ascending index order
        np.testing.assert_array_equal(vals.cpu().numpy()[t, :m], sc.cpu().numpy()[t, gi[t, :m]])


def test_topk_distinct_full_sort(csa):
    """A row of distinct values: the set equals torch.sort's first k."""
    T, N, k = 3, 33000, 700
    g = torch.Generator(device=DEV).manual_seed(5)
    sc = torch.stack([torch.randperm(N, generator=g, device=DEV).float() for _ in range(T)])
    idx, _ = csa.topk(sc, k)
    ref = torch.sort(sc, dim=1, descending=True).indices[:, :k]
    for t in range(T):
        assert set(idx[t].tolist()) == set(ref[t].tolist())


# ------------------------------------------------------------------------------------
# attention
# ------------------------------------------------------------------------------------

def _attn_inputs(seed, T, H, D, B, N, k, swa_rows, dt, pos, with_rope=True, bad_idx=True, rope_dim=64):
    q = W.normal((T, H, D), seed, "q", dtype=dt, device=DEV)
    kv = W.normal((B, N, D), seed, "kv", dtype=dt, device=DEV)
    swa = W.normal((B, swa_rows, D), seed, "swa", dtype=dt, device=DEV)
    sink = W.normal((H,), seed, "sink", device=DEV)
    q_seq = torch.tensor([t % B for t in range(T)], dtype=torch.int32, device=DEV)
    q_pos = torch.tensor(pos, dtype=torch.int64, device=DEV)
    idx = None
    if k > 0:
        idx = torch.stack([torch.from_numpy(W.distinct_sample(k, N, seed, f"i{t}")) for t in range(T)])
        idx = idx.to(torch.int32)
        if bad_idx:
            idx[0, 3] = -1
            idx[-1, 5] = N + 3
        idx = idx.to(DEV)
    swa_pos0 = torch.tensor([max(0, max(pos) - swa_rows + 1 - 3 * b) for b in range(B)], dtype=torch.int64,
                            device=DEV)
    rope = W.rope_table(q_pos.cpu(), rope_dim).to(DEV) if with_rope else None
    return q, kv, swa, sink, q_seq, q_pos, idx, swa_pos0, rope


@pytest.mark.parametrize("case", [
    # fp32 tiny-like (generic kernel)
    dict(T=40, H=8, D=128, B=1, N=256, k=64, swa=1024, dt=torch.float32, pos=None),
    # bf16 matrix-core kernel, split path (few queries): 300 + 128 slots = 13.4 tiles
    dict(T=3, H=128, D=512, B=3, N=2000, k=300, swa=130, dt=torch.bfloat16, pos=[8000, 8001, 100]),
    # bf16 matrix-core kernel, single pass (T * H / 64 >= 512)
    dict(T=256, H=128, D=512, B=1, N=600, k=64, swa=400, dt=torch.bfloat16, pos=None),
    # 64 heads (Flash shape), split path
    dict(T=2, H=64, D=512, B=2, N=900, k=512, swa=128, dt=torch.bfloat16, pos=[131072, 131072]),
    # SWA-only layers (k = 0, no compressed rows): Flash decode shape, a query near the start
    dict(T=3, H=64, D=512, B=2, N=900, k=0, swa=128, dt=torch.bfloat16, pos=[131072, 131072, 50]),
    # SWA-only, many queries (the 32-heads-per-wavefront kernel), and fp32
    dict(T=256, H=128, D=512, B=1, N=600, k=0, swa=400, dt=torch.bfloat16, pos=None),
    dict(T=40, H=8, D=128, B=1, N=256, k=0, swa=1024, dt=torch.float32, pos=None),
    # few queries, row-split form: 10 + 128 rows = 5 tiles over 3 splits of two row halves,
    # so the last split's second half starts past the end of its rows
    dict(T=2, H=128, D=512, B=2, N=900, k=10, swa=128, dt=torch.bfloat16, pos=[131072, 4000]),
    # one query of 64 heads: 64 split units of 2 tiles each
    dict(T=1, H=64, D=512, B=1, N=5000, k=4000, swa=128, dt=torch.bfloat16, pos=[40000]),
    # many queries with a top-k list longer than the 128-head kernel's LDS copy (1,024):
    # they take the 8-wavefront kernel; and one just inside it (ragged last main tile)
    dict(T=256, H=128, D=512, B=1, N=3000, k=1100, swa=200, dt=torch.bfloat16, pos=None),
    dict(T=256, H=128, D=512, B=1, N=3000, k=1000, swa=200, dt=torch.bfloat16, pos=None),
])
def test_sparse_attn(csa, orc, case):
    c = dict(case)
    say("sparse_attn", {k2: v for k2, v in c.items() if k2 != "dt"}, c["dt"])
    pos = c["pos"] or [int(p) for p in np.linspace(5, 1023, c["T"]).astype(np.int64)]
    q, kv, swa, sink, q_seq, q_pos, idx, p0, rope = _attn_inputs(
        100 + c["T"], c["T"], c["H"], c["D"], c["B"], c["N"], c["k"], c["swa"], c["dt"], pos)
    scale = 1.0 / np.sqrt(c["D"])
    out, lse = csa.sparse_attn(q, kv, sink, idx, scale, swa, p0, 128, q_seq, q_pos, rope, 64)
    torch.cuda.synchronize()
    ref, rlse = orc.sparse_attn(q, kv, sink, idx, scale, swa, p0, 128, q_seq, q_pos, rope, 64)
    tol = TOL_F32 if c["dt"] == torch.float32 else TOL_BF16
    assert_rel(out, ref, tol, "sparse attn out")
    assert_rel(lse, rlse, TOL_F32 if c["dt"] == torch.float32 else 2e-3, "sparse attn lse")


@pytest.mark.parametrize("T,H", [(256, 64), (256, 128), (2, 128), (3, 64)])
def test_sparse_attn_growing_logits(csa, orc, T, H):
    """Rows whose magnitude grows with the index, visited in index order: the running
    maximum keeps jumping by far more than the lazy headroom, so the rescaling of the
    accumulators runs many times (single pass for T=256, split otherwise); with 128 heads
    and 256 queries the 32-heads-per-wavefront kernel abandons its tile loop and takes its
    two-pass fallback."""
    say("sparse_attn growing", T, H)
    D, B, N, k = 512, 1, 700, 512
    pos = [8 * N + t for t in range(T)]
    # no RoPE here: the kernel rounds the rotated q to bf16 (as a model applying RoPE in
    # bf16 would), and with keys this large that rounding alone moves the logits by a few
    # percent of a unit, which is not what this test is about
    q, kv, swa, sink, q_seq, q_pos, idx, p0, rope = _attn_inputs(900 + T, T, H, D, B, N, k, 128,
                                                              torch.bfloat16, pos, with_rope=False,
                                                              bad_idx=False)
    grow = (1.0 + 0.05 * torch.arange(N, dtype=torch.float32, device=DEV)).view(1, N, 1)
    kv = (kv.float() * grow).to(torch.bfloat16)
    idx = torch.sort(idx, dim=1).values.contiguous()
    scale = 1.0 / np.sqrt(D)
    out, lse = csa.sparse_attn(q, kv, sink, idx, scale, swa, p0, 128, q_seq, q_pos, rope, 64)
    torch.cuda.synchronize()
    ref, rlse = orc.sparse_attn(q, kv, sink, idx, scale, swa, p0, 128, q_seq, q_pos, rope, 64)
    assert_rel(out, ref, TOL_BF16, "growing-logit attn out")
    assert_rel(lse, rlse, 2e-3, "growing-logit attn lse")


@pytest.mark.parametrize("case", [
    dict(T=4, H=128, N=300, B=4, pos=[300 * 128, 300 * 128 + 5, 200 * 128 - 1, 127]),   # decode, split
    dict(T=256, H=128, N=64, B=1, pos=None),                                          # causal prefill
    dict(T=5, H=8, N=40, B=2, pos=[5000, 5100, 130, 0, 4000], dt=torch.float32, D=128),
])
def test_hca_attn(csa, orc, case):
    c = dict(case)
    say("hca_attn", {k2: v for k2, v in c.items() if k2 != "dt"})
    dt = c.get("dt", torch.bfloat16)
    D = c.get("D", 512)
    pos = c["pos"] or [int(p) for p in np.linspace(60 * 128 - 40, 64 * 128 + 200, c["T"]).astype(np.int64)]
    q, summ, swa, sink, q_seq, q_pos, _, p0, rope = _attn_inputs(
        300 + c["T"], c["T"], c["H"], D, c["B"], c["N"], 0, 700, dt, pos)
    scale = 1.0 / np.sqrt(D)
    out, lse = csa.hca_attn(q, summ, sink, 128, scale, swa, p0, 128, q_seq, q_pos, rope, 64)
    torch.cuda.synchronize()
    ref, rlse = orc.hca_attn(q, summ, sink, 128, scale, swa, p0, 128, q_seq, q_pos, rope, 64)
    assert_rel(out, ref, TOL_F32 if dt == torch.float32 else TOL_BF16, "hca out")
    assert_rel(lse, rlse, TOL_F32 if dt == torch.float32 else 2e-3, "hca lse")


@pytest.mark.parametrize("T,H", [(256, 128), (4, 128)])
def test_hca_attn_growing_logits(csa, orc, T, H):
    """Summaries whose magnitude grows with the index: the running maximum keeps jumping
    past the headroom. With 256 queries x 128 heads the 32-heads-per-wavefront kernel
    abandons its tile loop and takes its two-pass fallback; with 4 queries the split path
    rescales its accumulators."""
    say("hca_attn growing", T, H)
    D, B, N = 512, 1, 96
    pos = [int(p) for p in np.linspace(N * 128 - 500, N * 128 + 50, T).astype(np.int64)]
    q, summ, swa, sink, q_seq, q_pos, _, p0, rope = _attn_inputs(700 + T, T, H, D, B, N, 0, 300,
                                                                 torch.bfloat16, pos, with_rope=False)
    grow = (1.0 + 0.2 * torch.arange(N, dtype=torch.float32, device=DEV)).view(1, N, 1)
    summ = (summ.float() * grow).to(torch.bfloat16)
    scale = 1.0 / np.sqrt(D)
    out, lse = csa.hca_attn(q, summ, sink, 128, scale, swa, p0, 128, q_seq, q_pos, rope, 64)
    torch.cuda.synchronize()
    ref, rlse = orc.hca_attn(q, summ, sink, 128, scale, swa, p0, 128, q_seq, q_pos, rope, 64)
    assert_rel(out, ref, TOL_BF16, "growing-logit hca out")
    assert_rel(lse, rlse, 2e-3, "growing-logit hca lse")


@pytest.mark.parametrize("R", [18, 96])
@pytest.mark.parametrize("mode", ["sparse", "hca"])
def test_attn_rope_dims(csa, orc, mode, R):
    """RoPE widths whose rotated dims start inside a 4-dim output group (18) or reach past
    the last 64 dims (96), on the many-query kernel (256 queries x 128 heads)."""
    say("attn rope dims", mode, R)
    T, H, D = 256, 128, 512
    scale = 1.0 / np.sqrt(D)
    if mode == "sparse":
        B, N, k = 1, 600, 64
        pos = [int(p) for p in np.linspace(5, 1023, T).astype(np.int64)]
        q, kv, swa, sink, q_seq, q_pos, idx, p0, rope = _attn_inputs(40 + R, T, H, D, B, N, k, 400, torch.bfloat16,
                                                                     pos, rope_dim=R)
        out, lse = csa.sparse_attn(q, kv, sink, idx, scale, swa, p0, 128, q_seq, q_pos, rope, R)
        torch.cuda.synchronize()
        ref, rlse = orc.sparse_attn(q, kv, sink, idx, scale, swa, p0, 128, q_seq, q_pos, rope, R)
    else:
        B, N = 1, 64
        pos = [int(p) for p in np.linspace(60 * 128 - 40, 64 * 128 + 200, T).astype(np.int64)]
        q, summ, swa, sink, q_seq, q_pos, _, p0, rope = _attn_inputs(50 + R, T, H, D, B, N, 0, 700, torch.bfloat16,
                                                                     pos, rope_dim=R)
        out, lse = csa.hca_attn(q, summ, sink, 128, scale, swa, p0, 128, q_seq, q_pos, rope, R)
        torch.cuda.synchronize()
        ref, rlse = orc.hca_attn(q, summ, sink, 128, scale, swa, p0, 128, q_seq, q_pos, rope, R)
    assert_rel(out, ref, TOL_BF16, f"{mode} attn out, R={R}")
    assert_rel(lse, rlse, 2e-3, f"{mode} attn lse, R={R}")


def test_working_set_sizes_on_gpu(csa):
    """With q = 0 every logit is 0, so lse = log(L + e^sink) gives the row count L:
    1,152 rows per Pro query (1,024 + 128) and 8,320 for HCA at 2^20 tokens."""
    n = 1 << 20
    T, H, D, B = 2, 128, 512, 2
    q = torch.zeros((T, H, D), dtype=torch.bfloat16, device=DEV)
    kv = W.normal((B, 4096, D), 1, "kv", dtype=torch.bfloat16, device=DEV)
    swa = W.normal((B, 128, D), 1, "swa", dtype=torch.bfloat16, device=DEV)
    sink = W.normal((H,), 1, "sink", device=DEV)
    idx = torch.stack([torch.randperm(4096, device=DEV)[:1024] for _ in range(T)]).to(torch.int32)
    q_seq = torch.arange(T, dtype=torch.int32, device=DEV)
    q_pos = torch.full((T,), n, dtype=torch.int64, device=DEV)
    p0 = torch.full((B,), n - 127, dtype=torch.int64, device=DEV)
    _, lse = csa.sparse_attn(q, kv, sink, idx, 0.04, swa, p0, 128, q_seq, q_pos)
    L = torch.exp(lse.double()) - torch.exp(sink.double())[None]
    assert torch.allclose(L, torch.full_like(L, 1152.0), rtol=1e-4)
    summ = W.normal((B, 8192, D), 2, "summ", dtype=torch.bfloat16, device=DEV)
    _, lse = csa.hca_attn(q, summ, sink, 128, 0.04, swa, p0, 128, q_seq, q_pos)
    L = torch.exp(lse.double()) - torch.exp(sink.double())[None]
    assert torch.allclose(L, torch.full_like(L, 8320.0), rtol=1e-4)


def test_determinism(csa):
    """Two runs of the same call are bitwise identical (no float atomics in reductions)."""
    q, kv, swa, sink, q_seq, q_pos, idx, p0, rope = _attn_inputs(
        7, 3, 128, 512, 3, 2000, 300, 130, torch.bfloat16, [8000, 8001, 100])
    a, la = csa.sparse_attn(q, kv, sink, idx, 0.05, swa, p0, 128, q_seq, q_pos, rope, 64)
    b, lb = csa.sparse_attn(q, kv, sink, idx, 0.05, swa, p0, 128, q_seq, q_pos, rope, 64)
    assert torch.equal(a, b) and torch.equal(la, lb)


# ------------------------------------------------------------------------------------
# tiny end-to-end chain: compress -> index -> top-k -> sparse attention
# ------------------------------------------------------------------------------------

def test_tiny_chain(csa, orc):
    inp = W.tiny_inputs(DEV)
    kvc = csa.compress(inp["C_a"], inp["Z_a"], inp["C_b"], inp["Z_b"], ratio=4, overlap=1)
    sc = csa.index_scores(inp["q_I"], inp["w"], inp["k_I"], inp["q_seq"], inp["q_pos"])
    idx, _ = csa.topk(sc, 64)
    out, lse = csa.sparse_attn(inp["q"], kvc, inp["sink"], idx, 1 / np.sqrt(128), inp["swa"], inp["swa_pos0"], 128,
                               inp["q_seq"], inp["q_pos"], inp["rope_cs"], 64)
    torch.cuda.synchronize()
    rkv = orc.compress(inp["C_a"], inp["Z_a"], inp["C_b"], inp["Z_b"], ratio=4, overlap=1)
    rsc = orc.index_scores(inp["q_I"], inp["w"], inp["k_I"], inp["q_seq"], inp["q_pos"])
    ridx, _ = orc.topk(rsc, 64)
    rout, rlse = orc.sparse_attn(inp["q"], rkv, inp["sink"], ridx, 1 / np.sqrt(128), inp["swa"], inp["swa_pos0"], 128,
                                 inp["q_seq"], inp["q_pos"], inp["rope_cs"], 64)
    assert_rel(kvc, rkv, TOL_F32, "chain compress")
    assert_rel(sc, rsc, TOL_F32, "chain index")
    n_near_ties = check_topk_sets(idx, rsc, 64)
    # attention compared on the queries whose selected set equals the oracle's
    same = np.array([set(idx[t].cpu().tolist()) == set(ridx[t].tolist()) for t in range(1024)])
    assert same.sum() >= 1024 - n_near_ties
    assert_rel(out, rout, TOL_F32, "chain attention", mask=same)


def test_many_query_launches_past_grid_y(csa, orc):
    """More queries than grid.y holds (70,000 > 65,535): the bf16 scan, the shared-key scan
    and top-k go out in slices of queries. Rows on both sides of the slice boundary, and
    the last rows, are checked against the oracle."""
    T, N, k = 70000, 40, 8
    s = 6565
    qI = W.normal((T, 64, 128), s, "q", dtype=torch.bfloat16, device=DEV)
    w = W.normal((T, 64), s, "w", device=DEV)
    kI = W.normal((1, N, 64, 128), s, "k", dtype=torch.bfloat16, device=DEV)
    kS = W.normal((1, N, 1, 128), s, "ks", dtype=torch.bfloat16, device=DEV)
    q_seq = torch.zeros(T, dtype=torch.int32, device=DEV)
    q_pos = (torch.arange(T, dtype=torch.int64, device=DEV) % (4 * N + 8))
    sc = csa.index_scores(qI, w, kI, q_seq, q_pos)
    scs = csa.index_scores(qI, w, kS, q_seq, q_pos)
    idx, _ = csa.topk(sc, k)
    torch.cuda.synchronize()
    rows = torch.tensor(list(range(0, 8)) + list(range(65530, 65545)) + list(range(T - 8, T)), device=DEV)
    sub = lambda x: x.index_select(0, rows)
    ref = orc.index_scores(sub(qI), sub(w), kI, sub(q_seq), sub(q_pos))
    assert_rel(sub(sc), ref, TOL_F32, "index bf16, sliced launch")
    ref_s = orc.index_scores(sub(qI), sub(w), kS, sub(q_seq), sub(q_pos))
    assert_rel(sub(scs), ref_s, TOL_F32, "index shared keys, sliced launch")
    check_topk_sets(sub(idx), to_np(sub(sc)), k)
