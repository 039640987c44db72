"""The C ABI library loads, exports every symbol include/csa.h declares, and rejects bad
arguments synchronously. Every call here either fails validation or has nothing to
launch (T = 0, N = 0, no complete block): none reaches a kernel, so the fake pointer
values are never dereferenced."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "csa.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"\b(csa_\w+|hca_attn)\s*\(", src)
    return sorted(set(names))


@pytest.fixture(scope="module")
def L():
    import long_context_compressed_amd as csa
    if not os.path.exists(csa.LIB_PATH):
        from long_context_compressed_amd import build
        build.build()
    return csa.lib()


def test_exports_every_declared_symbol(L):
    import long_context_compressed_amd as csa
    names = _declared()
    assert set(names) == set(csa.EXPORTS), names
    for n in names:
        assert hasattr(L, n), n


def test_status_strings(L):
    assert L.csa_status_str(0) == b"CSA_OK"
    assert L.csa_status_str(2) == b"CSA_EUNSUPPORTED"
    assert L.csa_status_str(99) == b"CSA_UNKNOWN"


def _compress(L, **kw):
    a = dict(Ca=1, Cb=1, Za=1, Zb=1, cCb=None, cZb=None, bias=None, B=1, n=16, c=8, ratio=4, overlap=1,
             dt=0, out=1, bstride=0)
    a.update(kw)
    return L.csa_compress(a["Ca"], a["Cb"], a["Za"], a["Zb"], a["cCb"], a["cZb"], a["bias"], a["B"], a["n"],
                          a["c"], a["ratio"], a["overlap"], a["dt"], a["out"], a["bstride"], None)


def test_compress_validation(L):
    assert _compress(L, ratio=8) == 2          # valid but not built
    assert _compress(L, ratio=4, overlap=0) == 2
    assert _compress(L, c=0) == 1
    assert _compress(L, dt=2) == 1             # MXFP4 is not a compressor dtype
    assert _compress(L, Cb=None) == 1
    assert _compress(L, cCb=1, cZb=None) == 1
    assert _compress(L, ratio=128, overlap=0, cCb=1, cZb=1) == 1
    assert _compress(L, bstride=5) == 1
    assert b"bstride" in L.csa_last_error()
    assert _compress(L, n=3) == 0               # no complete block: nothing to launch


def test_index_scores_validation(L):
    f = lambda **kw: L.csa_index_scores(*[kw.get(k, v) for k, v in (
        ("q", 1), ("qs", None), ("w", 1), ("k", 1), ("ks", None), ("qseq", 1), ("qpos", 1), ("T", 2), ("B", 1),
        ("N", 8), ("H", 64), ("D", 128), ("kh", 64), ("ratio", 4), ("dt", 1), ("scores", 1), ("st", None))])
    assert f(H=32, kh=32) == 2
    assert f(kh=5) == 1                         # k_heads is H_I or 1
    assert f(kh=1, dt=0) == 2                   # shared keys are built for bf16 only
    assert f(kh=1, dt=2) == 2
    assert f(kh=1, T=0) == 0
    assert f(D=100, dt=2) == 1
    assert f(D=96, dt=2) == 2
    assert f(dt=2) == 1                         # MXFP4 without scales
    assert f(w=None) == 1
    assert f(ratio=0) == 1
    assert f(T=0) == 0 and f(N=0) == 0


def test_topk_validation(L):
    assert L.csa_topk(1, 4, 100, 0, 1, None, None, 0, None) == 1
    assert L.csa_topk(1, 4, 100, 5000, 1, None, None, 0, None) == 2
    assert L.csa_topk(1, 4, 100, 10, None, None, None, 0, None) == 1
    assert L.csa_topk(1, 0, 100, 10, None, None, None, 0, None) == 0


def test_topk_noalloc_validation(L):
    assert L.csa_topk_noalloc(1, 4, 100, 0, 1, None, None) == 1
    assert L.csa_topk_noalloc(1, 4, 100, 5000, 1, None, None) == 2
    assert L.csa_topk_noalloc(1, 4, 100, 10, None, None, None) == 1
    assert L.csa_topk_noalloc(1, 0, 100, 10, None, None, None) == 0
    # more chunk winners than the library's fixed 16 MiB scratch holds: refused up front
    assert L.csa_topk_noalloc(1, 512, 262144, 1024, 1, None, None) == 3
    assert b"scratch" in L.csa_last_error()


def test_compress_batch_validation(L):
    import long_context_compressed_amd as csa
    Job = csa._CompressJob

    def jobs(**kw):
        a = dict(C_a=1, C_b=1, Z_a=1, Z_b=1, carry_C_b=None, carry_Z_b=None, logit_bias=None, B=1, n=8, c=512,
                 ratio=4, overlap=1, out=1, out_bstride=0)
        a.update(kw)
        arr = (Job * 1)(Job(**a))
        return C.cast(arr, C.c_void_p)
    assert L.csa_compress_batch(None, 0, 1, None) == 0
    assert L.csa_compress_batch(None, 1, 1, None) == 1
    assert L.csa_compress_batch(jobs(), 9, 1, None) == 2
    assert L.csa_compress_batch(jobs(), 1, 2, None) == 1          # MXFP4 is not a compressor dtype
    assert L.csa_compress_batch(jobs(ratio=8), 1, 1, None) == 2
    assert L.csa_compress_batch(jobs(carry_C_b=1), 1, 1, None) == 1
    assert L.csa_compress_batch(jobs(C_b=None), 1, 1, None) == 1
    assert L.csa_compress_batch(jobs(out_bstride=5), 1, 1, None) == 1
    assert L.csa_compress_batch(jobs(n=3), 1, 1, None) == 0       # no complete block: nothing to launch


def test_index_topk_validation(L):
    def f(**kw):
        a = dict(T=4, B=1, N=262144, H=64, D=128, ratio=4, k=1024, idx=1, ws=None, wsb=0)
        a.update(kw)
        return L.csa_index_topk(1, 1, 1, 1, 1, 1, 1, a["T"], a["B"], a["N"], a["H"], a["D"], a["ratio"], a["k"],
                                a["idx"], None, a["ws"], a["wsb"], None)
    assert f(k=0) == 1
    assert f(k=5000) == 2
    assert f(H=32) == 2
    assert f(T=70000) == 2
    assert f(ratio=0) == 1
    assert f(idx=None) == 1
    assert f(T=0) == 0
    # the chunk winners need a workspace: refused before any launch
    assert L.csa_index_topk_workspace_bytes(4, 262144, 1024) >= 4 * 64 * 1024 * 8
    assert f(wsb=16) == 3
    # one chunk: its winners are the output, no workspace at all
    assert L.csa_index_topk_workspace_bytes(4, 4096, 1024) == 0


def test_attn_validation(L):
    def f(**kw):
        a = dict(q=1, kv=1, sink=1, idx=1, k=4, scale=0.1, swa=1, p0=1, rows=8, win=128, qseq=1, qpos=1,
                 cs=None, R=0, T=2, B=1, N=8, H=8, D=128, dt=0, out=1, lse=None, ws=None, wsb=0)
        a.update(kw)
        return L.csa_sparse_attn(a["q"], a["kv"], a["sink"], a["idx"], a["k"], C.c_float(a["scale"]), a["swa"],
                                 a["p0"], a["rows"], a["win"], a["qseq"], a["qpos"], a["cs"], a["R"], a["T"],
                                 a["B"], a["N"], a["H"], a["D"], a["dt"], a["out"], a["lse"], a["ws"], a["wsb"],
                                 None)
    assert f(D=100) == 2
    assert f(D=2048) == 2
    assert f(cs=1, R=3) == 1
    assert f(cs=1, R=256) == 1
    assert f(sink=None) == 1
    assert f(idx=None) == 1
    assert f(p0=None) == 1
    assert f(scale=float("nan")) == 1
    assert f(scale=0.0) == 2          # the matrix-core kernels assume a positive scale
    assert f(scale=-0.1) == 2
    assert f(k=-1) == 1
    assert f(dt=2) == 1
    assert f(T=0) == 0
    g = lambda **kw: L.hca_attn(1, 1, 1, kw.get("ratio", 128), C.c_float(kw.get("scale", 0.1)), 1, 1, 8, 128, 1,
                                1, None, 0, 2, 1, 8, 8, 128, 0, 1, None, None, 0, None)
    assert g(ratio=0) == 1
    assert g(scale=-1.0) == 2


def test_quantize_mxfp4_validation(L):
    f = lambda **kw: L.csa_quantize_mxfp4(kw.get("x", 1), kw.get("rows", 4), kw.get("D", 128), kw.get("dt", 0),
                                          kw.get("had", 1), kw.get("codes", 1), kw.get("scales", 1),
                                          kw.get("gr", 0), kw.get("gs", 0), None)
    assert f(D=100) == 1                        # not a multiple of 32
    assert f(D=96) == 2                         # valid, not built
    assert f(dt=2) == 1                         # MXFP4 is the output, not an input dtype
    assert f(x=None) == 1 and f(codes=None) == 1
    assert f(rows=-1) == 1
    assert f(gr=64, gs=10) == 1                 # groups would overlap
    assert f(gr=-1) == 1
    assert f(rows=0) == 0


def test_rmsnorm_rope_validation(L):
    f = lambda **kw: L.csa_rmsnorm_rope(kw.get("x", 16), kw.get("dti", 1), kw.get("rows", 4), kw.get("D", 512),
                                        kw.get("g", 48), kw.get("eps", 1e-6), kw.get("cs", 64), kw.get("R", 64),
                                        kw.get("grp", 1), kw.get("out", 32), kw.get("dto", 1), None)
    assert f(D=48) == 1                         # R = 64 > D
    assert f(D=100) == 2 and f(D=100, R=0) == 2  # valid, not built
    assert f(D=0) == 1 and f(rows=-1) == 1
    assert f(dti=2) == 1 and f(dto=2) == 1      # MXFP4 is neither an input nor an output here
    assert f(eps=-1.0) == 1 and f(eps=float("inf")) == 1 and f(eps=float("nan")) == 1
    assert f(R=3) == 1 and f(R=-2) == 1 and f(R=514) == 1
    assert f(grp=0) == 1
    assert f(R=2) == 2 and f(D=256, R=6) == 2  # R not a multiple of D / 64: not built
    assert f(x=None) == 1 and f(g=None) == 1 and f(out=None) == 1 and f(cs=None) == 1
    assert f(out=16, dto=0) == 1                # in place with a dtype change
    assert f(x=18) == 1 and f(out=40) == 1 and f(g=52) == 1 and f(cs=72) == 1  # not 16-byte aligned
    assert f(rows=0) == 0


def test_index_rescore_and_topk_ids_validation(L):
    r = lambda **kw: L.csa_index_rescore(*[kw.get(k, v) for k, v in (
        ("q", 1), ("w", 1), ("k", 1), ("cand", 1), ("M", 16), ("qseq", 1), ("qpos", 1), ("T", 2), ("B", 1),
        ("N", 8), ("H", 64), ("D", 128), ("ratio", 4), ("dt", 1), ("scores", 1), ("st", None))])
    assert r(dt=2) == 1                         # candidate lists re-score exact (bf16 / fp32) keys
    assert r(H=32) == 2
    assert r(cand=None) == 1
    assert r(M=-1) == 1
    assert r(T=0) == 0 and r(M=0) == 0
    assert L.csa_topk_ids(1, 1, 4, 100, 0, 1, None, None, 0, None) == 1
    assert L.csa_topk_ids(1, 1, 4, 100, 5000, 1, None, None, 0, None) == 2
    assert L.csa_topk_ids(1, None, 4, 100, 10, 1, None, None, 0, None) == 1
    assert L.csa_topk_ids(1, 1, 0, 100, 10, None, None, None, 0, None) == 0


def test_binding_rejects_short_rope_tables_before_launch():
    """The Python binding checks what the ABI cannot (table extents) and raises before any
    call is made: CPU tensors here, so reaching a launch would fail differently."""
    import torch
    import long_context_compressed_amd as csa
    x = torch.zeros((8, 4, 128), dtype=torch.bfloat16)
    g = torch.ones(128)
    with pytest.raises(ValueError, match="rope_group"):
        csa.rmsnorm_rope(x, g, 1e-6, rope_cs=torch.zeros((2, 64)), rope_group=4)  # needs 8 angle rows
    with pytest.raises(ValueError, match="gains"):
        csa.rmsnorm_rope(x, torch.ones(64), 1e-6)
    q = torch.zeros((3, 8, 128), dtype=torch.bfloat16)
    kv = torch.zeros((1, 16, 128), dtype=torch.bfloat16)
    idx = torch.zeros((3, 4), dtype=torch.int32)
    seq = torch.zeros(3, dtype=torch.int32)
    pos = torch.full((3,), 64, dtype=torch.int64)
    sink = torch.zeros(8)
    with pytest.raises(ValueError, match="rows for 3 queries"):
        csa.sparse_attn(q, kv, sink, idx, 0.1, None, None, 0, seq, pos, torch.zeros((2, 64)), 64)
    with pytest.raises(ValueError, match="rows for 3 queries"):
        csa.hca_attn(q, kv, sink, 4, 0.1, None, None, 0, seq, pos, torch.zeros((2, 64)), 64)
    with pytest.raises(ValueError, match="topk_idxs"):
        csa.sparse_attn(q, kv, sink, idx[:2], 0.1, None, None, 0, seq, pos)
