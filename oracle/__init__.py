"""ctypes wrapper of the fp64 CPU oracle (oracle.c).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the GPU library. Inputs are converted to
float64 numpy arrays here (bf16 and fp32 widen exactly); MXFP4 bytes are decoded
by the oracle's own table.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# CSA_ORACLE_LIB names another build of oracle.c (the sanitizer test's instrumented one)
LIB_PATH = os.environ.get("CSA_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
SRC_PATH = os.path.join(_HERE, "oracle.c")


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc (-O2, OpenMP, strict IEEE: no fast-math)."""
    if force or not os.path.exists(LIB_PATH):
        tmp = LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-std=c11", "-O2", "-fopenmp", "-fPIC", "-shared",
                               "-Wall", "-Wextra", "-o", tmp, SRC_PATH, "-lm"])
        os.replace(tmp, LIB_PATH)
    return LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        L = C.CDLL(LIB_PATH)
        P = C.c_void_p
        i32, i64, f64 = C.c_int, C.c_int64, C.c_double
        L.oracle_compress.argtypes = [P, P, P, P, P, P, P, i32, i64, i32, i32, i32, P]
        L.oracle_matmul_nt.argtypes = [P, P, i64, i64, i64, P]
        L.oracle_kv8_row_bytes.argtypes = [i32, i32]
        L.oracle_kv8_encode.argtypes = [P, i64, i32, i32, P]
        L.oracle_kv8_decode.argtypes = [P, i64, i32, i32, P]
        L.oracle_e4m3_table.argtypes = [P]
        L.oracle_compress_hidden.argtypes = [P, P, P, P, i32, i64, i64, i32, i32, i32, P]
        L.oracle_out_proj.argtypes = [P, i32, i32, i32, i32, P, i32, P, i32, P]
        L.oracle_index_scores.argtypes = [P, P, P, P, P, P, i32, i32, i64, i32, i32, i32, i32, P]
        L.oracle_mxfp4_decode.argtypes = [P, P, i64, P]
        L.oracle_mxfp4_encode.argtypes = [P, i64, i32, i32, P, P]
        L.oracle_hadamard.argtypes = [P, i64, i32, P]
        L.oracle_topk.argtypes = [P, i32, i64, i32, P, P]
        L.oracle_rmsnorm_rope.argtypes = [P, i64, i32, P, f64, P, i32, i64, P]
        L.oracle_sparse_attn.argtypes = [P, P, P, P, i32, f64, P, P, i32, i32, P, P, P, i32,
                                         i32, i32, i64, i32, i32, P, P]
        L.oracle_hca_attn.argtypes = [P, P, P, i32, f64, P, P, i32, i32, P, P, P, i32,
                                      i32, i32, i64, i32, i32, P, P]
        for f in ("oracle_kv8_row_bytes", "oracle_kv8_encode", "oracle_kv8_decode", "oracle_e4m3_table",
                  "oracle_compress", "oracle_matmul_nt", "oracle_compress_hidden", "oracle_out_proj", "oracle_index_scores", "oracle_mxfp4_decode", "oracle_mxfp4_encode",
                  "oracle_hadamard", "oracle_topk", "oracle_rmsnorm_rope",
                  "oracle_sparse_attn", "oracle_hca_attn"):
            getattr(L, f).restype = C.c_int
        _lib = L
    return _lib


def threads() -> int:
    """OpenMP threads the oracle uses (OMP_NUM_THREADS, else the affinity mask)."""
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit():
        return int(env)
    return len(os.sched_getaffinity(0))


# ---- marshalling -------------------------------------------------------------------

def _f64(x):
    if x is None:
        return None
    if hasattr(x, "detach"):  # torch tensor: widen on the host (exact for fp32 / bf16)
        import torch
        x = x.detach().to("cpu", torch.float64).numpy()
    return np.ascontiguousarray(x, dtype=np.float64)


def _arr(x, dt):
    if x is None:
        return None
    if hasattr(x, "detach"):
        x = x.detach().cpu().numpy()
    return np.ascontiguousarray(x, dtype=dt)


def _p(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what}: invalid arguments (rc={rc})")


# ---- the five steps ----------------------------------------------------------------

def compress(C_a, Z_a, C_b=None, Z_b=None, carry_C_b=None, carry_Z_b=None, bias=None,
             ratio=4, overlap=1):
    """Compressed entries [B][n//ratio][c] (fp64)."""
    Ca, Za = _f64(C_a), _f64(Z_a)
    B, n, c = Ca.shape
    Cb, Zb = _f64(C_b), _f64(Z_b)
    cCb, cZb, bi = _f64(carry_C_b), _f64(carry_Z_b), _f64(bias)
    out = np.empty((B, n // ratio, c), dtype=np.float64)
    rc = lib().oracle_compress(_p(Ca), _p(Cb), _p(Za), _p(Zb), _p(cCb), _p(cZb), _p(bi),
                               B, n, c, ratio, overlap, _p(out))
    _check(rc, "compress")
    return out


def kv8_row_bytes(D=512, R=64):
    n = lib().oracle_kv8_row_bytes(D, R)
    if n < 0:
        raise ValueError("kv8: D - R must be a non-negative multiple of 32")
    return n


def kv8_encode(x, R=64):
    """Rows x [..., D] (taken as fp32) -> uint8 [..., kv8_row_bytes(D, R)]: MXFP8 (E4M3 +
    E8M0 per 32) for dims 0..D-R-1, bf16 for the last R dims."""
    xa = _arr(x, np.float32)
    D = xa.shape[-1]
    rows = xa.size // D if D else 0
    out = np.zeros(xa.shape[:-1] + (kv8_row_bytes(D, R),), dtype=np.uint8)
    _check(lib().oracle_kv8_encode(_p(xa), rows, D, R, _p(out)), "kv8_encode")
    return out


def kv8_decode(rows, D=512, R=64):
    """uint8 rows [..., kv8_row_bytes(D, R)] -> fp64 [..., D]."""
    ra = _arr(rows, np.uint8)
    n = ra.size // kv8_row_bytes(D, R)
    out = np.empty(ra.shape[:-1] + (D,), dtype=np.float64)
    _check(lib().oracle_kv8_decode(_p(ra), n, D, R, _p(out)), "kv8_decode")
    return out


def e4m3_table():
    out = np.empty(256, dtype=np.float64)
    _check(lib().oracle_e4m3_table(_p(out)), "e4m3_table")
    return out


def matmul_nt(X, W):
    """Y = X W^T (fp64): X [M][K], W [N][K]."""
    Xa, Wa = _f64(X), _f64(W)
    M, K = Xa.shape
    N = Wa.shape[0]
    Y = np.empty((M, N), dtype=np.float64)
    _check(lib().oracle_matmul_nt(_p(Xa), _p(Wa), M, N, K, _p(Y)), "matmul_nt")
    return Y


def compress_hidden(H, W, carry_H=None, bias=None, ratio=4, overlap=1):
    """Compressed entries [B][n//ratio][c] (fp64) of hidden rows H [B][n][d] through the
    projections W [(1+overlap)*2][c][d] (W_Ca, W_Za, W_Cb, W_Zb)."""
    Ha, Wa = _f64(H), _f64(W)
    B, n, d = Ha.shape
    c = Wa.shape[1]
    cH, bi = _f64(carry_H), _f64(bias)
    out = np.empty((B, n // ratio, c), dtype=np.float64)
    rc = lib().oracle_compress_hidden(_p(Ha), _p(cH), _p(Wa), _p(bi), B, n, d, c, ratio, overlap, _p(out))
    _check(rc, "compress_hidden")
    return out


def out_proj(o, W_a, W_b=None):
    """Grouped output projection (fp64): o [T][H][D], W_a [G][d_g][(H/G)*D], W_b
    [d_model][G*d_g] or None -> [T][d_model] (or [T][G*d_g])."""
    oa, wa = _f64(o), _f64(W_a)
    T, H, D = oa.shape
    G, d_g, _ = wa.shape
    wb = _f64(W_b)
    width = wb.shape[0] if wb is not None else G * d_g
    out = np.empty((T, width), dtype=np.float64)
    rc = lib().oracle_out_proj(_p(oa), T, H, D, G, _p(wa), d_g, _p(wb), width if wb is not None else 0, _p(out))
    _check(rc, "out_proj")
    return out


def mxfp4_decode(codes, scales):
    """Decode MXFP4 bytes [..., D/2] + scales [..., D/32] to fp64 [..., D]."""
    cd = _arr(codes, np.uint8)
    sc = _arr(scales, np.uint8)
    D = cd.shape[-1] * 2
    out = np.empty(cd.shape[:-1] + (D,), dtype=np.float64)
    _check(lib().oracle_mxfp4_decode(_p(cd), _p(sc), out.size, _p(out)), "mxfp4_decode")
    return out


def mxfp4_encode(x, hadamard=False):
    """MXFP4 codes [..., D/2] and E8M0 scales [..., D/32] (uint8) of x [..., D] taken as
    float32 (bf16 and fp32 inputs widen exactly), after the single-precision Hadamard
    rotation when `hadamard`."""
    if hasattr(x, "detach"):  # torch tensor: widen on the host (exact for bf16)
        import torch
        x = x.detach().to("cpu", torch.float32).numpy()
    xf = np.ascontiguousarray(x, dtype=np.float32)
    D = xf.shape[-1]
    rows = xf.size // D
    codes = np.empty(xf.shape[:-1] + (D // 2,), dtype=np.uint8)
    scales = np.empty(xf.shape[:-1] + (D // 32,), dtype=np.uint8)
    _check(lib().oracle_mxfp4_encode(_p(xf), rows, D, int(bool(hadamard)), _p(codes), _p(scales)), "mxfp4_encode")
    return codes, scales


def hadamard(x):
    """The single-precision Hadamard rotation of the rows of x [..., D] (float32 out)."""
    if hasattr(x, "detach"):
        import torch
        x = x.detach().to("cpu", torch.float32).numpy()
    xf = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty_like(xf)
    D = xf.shape[-1]
    _check(lib().oracle_hadamard(_p(xf), xf.size // D, D, _p(out)), "hadamard")
    return out


def rmsnorm_rope(x, g, eps, rope_cs=None, rope_dim=0, group=1):
    """RMSNorm of each row of x [..., D] with gains g [D], then the last rope_dim dims
    rotated by rope_cs [rows // group][rope_dim/2][2] (row r takes table row r // group);
    fp64 out of x's shape."""
    xx, gg = _f64(x), _f64(g)
    D = xx.shape[-1]
    rows = xx.size // D
    cs = _f64(rope_cs)
    R = rope_dim if cs is not None else 0
    out = np.empty(xx.shape, dtype=np.float64)
    _check(lib().oracle_rmsnorm_rope(_p(xx), rows, D, _p(gg), float(eps), _p(cs), R, int(group), _p(out)),
           "rmsnorm_rope")
    return out


def index_scores(q_I, w, k_I, q_seq, q_pos, ratio=4, entry_ids=None):
    """Scores [T][N] (fp64, -inf where masked). k_I: [B][N][kh][Dh]."""
    q, wv, k = _f64(q_I), _f64(w), _f64(k_I)
    T, H, Dh = q.shape
    B, N, kh, _ = k.shape
    qs, qp = _arr(q_seq, np.int32), _arr(q_pos, np.int64)
    eid = _arr(entry_ids, np.int64)
    out = np.empty((T, N), dtype=np.float64)
    rc = lib().oracle_index_scores(_p(q), _p(wv), _p(k), _p(qs), _p(qp), _p(eid),
                                   T, B, N, H, Dh, kh, ratio, _p(out))
    _check(rc, "index_scores")
    return out


def topk(scores, k):
    """(idx [T][k] int32 sorted by score desc / index asc, -1 padded; vals [T][k])."""
    s = _f64(scores)
    T, N = s.shape
    idx = np.empty((T, k), dtype=np.int32)
    vals = np.empty((T, k), dtype=np.float64)
    _check(lib().oracle_topk(_p(s), T, N, k, _p(idx), _p(vals)), "topk")
    return idx, vals


def sparse_attn(q, kv, sink, topk_idxs, softmax_scale, swa, swa_pos0, window, q_seq, q_pos,
                rope_cs=None, rope_dim=0):
    """(out [T][H][D], lse [T][H]) in fp64."""
    qq, kk, sk, sw = _f64(q), _f64(kv), _f64(sink), _f64(swa)
    T, H, D = qq.shape
    B, N, _ = kk.shape
    idx = _arr(topk_idxs, np.int32)
    k = idx.shape[1] if idx is not None else 0
    p0 = _arr(swa_pos0, np.int64)
    swa_rows = sw.shape[1] if sw is not None else 0
    cs = _f64(rope_cs)
    out = np.empty((T, H, D), dtype=np.float64)
    lse = np.empty((T, H), dtype=np.float64)
    rc = lib().oracle_sparse_attn(_p(qq), _p(kk), _p(sk), _p(idx), k, float(softmax_scale),
                                  _p(sw), _p(p0), swa_rows, window,
                                  _p(_arr(q_seq, np.int32)), _p(_arr(q_pos, np.int64)),
                                  _p(cs), rope_dim if cs is not None else 0,
                                  T, B, N, H, D, _p(out), _p(lse))
    _check(rc, "sparse_attn")
    return out, lse


def hca_attn(q, summ, sink, ratio, softmax_scale, swa, swa_pos0, window, q_seq, q_pos,
             rope_cs=None, rope_dim=0):
    """(out [T][H][D], lse [T][H]) in fp64."""
    qq, sm, sk, sw = _f64(q), _f64(summ), _f64(sink), _f64(swa)
    T, H, D = qq.shape
    B, N, _ = sm.shape
    p0 = _arr(swa_pos0, np.int64)
    swa_rows = sw.shape[1] if sw is not None else 0
    cs = _f64(rope_cs)
    out = np.empty((T, H, D), dtype=np.float64)
    lse = np.empty((T, H), dtype=np.float64)
    rc = lib().oracle_hca_attn(_p(qq), _p(sm), _p(sk), ratio, float(softmax_scale),
                               _p(sw), _p(p0), swa_rows, window,
                               _p(_arr(q_seq, np.int32)), _p(_arr(q_pos, np.int64)),
                               _p(cs), rope_dim if cs is not None else 0,
                               T, B, N, H, D, _p(out), _p(lse))
    _check(rc, "hca_attn")
    return out, lse
