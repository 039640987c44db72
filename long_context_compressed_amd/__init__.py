"""Python binding of libcsa.so, the gfx950 CSA / HCA attention hot path.

Argument marshalling only: every step runs in the library's HIP kernels. Tensors
are torch tensors on the GPU (their data_ptr() is passed as a device pointer) and
every call is enqueued on torch's current HIP stream. The library must be built
(`python long_context_compressed_amd/build.py`); importing a function without it
raises, there is no fallback.
"""
from __future__ import annotations

import ctypes as C
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcsa.so")

F32, BF16, MXFP4 = 0, 1, 2
STATUS = {0: "CSA_OK", 1: "CSA_EINVAL", 2: "CSA_EUNSUPPORTED", 3: "CSA_EWORKSPACE", 4: "CSA_EHIP"}
EXPORTS = ("csa_compress", "csa_index_scores", "csa_index_rescore", "csa_quantize_mxfp4", "csa_rmsnorm_rope",
           "csa_topk_workspace_bytes",
           "csa_topk", "csa_topk_ids",
           "csa_attn_workspace_bytes", "csa_sparse_attn", "hca_attn", "csa_status_str",
           "csa_last_error")


class CsaError(RuntimeError):
    def __init__(self, fn, status, detail):
        super().__init__(f"{fn}: {STATUS.get(status, status)}: {detail}")
        self.status = status


_lib = None


def lib() -> C.CDLL:
    """Load libcsa.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with long_context_compressed_amd/build.py")
        L = C.CDLL(LIB_PATH)
        P, i32, i64, f32, sz = C.c_void_p, C.c_int, C.c_int64, C.c_float, C.c_size_t
        L.csa_compress.argtypes = [P, P, P, P, P, P, P, i32, i64, i32, i32, i32, i32, P, i64, P]
        L.csa_index_scores.argtypes = [P, P, P, P, P, P, P, i32, i32, i64, i32, i32, i32, i32, i32, P, P]
        L.csa_quantize_mxfp4.argtypes = [P, i64, i32, i32, i32, P, P, i64, i64, P]
        L.csa_rmsnorm_rope.argtypes = [P, i32, i64, i32, P, f32, P, i32, i64, P, i32, P]
        L.csa_index_rescore.argtypes = [P, P, P, P, i32, P, P, i32, i32, i64, i32, i32, i32, i32, P, P]
        L.csa_topk_ids.argtypes = [P, P, i32, i64, i32, P, P, P, sz, P]
        L.csa_topk_workspace_bytes.argtypes = [i32, i64, i32]
        L.csa_topk_workspace_bytes.restype = sz
        L.csa_topk.argtypes = [P, i32, i64, i32, P, P, P, sz, P]
        L.csa_attn_workspace_bytes.argtypes = [i32, i32, i32, i64]
        L.csa_attn_workspace_bytes.restype = sz
        L.csa_sparse_attn.argtypes = [P, P, P, P, i32, f32, P, P, i32, i32, P, P, P, i32,
                                      i32, i32, i64, i32, i32, i32, P, P, P, sz, P]
        L.hca_attn.argtypes = [P, P, P, i32, f32, P, P, i32, i32, P, P, P, i32,
                               i32, i32, i64, i32, i32, i32, P, P, P, sz, P]
        for f in ("csa_compress", "csa_index_scores", "csa_index_rescore", "csa_quantize_mxfp4", "csa_rmsnorm_rope",
                  "csa_topk",
                  "csa_topk_ids", "csa_sparse_attn", "hca_attn"):
            getattr(L, f).restype = C.c_int
        L.csa_status_str.argtypes = [C.c_int]
        L.csa_status_str.restype = C.c_char_p
        L.csa_last_error.argtypes = []
        L.csa_last_error.restype = C.c_char_p
        _lib = L
    return _lib


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream if isinstance(stream, int) else stream.cuda_stream


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _check(fn, rc):
    if rc != 0:
        raise CsaError(fn, rc, lib().csa_last_error().decode())


# ---- the five calls ------------------------------------------------------------------

def compress(C_a, Z_a, C_b=None, Z_b=None, carry_C_b=None, carry_Z_b=None, logit_bias=None,
             ratio=4, overlap=1, out=None, stream=None):
    """csa_compress. C_a, Z_a (, C_b, Z_b): [B][n][c] -> out [B][n//ratio][c] (or a view
    with a larger batch stride into an existing cache)."""
    B, n, c = C_a.shape
    if out is None:
        out = torch.empty((B, n // ratio, c), dtype=C_a.dtype, device=C_a.device)
    bstride = out.stride(0) if out.dim() == 3 else 0
    rc = lib().csa_compress(_ptr(C_a), _ptr(C_b), _ptr(Z_a), _ptr(Z_b), _ptr(carry_C_b),
                            _ptr(carry_Z_b), _ptr(logit_bias), B, n, c, ratio, overlap,
                            _dt(C_a), _ptr(out), bstride, _stream(stream))
    _check("csa_compress", rc)
    return out


def index_scores(q_I, w, k_I, q_seq, q_pos, ratio=4, q_I_scale=None, k_I_scale=None,
                 mxfp4=False, scores=None, stream=None):
    """csa_index_scores -> scores [T][N] fp32. k_I is [B][N][k_heads][D_I] (k_heads = 64
    per-head keys, 1 shared key). For MXFP4 pass the uint8 code tensors q_I [T][64][64],
    k_I [B][N][64][64] and their E8M0 scale tensors."""
    T = q_I.shape[0]
    B, N, k_heads = k_I.shape[0], k_I.shape[1], k_I.shape[2]
    H_I = q_I.shape[1]
    D_I = q_I.shape[2] * (2 if mxfp4 else 1)
    dt = MXFP4 if mxfp4 else _dt(q_I)
    if scores is None:
        scores = torch.empty((T, N), dtype=torch.float32, device=q_I.device)
    rc = lib().csa_index_scores(_ptr(q_I), _ptr(q_I_scale), _ptr(w), _ptr(k_I), _ptr(k_I_scale),
                                _ptr(q_seq), _ptr(q_pos), T, B, N, H_I, D_I, k_heads, ratio, dt,
                                _ptr(scores), _stream(stream))
    _check("csa_index_scores", rc)
    return scores


def index_rescore(q_I, w, k_I, cand, q_seq, q_pos, ratio=4, scores=None, stream=None):
    """csa_index_rescore -> scores [T][M] fp32 of the candidate entries cand [T][M] (per-head
    keys k_I [B][N][64][128], fp32 or bf16)."""
    T, M = cand.shape
    B, N = k_I.shape[0], k_I.shape[1]
    if scores is None:
        scores = torch.empty((T, M), dtype=torch.float32, device=q_I.device)
    rc = lib().csa_index_rescore(_ptr(q_I), _ptr(w), _ptr(k_I), _ptr(cand), M, _ptr(q_seq), _ptr(q_pos), T, B, N,
                                 q_I.shape[1], q_I.shape[2], ratio, _dt(q_I), _ptr(scores), _stream(stream))
    _check("csa_index_rescore", rc)
    return scores


def quantize_mxfp4(x, hadamard=False, codes=None, scales=None, group_rows=0, group_stride=0, stream=None):
    """csa_quantize_mxfp4 -> (codes [..., D/2] uint8, scales [..., D/32] uint8) of x [..., D]
    (fp32 or bf16), after the Hadamard rotation when `hadamard`. With group_rows > 0, input
    row r goes to output row (r // group_rows) * group_stride + r % group_rows of the given
    codes / scales tensors (their data pointers are the base)."""
    D = x.shape[-1]
    rows = x.numel() // D if D else 0
    if codes is None:
        codes = torch.empty(x.shape[:-1] + (D // 2,), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty(x.shape[:-1] + (D // 32,), dtype=torch.uint8, device=x.device)
    rc = lib().csa_quantize_mxfp4(_ptr(x), rows, D, _dt(x), int(bool(hadamard)), _ptr(codes), _ptr(scales),
                                  group_rows, group_stride, _stream(stream))
    _check("csa_quantize_mxfp4", rc)
    return codes, scales


def rmsnorm_rope(x, g, eps, rope_cs=None, rope_group=1, out=None, out_dtype=None, stream=None):
    """csa_rmsnorm_rope -> out [..., D]: RMSNorm of each row of x (fp32 or bf16) with fp32
    gains g [D], then the last R dims rotated by rope_cs [ceil(rows / rope_group)][R/2][2]
    (or [..][R]) fp32 (cos, sin) pairs. out may be x (same dtype) for the in-place form."""
    D = x.shape[-1]
    rows = x.numel() // D if D else 0
    if out is None:
        out = torch.empty(x.shape, dtype=out_dtype or x.dtype, device=x.device)
    R = 0 if rope_cs is None else int(rope_cs.numel() // rope_cs.shape[0])
    rc = lib().csa_rmsnorm_rope(_ptr(x), _dt(x), rows, D, _ptr(g), float(eps), _ptr(rope_cs), R, int(rope_group),
                                _ptr(out), _dt(out), _stream(stream))
    _check("csa_rmsnorm_rope", rc)
    return out


def topk_workspace_bytes(T, N, k) -> int:
    return int(lib().csa_topk_workspace_bytes(T, N, k))


def topk(scores, k, idx=None, vals=None, workspace=None, with_vals=False, stream=None):
    """csa_topk -> (idx [T][k] int32 ascending, -1 padded; vals or None)."""
    T, N = scores.shape
    if idx is None:
        idx = torch.empty((T, k), dtype=torch.int32, device=scores.device)
    if vals is None and with_vals:
        vals = torch.empty((T, k), dtype=torch.float32, device=scores.device)
    need = topk_workspace_bytes(T, N, k)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=scores.device)
    wsb = workspace.numel() * workspace.element_size() if workspace is not None else 0
    rc = lib().csa_topk(_ptr(scores), T, N, k, _ptr(idx), _ptr(vals), _ptr(workspace), wsb,
                        _stream(stream))
    _check("csa_topk", rc)
    return idx, vals


def topk_ids(scores, ids, k, idx=None, vals=None, workspace=None, with_vals=False, stream=None):
    """csa_topk_ids -> (entry ids [T][k] int32 of the k best candidates, list order, -1 padded;
    vals or None)."""
    T, M = scores.shape
    if idx is None:
        idx = torch.empty((T, k), dtype=torch.int32, device=scores.device)
    if vals is None and with_vals:
        vals = torch.empty((T, k), dtype=torch.float32, device=scores.device)
    need = topk_workspace_bytes(T, M, k)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=scores.device)
    wsb = workspace.numel() * workspace.element_size() if workspace is not None else 0
    rc = lib().csa_topk_ids(_ptr(scores), _ptr(ids), T, M, k, _ptr(idx), _ptr(vals), _ptr(workspace), wsb,
                            _stream(stream))
    _check("csa_topk_ids", rc)
    return idx, vals


def attn_workspace_bytes(T, H, D, max_rows) -> int:
    return int(lib().csa_attn_workspace_bytes(T, H, D, max_rows))


def sparse_attn(q, kv, attn_sink, topk_idxs, softmax_scale, swa_kv, swa_pos0, window, q_seq, q_pos,
                rope_cs=None, rope_dim=0, out=None, lse=None, workspace=None, with_lse=True, stream=None):
    """csa_sparse_attn -> (out [T][H][D], lse [T][H] or None)."""
    T, H, D = q.shape
    B, N = kv.shape[0], kv.shape[1]
    k = topk_idxs.shape[1] if topk_idxs is not None else 0
    swa_rows = swa_kv.shape[1] if swa_kv is not None else 0
    if out is None:
        out = torch.empty_like(q)
    if lse is None and with_lse:
        lse = torch.empty((T, H), dtype=torch.float32, device=q.device)
    need = attn_workspace_bytes(T, H, D, k + (window if swa_kv is not None else 0))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    wsb = workspace.numel() * workspace.element_size() if workspace is not None else 0
    rc = lib().csa_sparse_attn(_ptr(q), _ptr(kv), _ptr(attn_sink), _ptr(topk_idxs), k, float(softmax_scale),
                               _ptr(swa_kv), _ptr(swa_pos0), swa_rows, window, _ptr(q_seq), _ptr(q_pos),
                               _ptr(rope_cs), rope_dim if rope_cs is not None else 0, T, B, N, H, D,
                               _dt(q), _ptr(out), _ptr(lse), _ptr(workspace), wsb, _stream(stream))
    _check("csa_sparse_attn", rc)
    return out, lse


def hca_attn(q, summ, attn_sink, ratio, softmax_scale, swa_kv, swa_pos0, window, q_seq, q_pos,
             rope_cs=None, rope_dim=0, out=None, lse=None, workspace=None, with_lse=True, stream=None):
    """hca_attn -> (out [T][H][D], lse [T][H] or None)."""
    T, H, D = q.shape
    B, N = summ.shape[0], summ.shape[1]
    swa_rows = swa_kv.shape[1] if swa_kv is not None else 0
    if out is None:
        out = torch.empty_like(q)
    if lse is None and with_lse:
        lse = torch.empty((T, H), dtype=torch.float32, device=q.device)
    need = attn_workspace_bytes(T, H, D, N + (window if swa_kv is not None else 0))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    wsb = workspace.numel() * workspace.element_size() if workspace is not None else 0
    rc = lib().hca_attn(_ptr(q), _ptr(summ), _ptr(attn_sink), ratio, float(softmax_scale),
                        _ptr(swa_kv), _ptr(swa_pos0), swa_rows, window, _ptr(q_seq), _ptr(q_pos),
                        _ptr(rope_cs), rope_dim if rope_cs is not None else 0, T, B, N, H, D,
                        _dt(q), _ptr(out), _ptr(lse), _ptr(workspace), wsb, _stream(stream))
    _check("hca_attn", rc)
    return out, lse
