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

F32, BF16, MXFP4, KV8 = 0, 1, 2, 3
KV8_ROW_BYTES = 592  # one 512-dim compressed row in the FP8 storage format
STATUS = {0: "CSA_OK", 1: "CSA_EINVAL", 2: "CSA_EUNSUPPORTED", 3: "CSA_EWORKSPACE", 4: "CSA_EHIP"}
EXPORTS = ("csa_compress", "csa_compress_batch", "csa_compress_hidden", "csa_quantize_kv8", "csa_out_proj_workspace_bytes", "csa_out_proj",
           "csa_index_scores", "csa_index_topk_workspace_bytes", "csa_index_topk", "csa_index_rescore", "csa_quantize_mxfp4", "csa_rmsnorm_rope",
           "csa_topk_workspace_bytes",
           "csa_topk", "csa_topk_noalloc", "csa_topk_ids",
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
        L.csa_compress_batch.argtypes = [P, i32, i32, P]
        L.csa_quantize_kv8.argtypes = [P, i64, i32, P, i64, i64, P]
        L.csa_compress_hidden.argtypes = [P, P, P, P, i32, i64, i64, i32, i32, i32, i32, P, i64, P]
        L.csa_out_proj_workspace_bytes.argtypes = [i32, i32, i32]
        L.csa_out_proj_workspace_bytes.restype = sz
        L.csa_out_proj.argtypes = [P, i32, i32, i32, i32, P, i32, P, i32, i32, P, P, sz, P]
        L.csa_index_scores.argtypes = [P, P, P, P, P, P, P, i32, i32, i64, i32, i32, i32, i32, i32, P, P]
        L.csa_index_topk_workspace_bytes.argtypes = [i32, i64, i32]
        L.csa_index_topk_workspace_bytes.restype = sz
        L.csa_index_topk.argtypes = [P, P, P, P, P, P, P, i32, i32, i64, i32, i32, i32, i32, P, P, P, sz, P]
        L.csa_quantize_mxfp4.argtypes = [P, i64, i32, i32, i32, P, P, i64, i64, P]
        L.csa_rmsnorm_rope.argtypes = [P, i32, i64, i32, P, f32, P, i32, i64, P, i32, P]
        L.csa_index_rescore.argtypes = [P, P, P, P, i32, P, P, i32, i32, i64, i32, i32, i32, i32, P, P]
        L.csa_topk_ids.argtypes = [P, P, i32, i64, i32, P, P, P, sz, P]
        L.csa_topk_workspace_bytes.argtypes = [i32, i64, i32]
        L.csa_topk_workspace_bytes.restype = sz
        L.csa_topk.argtypes = [P, i32, i64, i32, P, P, P, sz, P]
        L.csa_topk_noalloc.argtypes = [P, i32, i64, i32, P, P, P]
        L.csa_attn_workspace_bytes.argtypes = [i32, i32, i32, i64]
        L.csa_attn_workspace_bytes.restype = sz
        L.csa_sparse_attn.argtypes = [P, P, P, P, i32, f32, P, P, i32, i32, P, P, P, i32,
                                      i32, i32, i64, i32, i32, i32, P, P, P, sz, P]
        L.hca_attn.argtypes = [P, P, P, i32, f32, P, P, i32, i32, P, P, P, i32,
                               i32, i32, i64, i32, i32, i32, P, P, P, sz, P]
        for f in ("csa_compress", "csa_compress_batch", "csa_compress_hidden", "csa_quantize_kv8", "csa_out_proj", "csa_index_scores", "csa_index_topk", "csa_index_rescore", "csa_quantize_mxfp4", "csa_rmsnorm_rope",
                  "csa_topk", "csa_topk_noalloc",
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


def _require(cond, fn, msg):
    """Host-side shape checks the C ABI cannot make (it sees pointers, not extents):
    raised before anything is enqueued."""
    if not cond:
        raise ValueError(f"{fn}: {msg}")


def _rope_rows(rope_cs):
    return 0 if rope_cs is None else int(rope_cs.shape[0])


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


def quantize_kv8(x, out=None, group_rows=0, group_stride=0, stream=None):
    """csa_quantize_kv8: rows x [..., 512] (fp32 or bf16) -> uint8 [..., 592] in the FP8 KV
    storage format. With group_rows > 0, input row r goes to output row
    (r // group_rows) * group_stride + r % group_rows of `out` (its data pointer is the base)."""
    D = x.shape[-1]
    fn = "quantize_kv8"
    _require(D == 512 and x.is_contiguous(), fn, "x must be a contiguous [..][512] tensor")
    rows = x.numel() // D
    if out is None:
        out = torch.empty(x.shape[:-1] + (KV8_ROW_BYTES,), dtype=torch.uint8, device=x.device)
    _require(out.dtype == torch.uint8, fn, "out must be uint8")
    if group_rows == 0:
        _require(out.is_contiguous() and out.numel() >= rows * KV8_ROW_BYTES, fn, "out must hold rows x 592 bytes")
    rc = lib().csa_quantize_kv8(_ptr(x), rows, _dt(x), _ptr(out), group_rows, group_stride, _stream(stream))
    _check("csa_quantize_kv8", rc)
    return out


def _attn_dt(q, kv):
    """The call's dtype: q's, or CSA_KV8 when the compressed rows are uint8 FP8-format rows."""
    return KV8 if kv.dtype == torch.uint8 else _dt(q)


class _CompressJob(C.Structure):
    # the layout of csa_compress_job in include/csa.h
    _fields_ = [("C_a", C.c_void_p), ("C_b", C.c_void_p), ("Z_a", C.c_void_p), ("Z_b", C.c_void_p),
                ("carry_C_b", C.c_void_p), ("carry_Z_b", C.c_void_p), ("logit_bias", C.c_void_p),
                ("B", C.c_int), ("n", C.c_int64), ("c", C.c_int), ("ratio", C.c_int), ("overlap", C.c_int),
                ("out", C.c_void_p), ("out_bstride", C.c_int64)]


def compress_batch(jobs, stream=None):
    """csa_compress_batch: `jobs` is a list of dicts with the arguments of compress()
    (C_a, Z_a, C_b, Z_b, carry_C_b, carry_Z_b, logit_bias, ratio, overlap, out); every
    `out` must be given (a tensor or a strided view into a cache). One launch for all."""
    arr = (_CompressJob * max(1, len(jobs)))()
    dt = None
    for i, j in enumerate(jobs):
        Ca, out = j["C_a"], j["out"]
        B, n, c = Ca.shape
        ratio = j.get("ratio", 4)
        _require(out is not None and out.dim() == 3 and out.shape[0] == B and out.shape[2] == c
                 and out.shape[1] >= n // ratio and out.stride(2) == 1 and out.stride(1) == c,
                 "csa_compress_batch", f"job {i}: out must be [B][>= n/ratio][c] with rows of c contiguous")
        d = _dt(Ca)
        _require(dt is None or d == dt, "csa_compress_batch", "all jobs must share one dtype")
        dt = d
        arr[i] = _CompressJob(_ptr(Ca), _ptr(j.get("C_b")), _ptr(j["Z_a"]), _ptr(j.get("Z_b")),
                              _ptr(j.get("carry_C_b")), _ptr(j.get("carry_Z_b")), _ptr(j.get("logit_bias")), B, n, c,
                              ratio, j.get("overlap", 1 if ratio == 4 else 0), _ptr(out), out.stride(0))
    rc = lib().csa_compress_batch(C.cast(arr, C.c_void_p), len(jobs), BF16 if dt is None else dt, _stream(stream))
    _check("csa_compress_batch", rc)


def compress_hidden(hidden, W, carry_hidden=None, logit_bias=None, ratio=4, overlap=1, out=None,
                    out_dtype=None, stream=None):
    """csa_compress_hidden. hidden [B][n][d] bf16, W [(1+overlap)*2][c][d] bf16 (Wa_C, Wa_Z,
    Wb_C, Wb_Z) -> out [B][n//ratio][c] (or a view with a larger batch stride)."""
    B, n, d = hidden.shape
    npj, c, d2 = W.shape
    fn = "compress_hidden"
    _require(hidden.dtype == torch.bfloat16 and W.dtype == torch.bfloat16, fn, "hidden and W must be bf16")
    _require(hidden.is_contiguous() and W.is_contiguous(), fn, "hidden and W must be contiguous")
    _require(d2 == d and npj == 2 * (1 + overlap), fn, f"W must be [{2 * (1 + overlap)}][c][{d}]")
    _require(carry_hidden is None or (carry_hidden.is_contiguous() and tuple(carry_hidden.shape) == (B, 4, d)),
             fn, "carry_hidden must be a contiguous [B][4][d] tensor")
    if out is None:
        out = torch.empty((B, n // ratio, c), dtype=out_dtype or torch.bfloat16, device=hidden.device)
    _require(out.stride(-1) == 1 and out.shape[-1] == c, fn, "out rows must be contiguous [..][c]")
    bstride = out.stride(0) if out.dim() == 3 else 0
    rc = lib().csa_compress_hidden(_ptr(hidden), _ptr(carry_hidden), _ptr(W), _ptr(logit_bias), B, n, d, c, ratio,
                                   overlap, _dt(out), _ptr(out), bstride, _stream(stream))
    _check("csa_compress_hidden", rc)
    return out


def out_proj_workspace_bytes(T, G, d_g) -> int:
    return int(lib().csa_out_proj_workspace_bytes(T, G, d_g))


def out_proj(o, W_a, W_b=None, out=None, out_dtype=None, workspace=None, stream=None):
    """csa_out_proj. o [T][H][D] bf16, W_a [G][d_g][(H/G)*D] bf16, W_b [d_model][G*d_g] bf16 or
    None -> out [T][d_model] (or [T][G*d_g] without W_b)."""
    T, H, D = o.shape
    G, d_g, K1 = W_a.shape
    fn = "out_proj"
    _require(o.dtype == torch.bfloat16 and W_a.dtype == torch.bfloat16, fn, "o and W_a must be bf16")
    _require(o.is_contiguous() and W_a.is_contiguous(), fn, "o and W_a must be contiguous")
    _require(H % G == 0 and K1 == (H // G) * D, fn, f"W_a must be [G][d_g][{(H // max(G, 1)) * D}]")
    d_model = 0
    if W_b is not None:
        _require(W_b.dtype == torch.bfloat16 and W_b.is_contiguous() and W_b.shape[1] == G * d_g, fn,
                 f"W_b must be a contiguous bf16 [d_model][{G * d_g}] tensor")
        d_model = W_b.shape[0]
    width = d_model if W_b is not None else G * d_g
    if out is None:
        out = torch.empty((T, width), dtype=out_dtype or torch.bfloat16, device=o.device)
    _require(out.is_contiguous() and tuple(out.shape) == (T, width), fn, f"out must be a contiguous [T][{width}]")
    need = out_proj_workspace_bytes(T, G, d_g) if W_b is not None else 0
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=o.device)
    wsb = workspace.numel() * workspace.element_size() if workspace is not None else 0
    rc = lib().csa_out_proj(_ptr(o), T, H, D, G, _ptr(W_a), d_g, _ptr(W_b), d_model, _dt(out), _ptr(out),
                            _ptr(workspace), wsb, _stream(stream))
    _check("csa_out_proj", rc)
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


def index_topk_workspace_bytes(T, N, k) -> int:
    return int(lib().csa_index_topk_workspace_bytes(T, N, k))


def index_topk_workspace(T, N, k, device):
    """A workspace for csa_index_topk (None when the call needs none)."""
    need = index_topk_workspace_bytes(T, N, k)
    return torch.empty(need, dtype=torch.uint8, device=device) if need > 0 else None


def index_topk(q_I, w, k_I, q_seq, q_pos, k, q_I_scale, k_I_scale, ratio=4, idx=None, vals=None, workspace=None,
               with_vals=False, stream=None):
    """csa_index_topk -> (idx [T][k] int32 ascending, -1 padded; vals or None): the MXFP4
    scan fused with the top-k (uint8 codes q_I [T][64][64], k_I [B][N][64][64] and their
    E8M0 scales)."""
    T = q_I.shape[0]
    B, N = k_I.shape[0], k_I.shape[1]
    fn = "csa_index_topk"
    _require(q_I.dtype == torch.uint8 and k_I.dtype == torch.uint8, fn, "MXFP4 codes are uint8")
    _require(tuple(q_I.shape[1:]) == (64, 64) and tuple(k_I.shape[2:]) == (64, 64), fn,
             "codes must be [T][64][64] and [B][N][64][64]")
    _require(q_I_scale is not None and k_I_scale is not None, fn, "both scale tensors are needed")
    _require(tuple(q_I_scale.shape) == (T, 64, 4) and tuple(k_I_scale.shape) == (B, N, 64, 4), fn,
             "scales must be [T][64][4] and [B][N][64][4]")
    _require(tuple(w.shape) == (T, 64) and tuple(q_seq.shape) == (T,) and tuple(q_pos.shape) == (T,), fn,
             "w must be [T][64], q_seq and q_pos [T]")
    if idx is None:
        idx = torch.empty((T, k), dtype=torch.int32, device=q_I.device)
    if vals is None and with_vals:
        vals = torch.empty((T, k), dtype=torch.float32, device=q_I.device)
    if workspace is None:
        workspace = index_topk_workspace(T, N, k, q_I.device)
    wsb = workspace.numel() * workspace.element_size() if workspace is not None else 0
    rc = lib().csa_index_topk(_ptr(q_I), _ptr(q_I_scale), _ptr(w), _ptr(k_I), _ptr(k_I_scale), _ptr(q_seq),
                              _ptr(q_pos), T, B, N, 64, 128, ratio, k, _ptr(idx), _ptr(vals), _ptr(workspace), wsb,
                              _stream(stream))
    _check("csa_index_topk", rc)
    return idx, vals


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
    fn = "rmsnorm_rope"
    _require(x.is_contiguous() and g.is_contiguous(), fn, "x and g must be contiguous")
    _require(g.numel() == D, fn, f"g has {g.numel()} gains for rows of {D}")
    if rope_cs is not None:
        _require(rope_cs.is_contiguous() and rope_cs.dtype == torch.float32, fn, "rope_cs must be contiguous fp32")
        _require(int(rope_group) >= 1 and _rope_rows(rope_cs) * int(rope_group) >= rows, fn,
                 f"rope_cs has {_rope_rows(rope_cs)} angle rows; {rows} rows at rope_group={rope_group} need "
                 f"{-(-rows // max(1, int(rope_group)))}")
    if out is None:
        out = torch.empty(x.shape, dtype=out_dtype or x.dtype, device=x.device)
    _require(out.is_contiguous() and out.numel() == x.numel(), fn, "out must be contiguous and as large as x")
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


def topk_noalloc(scores, k, idx=None, vals=None, with_vals=False, stream=None):
    """csa_topk_noalloc -> (idx [T][k] int32 ascending, -1 padded; vals or None), using the
    library's own device scratch instead of a workspace (the output tensors, when not given,
    are still allocated here by torch)."""
    T, N = scores.shape
    if idx is None:
        idx = torch.empty((T, k), dtype=torch.int32, device=scores.device)
    if vals is None and with_vals:
        vals = torch.empty((T, k), dtype=torch.float32, device=scores.device)
    rc = lib().csa_topk_noalloc(_ptr(scores), T, N, k, _ptr(idx), _ptr(vals), _stream(stream))
    _check("csa_topk_noalloc", rc)
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


def _check_attn_args(fn, q, kv, swa_kv, q_seq, q_pos, rope_cs, rope_dim):
    T, H, D = q.shape
    _require(q.is_contiguous() and kv.is_contiguous(), fn, "q and the key/value rows must be contiguous")
    _require(kv.dim() == 3 and ((kv.dtype == q.dtype and kv.shape[2] == D) or
                                (kv.dtype == torch.uint8 and kv.shape[2] == KV8_ROW_BYTES and D == 512
                                 and q.dtype == torch.bfloat16)),
             fn, "kv must be [B][N][D] in q's dtype, or uint8 [B][N][592] FP8-format rows with bf16 q")
    _require(swa_kv is None or (swa_kv.is_contiguous() and swa_kv.shape[0] == kv.shape[0]
                                and swa_kv.shape[2] == D), fn, "swa_kv must be a contiguous [B][rows][D] tensor")
    _require(q_seq.numel() >= T and q_pos.numel() >= T, fn, "q_seq and q_pos need T entries")
    if rope_cs is not None:
        _require(rope_cs.is_contiguous() and rope_cs.dtype == torch.float32, fn, "rope_cs must be contiguous fp32")
        _require(_rope_rows(rope_cs) >= T, fn, f"rope_cs has {_rope_rows(rope_cs)} rows for {T} queries")
        _require(rope_cs.numel() // max(1, _rope_rows(rope_cs)) >= rope_dim, fn,
                 f"rope_cs rows hold fewer than rope_dim = {rope_dim} values")


def sparse_attn(q, kv, attn_sink, topk_idxs, softmax_scale, swa_kv, swa_pos0, window, q_seq, q_pos,
                rope_cs=None, rope_dim=0, out=None, lse=None, workspace=None, with_lse=True, stream=None):
    """csa_sparse_attn -> (out [T][H][D], lse [T][H] or None)."""
    T, H, D = q.shape
    B, N = kv.shape[0], kv.shape[1]
    k = topk_idxs.shape[1] if topk_idxs is not None else 0
    swa_rows = swa_kv.shape[1] if swa_kv is not None else 0
    _check_attn_args("sparse_attn", q, kv, swa_kv, q_seq, q_pos, rope_cs, rope_dim)
    _require(topk_idxs is None or (topk_idxs.is_contiguous() and topk_idxs.shape[0] == T
                                   and topk_idxs.dtype == torch.int32), "sparse_attn",
             "topk_idxs must be a contiguous int32 [T][k] tensor")
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
                               _attn_dt(q, kv), _ptr(out), _ptr(lse), _ptr(workspace), wsb, _stream(stream))
    _check("csa_sparse_attn", rc)
    return out, lse


def hca_attn(q, summ, attn_sink, ratio, softmax_scale, swa_kv, swa_pos0, window, q_seq, q_pos,
             rope_cs=None, rope_dim=0, out=None, lse=None, workspace=None, with_lse=True, stream=None):
    """hca_attn -> (out [T][H][D], lse [T][H] or None)."""
    T, H, D = q.shape
    B, N = summ.shape[0], summ.shape[1]
    swa_rows = swa_kv.shape[1] if swa_kv is not None else 0
    _check_attn_args("hca_attn", q, summ, swa_kv, q_seq, q_pos, rope_cs, rope_dim)
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
                        _attn_dt(q, summ), _ptr(out), _ptr(lse), _ptr(workspace), wsb, _stream(stream))
    _check("hca_attn", rc)
    return out, lse
