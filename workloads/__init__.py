"""Seeded synthetic inputs for the CSA / HCA hot path.

This module is shared by the tests, the benchmark and the smoke check: it is the
only code that both the GPU library's callers and the CPU oracle's callers use.
It draws random tensors and encodes them (bf16 rounding, the MXFP4 block
encoding, RoPE angle tables); it computes none of the method's steps (no
compression, no index score, no selection, no attention).

Shapes follow the configuration table of "DeepSeek-V4 混合注意力：从压缩记忆到百万
上下文" (§2 table: 64/128 heads, indexer 64 x 128, top-k 512/1024, ratios 4 and
128, SWA 128) and the 1M-token arithmetic of its §3 (n/4 = 262,144 entries,
n/128 = 8,192 summaries).
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass, field

import numpy as np
import torch

# --------------------------------------------------------------------------------------
# seeds and raw draws
# --------------------------------------------------------------------------------------


def derive_seed(cfg_seed: int, name: str) -> int:
    """A 63-bit seed for tensor `name` of configuration `cfg_seed` (stable across runs)."""
    h = hashlib.sha256(f"{cfg_seed}:{name}".encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def normal(shape, cfg_seed: int, name: str, *, scale: float = 1.0, dtype=torch.float32,
           device="cpu", chunk_elems: int = 1 << 28) -> torch.Tensor:
    """N(0, scale^2) drawn in fp32 and rounded (RNE) to `dtype`.

    Large tensors are drawn in chunks of `chunk_elems` (each from its own seed) so
    that no fp32 copy of the whole tensor is ever held.
    """
    numel = int(np.prod(shape)) if len(shape) else 1
    out = torch.empty(numel, dtype=dtype, device=device)
    for c0 in range(0, numel, chunk_elems):
        c1 = min(numel, c0 + chunk_elems)
        g = _gen(derive_seed(cfg_seed, f"{name}#{c0 // chunk_elems}"), device)
        x = torch.randn(c1 - c0, generator=g, device=device, dtype=torch.float32)
        if scale != 1.0:
            x.mul_(scale)
        out[c0:c1] = x.to(dtype)
    return out.view(*shape)


def uniform(shape, cfg_seed: int, name: str, *, lo=0.0, hi=1.0, dtype=torch.float32,
            device="cpu") -> torch.Tensor:
    g = _gen(derive_seed(cfg_seed, name), device)
    x = torch.rand(*shape, generator=g, device=device, dtype=torch.float32)
    return (x * (hi - lo) + lo).to(dtype)


def randint(shape, cfg_seed: int, name: str, lo: int, hi: int, device="cpu") -> torch.Tensor:
    g = _gen(derive_seed(cfg_seed, name), device)
    return torch.randint(lo, hi, tuple(shape), generator=g, device=device, dtype=torch.int64)


def distinct_sample(n_pick: int, n_from: int, cfg_seed: int, name: str) -> np.ndarray:
    """`n_pick` distinct integers from [0, n_from), in random order (host)."""
    rng = np.random.Generator(np.random.Philox(derive_seed(cfg_seed, name)))
    return rng.choice(n_from, size=n_pick, replace=False).astype(np.int64)


# --------------------------------------------------------------------------------------
# encodings
# --------------------------------------------------------------------------------------

# Magnitudes of the 8 non-negative E2M1 codes (OCP Microscaling v1.0, FP4 E2M1).
_E2M1_GRID = torch.tensor([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=torch.float64)


def quantize_mxfp4(x: torch.Tensor):
    """Encode `x` [..., D] (D % 32 == 0) as MXFP4 blocks of 32 along the last dim.

    Follows the OCP Microscaling v1.0 conversion: the block scale is
    2^(floor(log2(amax)) - 2) stored as E8M0 (biased by 127), each element is x/scale
    rounded to the nearest E2M1 value (ties to the even code), saturating at +-6.
    Returns (codes uint8 [..., D/2] with the even element in the low nibble,
             scales uint8 [..., D/32]).
    """
    D = x.shape[-1]
    assert D % 32 == 0
    xb = x.to(torch.float64).reshape(-1, D // 32, 32)
    amax = xb.abs().amax(dim=-1)
    e = torch.where(amax > 0, torch.floor(torch.log2(torch.where(amax > 0, amax, 1.0))) - 2,
                    torch.full_like(amax, -127.0))
    e = e.clamp(-127, 127)
    scaled = xb / torch.pow(2.0, e).unsqueeze(-1)
    mag = scaled.abs().clamp(max=6.0)
    grid = _E2M1_GRID.to(x.device)
    # nearest grid point, ties to the even code index
    d = (mag.unsqueeze(-1) - grid).abs()
    best = d.min(dim=-1, keepdim=True).values
    cand = (d == best)
    idx = torch.arange(8, device=x.device)
    # among tied candidates prefer the even code index
    score = torch.where(cand, (idx % 2) * 16 + idx, torch.full_like(idx, 1000))
    code = score.argmin(dim=-1)
    sign = ((scaled < 0) & (code > 0)).to(torch.int64) << 3
    nib = (code | sign).to(torch.uint8).reshape(*x.shape[:-1], D)
    codes = (nib[..., 0::2] | (nib[..., 1::2] << 4)).contiguous()
    scales = (e + 127).to(torch.uint8).reshape(*x.shape[:-1], D // 32).contiguous()
    return codes, scales


def normal_mxfp4(shape, cfg_seed: int, name: str, device="cpu", chunk_rows: int = 1 << 17):
    """MXFP4 codes [..., D/2] and E8M0 scales [..., D/32] of an N(0,1) tensor of `shape`
    [..., D], drawn and encoded (quantize_mxfp4) in chunks of rows, each chunk from its own
    seed, so that no fp32 copy of the whole tensor is held.
    """
    D = shape[-1]
    rows = int(np.prod(shape[:-1])) if len(shape) > 1 else 1
    codes = torch.empty((rows, D // 2), dtype=torch.uint8, device=device)
    scales = torch.empty((rows, D // 32), dtype=torch.uint8, device=device)
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        g = _gen(derive_seed(cfg_seed, f"{name}#{r0 // chunk_rows}"), device)
        c, sc = quantize_mxfp4(torch.randn((r1 - r0, D), generator=g, device=device, dtype=torch.float32))
        codes[r0:r1] = c
        scales[r0:r1] = sc
    return codes.view(*shape[:-1], D // 2), scales.view(*shape[:-1], D // 32)


KV8_ROW_BYTES = 592  # 448 E4M3 codes + 64 bf16 + 14 E8M0 scales + 2 zero bytes


def random_kv8(rows_shape, cfg_seed: int, name: str, device="cpu", chunk_rows: int = 1 << 18):
    """Synthetic compressed KV rows already in the FP8 storage format [..., 592] bytes: each
    of the 448 codes a uniformly drawn finite E4M3 code (the two NaN codes 0x7F, 0xFF
    excluded), each of the 14 E8M0 block scales drawn from 2^-9 .. 2^-7 (so the decoded
    values lie within about +-3.5, like N(0,1) rows), the 64 RoPE dims N(0,1) rounded to
    bf16, two zero bytes. Drawn in chunks of rows, each from its own seed."""
    rows = int(np.prod(rows_shape)) if len(rows_shape) else 1
    out = torch.zeros((rows, KV8_ROW_BYTES), dtype=torch.uint8, device=device)
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        g = _gen(derive_seed(cfg_seed, f"{name}#{r0 // chunk_rows}"), device)
        m = r1 - r0
        code = torch.randint(0, 254, (m, 448), generator=g, device=device, dtype=torch.int32)
        code = code + (code >= 0x7F).to(torch.int32)  # skip 0x7F: values 0..253 -> 0..0x7E, 0x80..0xFE
        out[r0:r1, :448] = code.to(torch.uint8)
        rope = torch.randn((m, 64), generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)
        out[r0:r1, 448:576] = rope.view(torch.uint8).view(m, 128)
        out[r0:r1, 576:590] = torch.randint(118, 121, (m, 14), generator=g, device=device, dtype=torch.int32).to(
            torch.uint8)
    return out.view(*rows_shape, KV8_ROW_BYTES)


def rope_table(positions: torch.Tensor, rope_dim: int, base: float = 10000.0) -> torch.Tensor:
    """(cos, sin) angle table [T][rope_dim/2][2] fp32 for absolute `positions` [T].

    Pair p of the rotated block turns by pos * base^(-2p/rope_dim). The library and
    the oracle both take this table as an input; neither computes angles itself.
    """
    pos = positions.to(torch.float64).cpu()
    p = torch.arange(rope_dim // 2, dtype=torch.float64)
    inv = base ** (-2.0 * p / rope_dim)
    ang = pos[:, None] * inv[None, :]
    return torch.stack([torch.cos(ang), torch.sin(ang)], dim=-1).to(torch.float32)


# --------------------------------------------------------------------------------------
# configurations
# --------------------------------------------------------------------------------------

@dataclass(frozen=True)
class Config:
    name: str
    seed: int
    dtype: str            # "f32" | "bf16"
    B: int                # independent sequences
    T: int                # queries
    n: int                # context tokens before the queries (decode: query at t = n)
    c: int               # compressed KV width = attention head dim D
    H_I: int = 64
    D_I: int = 128
    k: int = 64
    H: int = 8
    window: int = 128
    rope_dim: int = 64
    ratio: int = 4
    idx_dtype: str = ""   # indexer operand encoding ("" = same as dtype, or "mxfp4")
    notes: dict = field(default_factory=dict)

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    @property
    def N(self) -> int:
        return self.n // self.ratio

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.c))


TINY = Config("tiny_prefill", 1001, "f32", B=1, T=1024, n=1024, c=128, k=64, H=8)
FLASH = Config("flash_decode_128k", 1002, "bf16", B=16, T=16, n=131072, c=512, k=512, H=64)
PRO = Config("pro_decode_1m", 1003, "bf16", B=4, T=4, n=1 << 20, c=512, k=1024, H=128)
PRO_PREFILL = Config("pro_prefill_chunk", 1004, "bf16", B=1, T=8192, n=65536, c=512, k=1024,
                     H=128, idx_dtype="mxfp4")
HCA = Config("hca_1m", 1005, "bf16", B=4, T=4, n=1 << 20, c=512, k=0, H=128, ratio=128)
HCA_PREFILL_T = 4096

CONFIGS = {c.name: c for c in (TINY, FLASH, PRO, PRO_PREFILL, HCA)}


def tiny_inputs(device="cpu", cfg: Config = TINY) -> dict:
    """All tensors of the tiny fp32 prefill (batch 1, 1024 tokens, hidden 256).

    C^a, C^b, Z^a, Z^b come from a synthetic hidden state H [n][256] ~ N(0,1)
    times four projection matrices [256][c] ~ 0.05 N(0,1), formed in fp64 and
    rounded to fp32 (the projection itself is upstream of the path).
    """
    s, n, c = cfg.seed, cfg.n, cfg.c
    hid = normal((n, 256), s, "hidden", dtype=torch.float64)
    proj = {}
    for nm in ("C_a", "C_b", "Z_a", "Z_b"):
        W = normal((256, c), s, f"W_{nm}", scale=0.05, dtype=torch.float64)
        proj[nm] = (hid @ W).to(torch.float32).reshape(1, n, c).to(device)
    T = cfg.T
    q_pos = torch.arange(T, dtype=torch.int64)
    inp = dict(proj)
    inp.update(
        q_I=normal((T, cfg.H_I, cfg.D_I), s, "q_I", device=device),
        w=uniform((T, cfg.H_I), s, "w", device=device),
        k_I=normal((1, cfg.N, cfg.H_I, cfg.D_I), s, "k_I", device=device),
        q=normal((T, cfg.H, cfg.c), s, "q", device=device),
        swa=normal((1, n, cfg.c), s, "swa", device=device),
        swa_pos0=torch.zeros(1, dtype=torch.int64, device=device),
        sink=normal((cfg.H,), s, "sink", device=device),
        q_seq=torch.zeros(T, dtype=torch.int32, device=device),
        q_pos=q_pos.to(device),
        rope_cs=rope_table(q_pos, cfg.rope_dim).to(device),
    )
    return inp


def decode_inputs(cfg: Config, device="cpu", with_index=True, shared_keys=False, mxfp4=False) -> dict:
    """Decode-step tensors for B independent sequences, one query each at t = n.

    Index keys, compressed KV, SWA rows, queries and sinks are N(0,1); the indexer
    head weights are N(0,1) for the Pro shape and 0.05 N(0,1) for the Flash shape
    (projection-derived). Tensors are bf16 except w, sink (fp32).
    mxfp4: the stored index keys are MXFP4 (k_I codes [B][N][64][64] + k_I_scale
    [B][N][64][4], encoded from N(0,1); a Hadamard rotation of iid N(0,1) vectors is again
    iid N(0,1), so these stand for rotated keys); q_I stays bf16 (the step encodes it).
    """
    s, B, N, D, dt = cfg.seed, cfg.B, cfg.N, cfg.c, cfg.torch_dtype
    n = cfg.n
    wscale = 0.05 if cfg.name.startswith("flash") else 1.0
    inp = dict(
        q=normal((cfg.T, cfg.H, D), s, "q", dtype=dt, device=device),
        kv=normal((B, N, D), s, "kv", dtype=dt, device=device),
        swa=normal((B, cfg.window, D), s, "swa", dtype=dt, device=device),
        swa_pos0=torch.full((B,), n - cfg.window + 1, dtype=torch.int64, device=device),
        sink=normal((cfg.H,), s, "sink", device=device),
        q_seq=torch.arange(cfg.T, dtype=torch.int32, device=device) % B,
        q_pos=torch.full((cfg.T,), n, dtype=torch.int64, device=device),
        rope_cs=rope_table(torch.full((cfg.T,), n), cfg.rope_dim).to(device),
    )
    if with_index:
        inp["q_I"] = normal((cfg.T, cfg.H_I, cfg.D_I), s, "q_I", dtype=dt, device=device)
        inp["w"] = normal((cfg.T, cfg.H_I), s, "w", scale=wscale, device=device)
        if shared_keys:  # one 128-dim key per entry for every head
            inp["k_I"] = normal((B, N, 1, cfg.D_I), s, "k_I_shared", dtype=dt, device=device)
        elif mxfp4:
            inp["k_I"], inp["k_I_scale"] = normal_mxfp4((B, N, cfg.H_I, cfg.D_I), s, "k_I_fp4", device=device)
        else:
            inp["k_I"] = normal((B, N, cfg.H_I, cfg.D_I), s, "k_I", dtype=dt, device=device)
    return inp


def decode_step_inputs(cfg: Config, device="cpu", shared_keys=False, mxfp4=False, kv8=False) -> dict:
    """Everything one decode step of a CSA layer plus an HCA layer reads, for B sequences.

    On top of decode_inputs: the block [n-4, n) that completes with the step (a- and
    b-branch contents/logits for the attention KV and for the index keys, and the carry
    block [n-8, n-4)), the HCA summaries [B][n/128][D] with their own sinks, and the
    ratio-128 block that completes the last summary. All N(0,1) bf16 (sinks fp32).
    shared_keys: the index keys are one 128-dim key per entry for all heads.
    mxfp4: the stored index keys are MXFP4 (see decode_inputs).
    kv8: the compressed KV rows and the HCA summaries are stored in the FP8 format
    (random_kv8: [B][N][592] and [B][n/128][592] bytes).
    """
    s, B, D, bf = cfg.seed, cfg.B, cfg.c, torch.bfloat16
    NH = cfg.n // 128
    inp = decode_inputs(cfg, device, shared_keys=shared_keys, mxfp4=mxfp4)
    if kv8:
        del inp["kv"]
        inp["kv"] = random_kv8((B, cfg.N), s, "kv8", device=device)
        inp["summ"] = random_kv8((B, NH), HCA.seed, "summ8", device=device)
    else:
        inp["summ"] = normal((B, NH, D), HCA.seed, "summ", dtype=bf, device=device)
    inp["sink_h"] = normal((cfg.H,), HCA.seed, "sink", device=device)
    inp["blk"] = {nm: normal((B, 4, D), s, "new_" + nm, dtype=bf, device=device) for nm in ("Ca", "Cb", "Za", "Zb")}
    inp["carry"] = {nm: normal((B, 4, D), s, "carry_" + nm, dtype=bf, device=device) for nm in ("C", "Z")}
    KW = cfg.D_I if shared_keys else cfg.H_I * cfg.D_I
    inp["iblk"] = {nm: normal((B, 4, KW), s, "inew_" + nm, dtype=bf, device=device) for nm in ("Ca", "Cb", "Za", "Zb")}
    inp["icarry"] = {nm: normal((B, 4, KW), s, "icarry_" + nm, dtype=bf, device=device) for nm in ("C", "Z")}
    inp["hblk"] = {nm: normal((B, 128, D), HCA.seed, "hnew_" + nm, dtype=bf, device=device) for nm in ("C", "Z")}
    return inp


def prefill_inputs(name: str, device="cpu") -> dict:
    """The tensors of one prefill chunk.

    "pro_prefill_chunk": 8,192 new tokens at positions 65,536..73,727 of one sequence.
      kv [1][18432][512] (rows 0..16,383 are the old cache, 16,384.. are rewritten by the
      compressor from Ca/Cb/Za/Zb [1][8192][512] and the carry of block 16,383);
      MXFP4 index operands q_I [8192][64][128] and k_I [1][18432][64][128] (encoded from
      N(0,1)); w [8192][64] N(0,1); q [8192][128][512]; SWA rows for positions
      65,409..73,727; sinks [128]; RoPE tables at each query's position.
    "hca_prefill_4k": the last 4,096 tokens of a 2^20 context. summaries [1][8192][512]
      (the last 32 rewritten from C/Z [1][4096][512]); q [4096][128][512]; SWA rows for
      positions 2^20 - 4,223 .. 2^20 - 1; sinks [128].
    """
    bf = torch.bfloat16
    if name == "pro_prefill_chunk":
        cfg = PRO_PREFILL
        T, n0, D, H, s = cfg.T, cfg.n, cfg.c, cfg.H, cfg.seed
        N = (n0 + T) // 4
        qc, qsc = quantize_mxfp4(normal((T, 64, 128), s, "q_I", device=device))
        kc, ksc = quantize_mxfp4(normal((1, N, 64, 128), s, "k_I", device=device))
        q_pos = torch.arange(n0, n0 + T, dtype=torch.int64, device=device)
        return dict(
            cfg=cfg, T=T, N=N, old=n0 // 4, D=D, H=H, k=cfg.k,
            kv=normal((1, N, D), s, "kv", dtype=bf, device=device),
            C={nm: normal((1, T, D), s, nm, dtype=bf, device=device) for nm in ("Ca", "Cb", "Za", "Zb")},
            carry={nm: normal((1, 4, D), s, "carry_" + nm, dtype=bf, device=device) for nm in ("C", "Z")},
            q_I=qc, q_I_scale=qsc, k_I=kc, k_I_scale=ksc,
            w=normal((T, 64), s, "w", device=device),
            q=normal((T, H, D), s, "q", dtype=bf, device=device),
            swa=normal((1, T + cfg.window - 1, D), s, "swa", dtype=bf, device=device),
            swa_pos0=torch.tensor([n0 - cfg.window + 1], dtype=torch.int64, device=device),
            sink=normal((H,), s, "sink", device=device),
            q_pos=q_pos,
            q_seq=torch.zeros(T, dtype=torch.int32, device=device),
            rope_cs=rope_table(q_pos.cpu(), cfg.rope_dim).to(device),
        )
    if name == "hca_prefill_4k":
        cfg = HCA
        T, n, D, H, s = HCA_PREFILL_T, cfg.n, cfg.c, cfg.H, cfg.seed
        NH = n // 128
        q_pos = torch.arange(n - T, n, dtype=torch.int64, device=device)
        return dict(
            cfg=cfg, T=T, NH=NH, D=D, H=H,
            summ=normal((1, NH, D), s, "summ", dtype=bf, device=device),
            C=normal((1, T, D), s, "C", dtype=bf, device=device),
            Z=normal((1, T, D), s, "Z", dtype=bf, device=device),
            q=normal((T, H, D), s, "q", dtype=bf, device=device),
            swa=normal((1, T + cfg.window - 1, D), s, "swa", dtype=bf, device=device),
            swa_pos0=torch.tensor([n - T - cfg.window + 1], dtype=torch.int64, device=device),
            sink=normal((H,), s, "sink", device=device),
            q_pos=q_pos,
            q_seq=torch.zeros(T, dtype=torch.int32, device=device),
            rope_cs=rope_table(q_pos.cpu(), cfg.rope_dim).to(device),
        )
    raise ValueError(f"unknown prefill workload {name!r}")
