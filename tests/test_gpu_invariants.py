"""Invariants of the attention calls checked on the GPU alone ("DeepSeek-V4 混合注意力" §4.2,
§5, §6): each compares the GPU path with itself under a transformation the definition fixes,
on the row-split (few queries) and the many-query kernels.

- sink-softened probabilities: with every row equal to one vector v, o = (sum p) v and
  sum p = 1 - e^(sink - lse) < 1 (§6: the sink only adds e^sink to the denominator);
- the dense special case: sparse attention whose top-k list holds every visible entry
  equals hca_attn at ratio 4 over the same rows (§4.2 vs §5);
- index handling: permuting a query's top-k list leaves o unchanged to rounding, and a
  -1 in the list is the same as leaving that slot out;
- RoPE: an identity (cos 1, sin 0) table is the same as no RoPE, bit for bit.
(The working-set sizes by lse and bitwise determinism are in test_gpu_parity.py.)
"""
import numpy as np
import pytest
import torch

import workloads as W
from tests.helpers import TOL_BF16, assert_rel
from tests.test_gpu_parity import _attn_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"
D = 512
SCALE = 1.0 / np.sqrt(D)

# (T, H, B, N, k, positions): few queries (rows split over workgroups, merged) and many
# queries (one workgroup per 128 heads of a query)
SHAPES = [
    (3, 128, 3, 2000, 300, [8000, 8001, 600]),
    (256, 128, 1, 600, 64, None),
]


@pytest.fixture(scope="module")
def csa():
    import long_context_compressed_amd as m
    m.lib()
    return m


def say(*a):
    print(*a, flush=True)


def _pos(T, pos):
    return pos or [int(p) for p in np.linspace(300, 2300, T).astype(np.int64)]


@pytest.mark.parametrize("T,H,B,N,k,pos", SHAPES)
def test_sink_softened_mass(csa, T, H, B, N, k, pos):
    say("sink mass", T, H)
    q, kv, swa, sink, q_seq, q_pos, idx, p0, _ = _attn_inputs(61 + T, T, H, D, B, N, k, 130, torch.bfloat16,
                                                               _pos(T, pos), with_rope=False)
    v = (1.0 + 0.5 * W.uniform((D,), 61, "v", device=DEV)).to(torch.bfloat16)
    kv = v.view(1, 1, D).expand(B, N, D).contiguous()
    swa = v.view(1, 1, D).expand(B, swa.shape[1], D).contiguous()
    sink = sink * 2.0  # sinks from about -6 to 6: masses from nearly 1 to well below
    out, lse = csa.sparse_attn(q, kv, sink, idx, SCALE, swa, p0, 128, q_seq, q_pos)
    torch.cuda.synchronize()
    vf = v.float()
    mass = (out.float() @ vf) / (vf @ vf)                              # [T][H]
    expect = 1.0 - torch.exp(sink.view(1, H) - lse)                   # 1 - e^(sink - lse)
    assert torch.all(expect < 1.0)
    assert_rel(mass, expect, TOL_BF16, "sum of the sink-softened probabilities")
    # o is that mass times v in every dim (every row is v)
    assert_rel(out.float(), mass.unsqueeze(-1) * vf, TOL_BF16, "o = (sum p) v")


@pytest.mark.parametrize("T,H,B,N,pos", [
    (3, 128, 3, 700, [4 * 600 + 1, 4 * 700, 130]),   # few queries: both calls split their rows
    (256, 128, 1, 520, None),                         # many queries
])
def test_dense_special_case(csa, T, H, B, N, pos):
    """A top-k list of every visible entry (in index order, -1 after them) makes the sparse
    call the dense one: it equals hca_attn(ratio = 4) over the same rows and SWA."""
    say("sparse(k >= visible) == hca(ratio 4)", T, H)
    pos = pos or [int(p) for p in np.linspace(40, 4 * N, T).astype(np.int64)]
    q, kv, swa, sink, q_seq, q_pos, _, p0, rope = _attn_inputs(71 + T, T, H, D, B, N, 0, 130, torch.bfloat16, pos)
    nvis = [min(N, p // 4) for p in pos]
    k = max(nvis) + 7
    idx = torch.full((T, k), -1, dtype=torch.int32)
    for t, nv in enumerate(nvis):
        idx[t, :nv] = torch.arange(nv, dtype=torch.int32)
    idx = idx.to(DEV)
    a, la = csa.sparse_attn(q, kv, sink, idx, SCALE, swa, p0, 128, q_seq, q_pos, rope, 64)
    b, lb = csa.hca_attn(q, kv, sink, 4, SCALE, swa, p0, 128, q_seq, q_pos, rope, 64)
    torch.cuda.synchronize()
    assert_rel(a, b, TOL_BF16, "sparse with every visible entry vs hca ratio 4")
    assert_rel(la, lb, 2e-3, "lse")


@pytest.mark.parametrize("T,H,B,N,k,pos", SHAPES)
def test_index_permutation_and_padding(csa, T, H, B, N, k, pos):
    say("index permutation / -1", T, H)
    q, kv, swa, sink, q_seq, q_pos, idx, p0, rope = _attn_inputs(81 + T, T, H, D, B, N, k, 130, torch.bfloat16,
                                                                 _pos(T, pos), bad_idx=False)
    o, lo = csa.sparse_attn(q, kv, sink, idx, SCALE, swa, p0, 128, q_seq, q_pos, rope, 64)
    g = torch.Generator().manual_seed(81)
    perm = torch.stack([torch.randperm(k, generator=g) for _ in range(T)]).to(DEV)
    op, lp = csa.sparse_attn(q, kv, sink, torch.gather(idx, 1, perm).contiguous(), SCALE, swa, p0, 128, q_seq,
                             q_pos, rope, 64)
    # slot j of every query set to -1, against the list with slot j left out
    j = k // 3
    drop = idx.clone()
    drop[:, j] = -1
    cut = torch.cat([idx[:, :j], idx[:, j + 1:]], dim=1).contiguous()
    od, ld = csa.sparse_attn(q, kv, sink, drop, SCALE, swa, p0, 128, q_seq, q_pos, rope, 64)
    oc, lc = csa.sparse_attn(q, kv, sink, cut, SCALE, swa, p0, 128, q_seq, q_pos, rope, 64)
    torch.cuda.synchronize()
    # "to rounding": another row order moves the softmax's reference maximum and the rows'
    # split boundaries, so P and the partial sums round to bf16 differently
    assert_rel(op, o, TOL_BF16, "permuted top-k list")
    assert_rel(lp, lo, 2e-3, "permuted top-k list: lse")
    assert_rel(od, oc, TOL_BF16, "-1 slot vs slot left out")
    assert_rel(ld, lc, 2e-3, "-1 slot vs slot left out: lse")
    assert not torch.equal(od, o), "dropping a row changed nothing"


@pytest.mark.parametrize("T,H,B,N,k,pos", SHAPES)
@pytest.mark.parametrize("mode", ["sparse", "hca"])
def test_identity_rope_table(csa, mode, T, H, B, N, k, pos):
    say("identity RoPE", mode, T, H)
    pos = _pos(T, pos)
    q, kv, swa, sink, q_seq, q_pos, idx, p0, _ = _attn_inputs(91 + T, T, H, D, B, N, k, 130, torch.bfloat16, pos,
                                                               with_rope=False)
    ident = torch.zeros((T, 32, 2), dtype=torch.float32, device=DEV)
    ident[..., 0] = 1.0
    if mode == "sparse":
        a, la = csa.sparse_attn(q, kv, sink, idx, SCALE, swa, p0, 128, q_seq, q_pos, ident, 64)
        b, lb = csa.sparse_attn(q, kv, sink, idx, SCALE, swa, p0, 128, q_seq, q_pos)
    else:
        a, la = csa.hca_attn(q, kv, sink, 4, SCALE, swa, p0, 128, q_seq, q_pos, ident, 64)
        b, lb = csa.hca_attn(q, kv, sink, 4, SCALE, swa, p0, 128, q_seq, q_pos)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(la, lb)
