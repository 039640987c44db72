"""csa_topk_noalloc (the allocation-free top-k) against csa_topk with a caller workspace.

Both go through the C ABI on the same scores; the outputs are integer indices and the
scores they select, so they must agree bit for bit. Two calls in a row on the library's
shared device scratch, the second with a smaller input, check that nothing of the first
call's scratch contents leaks into the second. The oracle top-k rule is checked too.
"""
import numpy as np
import pytest
import torch

import workloads as W
from tests.helpers import check_topk_sets, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def csa():
    import long_context_compressed_amd as m
    m.lib()
    return m


def _scores(T, N, seed, masked_tail=0):
    s = W.normal((T, N), seed, "noalloc_scores", device=DEV)
    if masked_tail:
        s[:, N - masked_tail:] = -float("inf")
    return s


def _both(csa, s, k):
    ws = torch.empty(max(1, csa.topk_workspace_bytes(s.shape[0], s.shape[1], k)), dtype=torch.uint8, device=DEV)
    ref_idx, ref_val = csa.topk(s, k, workspace=ws, with_vals=True)
    idx, val = csa.topk_noalloc(s, k, with_vals=True)
    torch.cuda.synchronize()
    return ref_idx, ref_val, idx, val


def test_topk_noalloc_matches_workspace_call_twice(csa):
    # first call: the decode shape (4 rows of 262,144 scores, k = 1,024: the multi-level
    # path, 1 MiB of scratch); second call: smaller (3 rows of 100,000 with a masked tail)
    for T, N, k, seed, tail in ((4, 262144, 1024, 31, 0), (3, 100000, 512, 32, 1000)):
        print("topk_noalloc", T, N, k, flush=True)
        s = _scores(T, N, seed, tail)
        ref_idx, ref_val, idx, val = _both(csa, s, k)
        assert torch.equal(idx, ref_idx), f"T={T} N={N}: indices differ from csa_topk"
        assert torch.equal(val.view(torch.int32), ref_val.view(torch.int32)), f"T={T} N={N}: values differ"
        check_topk_sets(idx, to_np(s), k)


def test_topk_noalloc_single_chunk_and_limits(csa):
    # a row short enough for one chunk (no scratch use) and T = 0
    s = _scores(5, 3000, 33)
    ref_idx, ref_val, idx, val = _both(csa, s, 64)
    assert torch.equal(idx, ref_idx)
    csa.topk_noalloc(torch.empty((0, 100), device=DEV), 8)
    # a request beyond the fixed scratch is refused before anything is launched
    need = csa.topk_workspace_bytes(512, 262144, 1024)
    assert need > (16 << 20)
    big = torch.empty((512, 262144), dtype=torch.float32, device=DEV)
    with pytest.raises(csa.CsaError) as e:
        csa.topk_noalloc(big, 1024)
    assert e.value.status == 3 and "scratch" in str(e.value)
