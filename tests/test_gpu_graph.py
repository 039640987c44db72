"""The decode step replayed from HIP graphs gives the eager step's results, replay after
replay, with eager work and synchronisations between the replays."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.mark.parametrize("fp4", [False, True])
def test_decode_step_graph_replays(fp4):
    import long_context_compressed_amd  # noqa: F401  (loads the library)
    from long_context_compressed_amd import pipeline

    print("decode step graph replays, mxfp4 keys" if fp4 else "decode step graph replays", flush=True)
    cfg = W.Config("graph_decode", 1007, "bf16", B=4, T=4, n=1 << 16, c=512, k=512, H=128)
    inp = W.decode_step_inputs(cfg, DEV, mxfp4=fp4)
    step = pipeline.DecodeStep(inp, cfg.k, cfg.window, cfg.rope_dim, cfg.scale)
    step()
    torch.cuda.synchronize()
    names = tuple(n for n in ("scores", "idx", "out", "lse", "out_h", "lse_h") if getattr(step, n) is not None)
    ref = {n: getattr(step, n).clone() for n in names}
    step.capture()
    for r in range(3):
        for n in names:  # clobber the outputs, so each replay has to write them again
            getattr(step, n).fill_(-7)
        x = torch.randn(1 << 20, device=DEV)  # eager work between replays
        (x * 2).sum().item()
        step()
        torch.cuda.synchronize()
        for n in names:
            a, b = getattr(step, n), ref[n]
            assert torch.equal(a, b), f"replay {r}: {n} differs from the eager step"
