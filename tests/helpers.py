"""Shared test helpers: tolerance checks written out in the tests' own terms."""
import numpy as np
import torch

# Correctness bars: fp32 outputs within 1e-4 and bf16 outputs within 2e-2 of the oracle,
# measured as max|gpu - ref| / max|ref| over the whole output tensor.
TOL_F32 = 1e-4
TOL_BF16 = 2e-2


def to_np(x):
    if isinstance(x, torch.Tensor):
        return x.detach().to("cpu", torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def rel_err(gpu, ref, mask=None):
    g, r = to_np(gpu), to_np(ref)
    if mask is not None:
        g, r = g[mask], r[mask]
    fin = np.isfinite(r)
    assert np.array_equal(np.isfinite(g), fin), "finite / -inf pattern differs"
    if not fin.any():
        return 0.0
    scale = np.abs(r[fin]).max()
    return float(np.abs(g[fin] - r[fin]).max() / (scale if scale > 0 else 1.0))


def assert_rel(gpu, ref, tol, what="", mask=None):
    e = rel_err(gpu, ref, mask)
    assert e <= tol, f"{what}: max-abs error {e:.3e} relative to max|ref| exceeds {tol:.1e}"
    return e


def check_topk_sets(gpu_idx, ref_scores, k, rel_tie=1e-5):
    """Top-k rule: every index in the symmetric difference of the GPU set and the oracle's
    top-k set has an oracle score within rel_tie of the k-th score; the GPU set holds
    exactly min(k, #finite) distinct finite entries, the rest -1."""
    import oracle
    ref_idx, ref_vals = oracle.topk(ref_scores, k)
    gi = to_np(gpu_idx).astype(np.int64)
    s = np.asarray(ref_scores, dtype=np.float64)
    T = s.shape[0]
    n_diff = 0
    for t in range(T):
        nfin = int(np.isfinite(s[t]).sum())
        m = min(k, nfin)
        g = gi[t]
        gv = g[g >= 0]
        assert len(gv) == m and len(np.unique(gv)) == m, f"row {t}: {len(gv)} valid of {m}"
        assert np.all(g[m:] == -1), f"row {t}: padding"
        assert np.all(np.isfinite(s[t, gv])), f"row {t}: selected a masked entry"
        r = set(ref_idx[t, :m].tolist())
        diff = r.symmetric_difference(set(gv.tolist()))
        if diff:
            n_diff += 1
            tau = ref_vals[t, m - 1]
            for i in diff:
                assert abs(s[t, i] - tau) <= rel_tie * abs(tau), f"row {t}: index {i} is not a near-tie"
    return n_diff
