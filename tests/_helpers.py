"""Shared test helpers: the parity metric and device marshalling."""

import numpy as np

# Output tolerance: the relative error of each token's output row,
# ||y_t - r_t|| / ||r_t||, is at most 2e-2 against the fp64 oracle fed the
# same quantised values.  Single elements are also bounded, relative to the
# row's RMS, by ELEM_TOL: an FP8 re-quantisation code that legitimately rounds
# the other way at a rounding midpoint moves a few elements by a few percent.
REL_TOL = 2e-2
ELEM_TOL = 1e-1
# Routing-weight tolerance (absolute) and the sum-to-one tolerance.
W_TOL = 1e-5


def rel_err(y: np.ndarray, r: np.ndarray) -> np.ndarray:
    """Elementwise |y - r| / max(|r|, rms of the token's reference row)."""
    rms = np.sqrt((r ** 2).mean(axis=1, keepdims=True))
    floor = np.maximum(rms, 1e-30)
    return np.abs(y - r) / np.maximum(np.abs(r), floor)


def token_rel_l2(y: np.ndarray, r: np.ndarray) -> np.ndarray:
    """Per-token relative L2 error ||y_t - r_t|| / ||r_t||."""
    return np.linalg.norm(y - r, axis=1) / np.maximum(np.linalg.norm(r, axis=1), 1e-30)


def elem_err(y: np.ndarray, r: np.ndarray) -> np.ndarray:
    """Elementwise |y - r| / rms of the token's reference row."""
    rms = np.sqrt((r ** 2).mean(axis=1, keepdims=True))
    return np.abs(y - r) / np.maximum(rms, 1e-30)


def check_output(y: np.ndarray, r: np.ndarray, what: str = ""):
    tl = token_rel_l2(y, r)
    ee = elem_err(y, r)
    assert tl.max() <= REL_TOL, f"{what}: max token relative L2 error {tl.max():.3e} (token {tl.argmax()})"
    assert ee.max() <= ELEM_TOL, f"{what}: max element error {ee.max():.3e} of the row RMS"
    return float(tl.max()), float(ee.max())


def to_dev(inp: dict, device="cuda"):
    return {k: (None if v is None else v.to(device)) for k, v in inp.items()}


def topk_gaps(logits: np.ndarray, k: int) -> np.ndarray:
    """Smallest gap between adjacent sorted logits among positions 1..k+1
    of each token (the places where a near-tie can change the selection or
    its order)."""
    l = -np.sort(-logits, axis=1)
    kk = min(k + 1, l.shape[1])
    if kk < 2:
        return np.full(l.shape[0], np.inf)
    return np.abs(np.diff(l[:, :kk], axis=1)).min(axis=1)


def check_routing(ids_gpu, w_gpu, logits_ref, ids_ref, k, delta):
    """Bit-exact ids except on tokens whose fp64 logits have a near-tie
    (gap < delta); those must still pick a valid top-k under the tie.  The
    weights must be within W_TOL of the softmax of the oracle's logits over
    the GPU's ids and sum to one."""
    same = (ids_gpu == ids_ref).all(axis=1)
    gaps = topk_gaps(logits_ref, k)
    bad = ~same & (gaps >= delta)
    assert not bad.any(), f"{bad.sum()} tokens routed differently without a near-tie, e.g. {np.flatnonzero(bad)[:5]}"
    for t in np.flatnonzero(~same):
        sel = logits_ref[t, ids_gpu[t]]
        kth = -np.sort(-logits_ref[t])[k - 1]
        assert len(set(ids_gpu[t].tolist())) == k
        assert sel.min() >= kth - delta, f"token {t}: selected logit below the k-th by more than delta"
    sel = np.take_along_axis(logits_ref, ids_gpu, axis=1)
    e = np.exp(sel - sel.max(axis=1, keepdims=True))
    w_ref = e / e.sum(axis=1, keepdims=True)
    assert np.abs(w_gpu - w_ref).max() <= W_TOL
    assert np.abs(w_gpu.sum(axis=1) - 1).max() <= W_TOL
    return int((~same).sum())
