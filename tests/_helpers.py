"""Shared test helpers: the parity metric and device marshalling."""

import numpy as np

# Output tolerance (the layer's stated bound): every element satisfies
# |y - r| / max(|r|, rms of the token's reference row) <= 2e-2, r being the
# fp64 oracle fed the same quantised values; the per-token relative L2 error
# is held to the same bound as an extra check.
REL_TOL = 2e-2
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


def check_output(y: np.ndarray, r: np.ndarray, what: str = ""):
    assert np.all(np.isfinite(y)), f"{what}: non-finite output"
    re = rel_err(y, r)
    tl = token_rel_l2(y, r)
    t, c = np.unravel_index(re.argmax(), re.shape)
    assert re.max() <= REL_TOL, f"{what}: max element relative error {re.max():.3e} at (token row {t}, channel {c})"
    assert tl.max() <= REL_TOL, f"{what}: max token relative L2 error {tl.max():.3e} (token row {tl.argmax()})"
    return float(re.max()), float(tl.max())


def to_dev(inp: dict, device="cuda"):
    return {k: (None if v is None else v.to(device)) for k, v in inp.items()}


def near_tie_tokens(logits: np.ndarray, lerr: np.ndarray, k: int) -> np.ndarray:
    """Tokens whose top-k selection or order can differ between the oracle
    and a device within lerr of each logit: two of the k+1 largest fp64
    logits (adjacent in sorted order) lie closer than the sum of their
    bounds."""
    order = np.argsort(-logits, axis=1, kind="stable")[:, : min(k + 1, logits.shape[1])]
    l = np.take_along_axis(logits, order, axis=1)
    e = np.take_along_axis(lerr, order, axis=1)
    if l.shape[1] < 2:
        return np.zeros(logits.shape[0], dtype=bool)
    return (np.diff(-l, axis=1) < e[:, 1:] + e[:, :-1]).any(axis=1)


def check_routing(ids_gpu, w_gpu, logits_ref, ids_ref, k, lerr):
    """Bit-exact ids (set and order) except on near-tie tokens (lerr: the
    oracle's bound [T, E] on the device's logit error); those must still be a
    valid selection and order under the bound: k distinct experts, each
    selected logit no lower than any unselected one beyond their bounds,
    and the ids in descending logit order within their bounds.  The weights
    must be within W_TOL of the softmax of the oracle's logits over the
    device's ids and sum to one."""
    lerr = np.broadcast_to(np.asarray(lerr, dtype=np.float64), logits_ref.shape)
    same = (ids_gpu == ids_ref).all(axis=1)
    tie = near_tie_tokens(logits_ref, lerr, k)
    bad = ~same & ~tie
    assert not bad.any(), f"{bad.sum()} tokens routed differently without a near-tie, e.g. {np.flatnonzero(bad)[:5]}"
    E = logits_ref.shape[1]
    for t in np.flatnonzero(~same):
        sel = ids_gpu[t]
        assert len(set(sel.tolist())) == k and sel.min() >= 0 and sel.max() < E, f"token {t}: invalid ids {sel}"
        ls, es = logits_ref[t, sel], lerr[t, sel]
        rest = np.setdiff1d(np.arange(E), sel)
        if rest.size:
            lr, er = logits_ref[t, rest], lerr[t, rest]
            assert np.all(ls[:, None] + es[:, None] + er[None, :] >= lr[None, :]), \
                f"token {t}: a selected logit is below an unselected one beyond their bounds"
        assert np.all(ls[:-1] + es[:-1] + es[1:] >= ls[1:]), f"token {t}: ids not in descending logit order"
    sel = np.take_along_axis(logits_ref, ids_gpu, axis=1)
    e = np.exp(sel - sel.max(axis=1, keepdims=True))
    w_ref = e / e.sum(axis=1, keepdims=True)
    assert np.abs(w_gpu - w_ref).max() <= W_TOL
    assert np.abs(w_gpu.sum(axis=1) - 1).max() <= W_TOL
    return int((~same).sum())
