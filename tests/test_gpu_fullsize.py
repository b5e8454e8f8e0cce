"""Parity at the full sizes of the benchmark workloads, in the launch
configuration bench.py times (persistent kernel, one workgroup per CU):

- routing (ids, order, weights) against the fp64 oracle for every token,
  bit-exact except at near-ties within the derived logit bound;
- expert offsets and the permutation bit-exact against the oracle's
  permutation of the device's ids;
- the output rows of a sample of tokens, element by element, against the
  oracle computed for those tokens only (fed the device's ids and its
  intermediate codes and scales, which must lie in the derived windows).
  The sample covers every active expert (its first and last permuted row),
  every 16-row subtile position of its GEMM row tiles (ceil(rows / 144)
  tiles per expert, see expert_tiles), and the last row of every
  expert's last tile; the decode workload samples every token;
- the separate-kernel pipeline bitwise equal to the persistent kernel, the
  persistent kernel run on a workspace filled with NaN bytes first, so that
  a read of any intermediate or staging row before its writer has finished
  would show.
"""

import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from workloads import gen

from tests._helpers import check_output, check_routing

pytestmark = pytest.mark.gpu

FULL = ["dsv3_fp8", "dsv3_fp8xfp4", "decode_fp8_zipf", "mega_e1024_fp4_zipf"]
TILE_ROWS = 144          # most rows of a GEMM row tile for FP8 activations
SUBTILE = 16


@pytest.fixture(scope="module")
def L(gpu_lib):
    from moe_layer_router_amd import layer
    return layer


def expert_tiles(lo: int, hi: int):
    """The row tiles of an expert with permuted rows [lo, hi): g =
    ceil(n / 144) tiles, full ones and a remainder when the remainder has at
    most 64 rows, else g tiles of equal size to one row (the larger first)."""
    n = hi - lo
    gn = -(-n // TILE_ROWS)
    if gn > 1 and n - (gn - 1) * TILE_ROWS > 64:
        q, rem = divmod(n, gn)
    else:
        q, rem = TILE_ROWS, 0
    out = []
    for i in range(gn):
        r0 = i * q + min(i, rem)
        out.append((lo + r0, min(q + (i < rem), n - r0)))
    return out


def coverage_tokens(offsets: np.ndarray, perm: np.ndarray, k: int, T: int, min_tokens: int, seed: int = 0):
    """Tokens whose permuted rows cover, for every active expert, its first
    row and its last row (the last row of its last tile) and, in each of its
    tiles, one row at subtile position (e + 3 i) mod (the tile's subtiles) and
    lane (e % 16); the subtile positions are then each covered by many
    experts.  Topped up with random tokens to min_tokens."""
    rows = []
    E = offsets.size - 1
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        rows += [lo, hi - 1]
        for i, (r0, n) in enumerate(expert_tiles(lo, hi)):
            ps = (e + 3 * i) % (-(-n // SUBTILE))
            rows.append(r0 + SUBTILE * ps + min(e % SUBTILE, n - 1 - SUBTILE * ps))
    toks = set((perm[np.array(rows)] // k).tolist()) | {0, T - 1}
    rng = np.random.default_rng(seed)
    while len(toks) < min(min_tokens, T):
        toks.add(int(rng.integers(T)))
    return np.array(sorted(toks))


def subtile_positions(tokens: np.ndarray, offsets: np.ndarray, perm: np.ndarray, k: int):
    """The 16-row subtile positions (within their GEMM row tiles) of the
    permuted rows of the given tokens, and the positions any tile has."""
    row_of = np.empty_like(perm)
    row_of[perm] = np.arange(perm.size)
    rows = set(row_of[(tokens[:, None] * k + np.arange(k)).ravel()].tolist())
    got, have = set(), set()
    for e in range(offsets.size - 1):
        for r0, n in expert_tiles(int(offsets[e]), int(offsets[e + 1])):
            have |= set(range(-(-n // SUBTILE)))
            got |= {(r - r0) // SUBTILE for r in range(r0, r0 + n) if r in rows}
    return got, have


@pytest.mark.parametrize("name", FULL)
def test_full_size_workload(L, name):
    cfg = gen.CONFIGS[name]
    print(f"[fullsize] {name}: generating inputs", flush=True)
    raw = gen.make_inputs(cfg, seed=0, device="cuda")
    inp = L.pack_weights(raw)
    ws = L.Workspace("cuda")
    desc = L.desc_from_inputs(inp, cfg.k, "mega")
    ws.get(L.lib.moe_workspace_size(desc)).fill_(0xFF)       # NaN in every fp32 / BF16 / E4M3 slot
    torch.cuda.synchronize()
    print(f"[fullsize] {name}: persistent kernel on a NaN-filled workspace, then separate kernels", flush=True)
    out = L.forward(inp, cfg.k, mode="mega", workspace=ws)
    torch.cuda.synchronize()
    assert int(out["workspace"][:4].view(torch.int32).item()) == 0, "device watchdog fired"
    inter, isc = L.intermediate(out)
    inter, isc = inter.cpu().numpy(), isc.cpu().numpy()
    mega = {key: out[key].clone() for key in ("y", "topk_ids", "topk_weights", "perm", "expert_offsets")}
    sep = L.forward(inp, cfg.k, mode="separate")
    torch.cuda.synchronize()
    for key in mega:
        assert torch.equal(mega[key], sep[key]), f"{name}: separate kernels differ from the persistent kernel in {key}"
    assert torch.isfinite(mega["y"].float()).all()

    print(f"[fullsize] {name}: oracle routing", flush=True)
    spec = gen.spec_of(cfg)
    ov = gen.oracle_view(raw, lazy_weights=True)
    xh, logits, ids_ref, _ = O.route(spec, ov)
    lerr = O.logit_bound(spec, ov)
    ids = mega["topk_ids"].cpu().numpy().astype(np.int64)
    n_tie = check_routing(ids, mega["topk_weights"].cpu().numpy(), logits, ids_ref, cfg.k, lerr)
    counts, offsets, perm, _ = O.permutation(ids, cfg.E)
    assert np.array_equal(mega["expert_offsets"].cpu().numpy(), offsets)
    assert np.array_equal(mega["perm"].cpu().numpy(), perm)

    sample = coverage_tokens(offsets, perm, cfg.k, cfg.T, min_tokens=256)
    if cfg.T <= 256:
        sample = np.arange(cfg.T)
    got, have = subtile_positions(sample, offsets, perm, cfg.k)
    assert got == have, (got, have)
    print(f"[fullsize] {name}: oracle output of {sample.size} tokens ({n_tie} near-tie routings)", flush=True)
    ref = O.layer(spec, ov, ids=ids, tokens=sample, inter=inter, inter_scales=isc)
    y = mega["y"][torch.as_tensor(sample, device="cuda")].float().cpu().numpy()
    err = check_output(y, ref["y"], name)
    print(f"[fullsize] {name}: max element error {err[0]:.2e}, max token L2 {err[1]:.2e}", flush=True)
