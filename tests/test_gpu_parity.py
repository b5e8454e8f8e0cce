"""Parity of the HIP path against the fp64 oracle, through the C ABI, at
sizes the oracle finishes in seconds (several tiles and ragged tails)."""

import numpy as np
import pytest
import torch

from oracle import formats as F
from oracle import moe_oracle as O
from workloads import gen
from tests._helpers import W_TOL, check_output, check_routing, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def L(gpu_lib):
    from moe_layer_router_amd import layer
    return layer


# ------------------------------------------------------------------- routing
@pytest.mark.parametrize("T,H,E,k,bias,dups", [
    (300, 1024, 40, 6, True, ((3, 17), (5, 6))),     # ragged T, E not a multiple of 64, ties
    (64, 256, 8, 2, False, ((0, 1),)),
    (129, 512, 1024, 16, True, ((10, 900),)),
    (77, 384, 256, 8, False, ()),
])
def test_router_exact_inputs_bit_exact(L, T, H, E, k, bias, dups):
    """On inputs where fp32 accumulation is exact in any order, logits, ids
    (with deliberate ties) and the permutation match the oracle bit for bit."""
    inp = gen.make_exact_router_inputs(T, H, E, seed=T + E, dup_pairs=dups, with_bias=bias)
    out = L.route(to_dev(inp), k, E)
    torch.cuda.synchronize()
    spec = O.Spec(T, H, E, k, 128)
    ov = gen.oracle_view(inp)
    xh, logits, ids, w = O.route(spec, ov)
    assert np.array_equal(out["logits"].cpu().numpy().astype(np.float64), logits)
    assert np.array_equal(out["topk_ids"].cpu().numpy(), ids)
    wg = out["topk_weights"].cpu().numpy()
    assert np.abs(wg - w).max() <= W_TOL
    assert np.abs(wg.sum(axis=1) - 1).max() <= W_TOL


def test_router_zero_weights_pick_first_k(L):
    inp = gen.make_exact_router_inputs(100, 256, 32, seed=1)
    inp["router_w"] = torch.zeros_like(inp["router_w"])
    out = L.route(to_dev(inp), 5, 32)
    ids = out["topk_ids"].cpu().numpy()
    assert (ids == np.arange(5)).all()
    assert np.array_equal(out["topk_weights"].cpu().numpy(), np.full((100, 5), 0.2, dtype=np.float32))


def test_router_bf16_activations_exact(L):
    inp = gen.make_exact_router_inputs(70, 512, 24, seed=2, dup_pairs=((1, 2),), with_bias=True)
    vals = torch.tensor(gen.oracle_view(inp)["x"]).view(torch.float8_e4m3fn).to(torch.float32)
    inp["x"] = vals.to(torch.bfloat16)
    inp["x_scales"] = None
    out = L.route(to_dev(inp), 4, 24)
    spec = O.Spec(70, 512, 24, 4, 128, "bf16", "bf16")
    xh, logits, ids, w = O.route(spec, gen.oracle_view(inp))
    assert np.array_equal(out["logits"].cpu().numpy().astype(np.float64), logits)
    assert np.array_equal(out["topk_ids"].cpu().numpy(), ids)


def test_router_gaussian_near_tie_rule(L):
    cfg = gen.LayerConfig("route_gauss", 512, 2048, 256, 8, 128, "fp8", "fp8")
    inp = gen.make_inputs(cfg, seed=3)
    out = L.route(to_dev(inp), 8, 256)
    spec = gen.spec_of(cfg)
    xh, logits, ids, w = O.route(spec, gen.oracle_view(inp))
    lg = out["logits"].cpu().numpy().astype(np.float64)
    ov = gen.oracle_view(inp)
    lerr = O.logit_bound(spec, ov)
    assert np.all(np.abs(lg - logits) <= lerr), "device logits outside the derived accumulation bound"
    check_routing(out["topk_ids"].cpu().numpy(), out["topk_weights"].cpu().numpy(), logits, ids, 8, lerr)


# --------------------------------------------------------------- permutation
def _perm_case(ids, E):
    return O.permutation(np.asarray(ids, dtype=np.int64), E)


@pytest.mark.parametrize("T,k,E,kind", [
    (1000, 8, 256, "random"),
    (300, 16, 1024, "random"),
    (513, 1, 4, "one_expert"),
    (700, 4, 64, "skewed"),
    (1, 1, 1, "random"),
    (257, 3, 5, "random"),
])
def test_permutation_bit_exact(L, T, k, E, kind):
    rng = np.random.default_rng(T * 7 + k)
    if kind == "one_expert":
        ids = np.full((T, k), 2)
    elif kind == "skewed":
        p = 1.0 / np.arange(1, E + 1) ** 1.5
        p /= p.sum()
        ids = np.stack([rng.choice(E, size=k, replace=False, p=p) for _ in range(T)])
    else:
        ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)])
    out = L.permute(torch.tensor(ids, dtype=torch.int32, device="cuda"), E)
    torch.cuda.synchronize()
    counts, offsets, perm, row_of = _perm_case(ids, E)
    assert np.array_equal(out["expert_offsets"].cpu().numpy(), offsets)
    assert np.array_equal(out["perm"].cpu().numpy(), perm)
    assert np.array_equal(out["row_of"].cpu().numpy(), row_of)


# --------------------------------------------------------------- whole layer
SMALL = [
    gen.LayerConfig("s_fp8", 300, 512, 16, 4, 256, "fp8", "fp8"),
    gen.LayerConfig("s_fp4", 300, 512, 16, 4, 256, "fp8", "fp4"),
    gen.LayerConfig("s_bf16", 200, 256, 8, 2, 256, "bf16", "bf16"),
    gen.CONFIGS["tiny_bf16"],
    gen.LayerConfig("s_multitile", 600, 384, 4, 2, 384, "fp8", "fp8"),     # >128 rows per expert, H % 256 != 0
    gen.LayerConfig("s_zipf_fp4", 256, 1024, 64, 8, 256, "fp8", "fp4", zipf=1.1),
    gen.LayerConfig("s_one_token", 1, 256, 4, 2, 128, "fp8", "fp8"),          # T = 1
    gen.LayerConfig("s_max_h", 40, 16384, 2, 1, 128, "fp8", "fp8"),           # largest H
    gen.LayerConfig("s_max_i", 40, 128, 2, 2, 16384, "fp8", "fp4"),           # largest I
    gen.LayerConfig("s_k_eq_e", 50, 256, 4, 4, 128, "bf16", "bf16"),          # every expert for every token
    gen.LayerConfig("s_bf16in_fp8", 300, 512, 16, 4, 256, "bf16", "fp8"),     # BF16 input quantised in the layer
    gen.LayerConfig("s_bf16in_fp4", 600, 384, 8, 2, 256, "bf16", "fp4"),      # (several 256-token blocks)
    # power-of-two scales for the layer's own quantisations: FP8 weights keep
    # the promotion; FP4 weights run the down GEMM (and, with BF16 input, the
    # gate|up GEMM too) with every scale in the matrix-core instruction
    gen.LayerConfig("s_fp8_pow2", 300, 512, 16, 4, 256, "fp8", "fp8", scales="pow2"),
    gen.LayerConfig("s_fp4_pow2", 600, 512, 16, 4, 384, "fp8", "fp4", scales="pow2"),
    gen.LayerConfig("s_bf16in_fp4_pow2", 300, 1024, 8, 2, 256, "bf16", "fp4", scales="pow2"),
    # per-channel FP8 weight scales (one per output row), applied after the K sum
    gen.LayerConfig("s_fp8_chan", 300, 512, 16, 4, 256, "fp8", "fp8", wscale="channel"),
    gen.LayerConfig("s_chan_multitile", 600, 384, 4, 2, 384, "fp8", "fp8", wscale="channel"),   # H % 256 != 0
    gen.LayerConfig("s_bf16in_fp8_chan", 300, 512, 16, 4, 256, "bf16", "fp8", wscale="channel", scales="pow2"),
]


def device_intermediate(L, out, weight):
    """The device's intermediate in the form the oracle takes: (E4M3 codes
    [T*k, I], fp32 scales [T*k, I/128]) for FP8 / FP4 experts, or (BF16 bit
    patterns, None) for all-BF16 layers."""
    inter, sc = L.intermediate(out)
    if weight != "bf16":
        return inter.cpu().numpy(), sc.cpu().numpy()
    return inter.cpu().view(torch.int16).numpy().view(np.uint16), None


def _layer_check(L, cfg, mode, inp=None, routing=None, seed=0, exact=False):
    if inp is None:
        inp = (gen.make_exact_layer_inputs if exact else gen.make_inputs)(cfg, seed=seed)
    out = L.forward(L.pack_weights(to_dev(inp)), cfg.k, mode=mode, inter_scale=cfg.scales,
                    routing=None if routing is None else tuple(torch.as_tensor(r).cuda() for r in routing))
    torch.cuda.synchronize()
    assert int(out["workspace"][:4].view(torch.int32).item()) == 0, "device watchdog fired"
    spec = gen.spec_of(cfg)
    ov = gen.oracle_view(inp)
    ids_gpu = out["topk_ids"].cpu().numpy().astype(np.int64)
    if routing is None:
        xh, logits, ids_ref, _ = O.route(spec, ov)
        lerr = O.logit_bound(spec, ov)
        check_routing(ids_gpu, out["topk_weights"].cpu().numpy(), logits, ids_ref, cfg.k, lerr)
    inter, isc = device_intermediate(L, out, cfg.weight)
    ref = O.layer(spec, ov, ids=ids_gpu, inter=inter, inter_scales=isc)
    y = out["y"].float().cpu().numpy()
    err = check_output(y, ref["y"], f"{cfg.name}/{mode}")
    assert np.array_equal(out["perm"].cpu().numpy(), ref["perm"])
    assert np.array_equal(out["expert_offsets"].cpu().numpy(), ref["offsets"])
    return out, err


@pytest.mark.parametrize("cfg", SMALL, ids=lambda c: c.name)
@pytest.mark.parametrize("mode", ["separate", "mega"])
def test_layer_matches_oracle(L, cfg, mode):
    _layer_check(L, cfg, mode)


EXACT = [
    gen.LayerConfig("x_fp8", 300, 1024, 16, 4, 256, "fp8", "fp8"),
    gen.LayerConfig("x_fp4", 300, 1024, 16, 4, 256, "fp8", "fp4"),
    gen.LayerConfig("x_bf16", 200, 512, 8, 2, 256, "bf16", "bf16"),
    gen.LayerConfig("x_fp8_chan", 300, 1024, 16, 4, 256, "fp8", "fp8", wscale="channel"),
]


@pytest.mark.parametrize("cfg", EXACT, ids=lambda c: c.name)
@pytest.mark.parametrize("mode", ["separate", "mega"])
def test_layer_exact_gemm_inputs(L, cfg, mode):
    """Inputs on which the gate|up GEMM is exact in fp32: routing bit-exact
    (zero logit bound), intermediate codes and scales equal to the oracle's
    except within a few fp32 units of a rounding midpoint."""
    _layer_check(L, cfg, mode, exact=True)


@pytest.mark.parametrize("cfg", SMALL[:3], ids=lambda c: c.name)
def test_mega_equals_separate_bitwise_and_deterministic(L, cfg):
    inp = L.pack_weights(to_dev(gen.make_inputs(cfg, seed=4)))
    a = L.forward(inp, cfg.k, mode="separate")
    b = L.forward(inp, cfg.k, mode="mega")
    c = L.forward(inp, cfg.k, mode="mega")
    torch.cuda.synchronize()
    for key in ("y", "topk_ids", "topk_weights", "perm", "expert_offsets"):
        assert torch.equal(a[key], b[key]), key
        assert torch.equal(b[key], c[key]), key


@pytest.mark.parametrize("mode", ["separate", "mega"])
def test_given_routing_skew_and_empty_experts(L, mode):
    """Routing fed in: every token to experts 5 and 0 (two hot experts, the
    rest empty), with uneven weights that are not the router's softmax."""
    cfg = gen.LayerConfig("given", 333, 512, 8, 2, 256, "fp8", "fp8")
    inp = gen.make_inputs(cfg, seed=5)
    ids = np.tile(np.array([[5, 0]], dtype=np.int32), (333, 1))
    w = np.tile(np.array([[0.75, 0.25]], dtype=np.float32), (333, 1))
    out = L.forward(L.pack_weights(to_dev(inp)), 2, mode=mode, routing=(torch.tensor(ids), torch.tensor(w)))
    torch.cuda.synchronize()
    spec = gen.spec_of(cfg)
    ov = gen.oracle_view(inp)
    counts, offsets, perm, _ = O.permutation(ids.astype(np.int64), 8)
    assert np.array_equal(out["perm"].cpu().numpy(), perm)
    assert np.array_equal(out["expert_offsets"].cpu().numpy(), offsets)
    inter, isc = device_intermediate(L, out, cfg.weight)
    xh = O.decode_activations(spec, ov["x"], ov["x_scales"])
    y = np.zeros((333, 512))
    for j, e in enumerate((5, 0)):
        rows = np.arange(offsets[e], offsets[e + 1])          # every token, ascending
        assert np.array_equal(perm[rows] // 2, np.arange(333))
        wgu = O.decode_weight(spec, ov["w_gate_up"][e], ov["w_gate_up_scales"][e])
        wd = O.decode_weight(spec, ov["w_down"][e], ov["w_down_scales"][e])
        a, ea = O.intermediate_bound(spec, xh, wgu, False)
        ahat = O.quantise_intermediate(spec, a, ea, inter[rows], isc[rows])
        y += w[:, j:j + 1].astype(np.float64) * (ahat @ wd.T)
    check_output(out["y"].float().cpu().numpy(), y, f"given/{mode}")


POW2_EXACT = gen.LayerConfig("x_fp8_pow2", 300, 1024, 16, 4, 256, "fp8", "fp8", scales="pow2")


@pytest.mark.parametrize("cfg,exact", [(SMALL[0], False), (SMALL[1], False), (SMALL[4], False), (SMALL[2], False),
                                       (EXACT[0], True), (EXACT[1], True), (EXACT[2], True),
                                       (SMALL[12], False), (POW2_EXACT, True), (SMALL[15], False), (SMALL[16], False),
                                       (EXACT[3], True)],
                         ids=["s_fp8", "s_fp4", "s_multitile", "s_bf16", "x_fp8", "x_fp4", "x_bf16", "s_fp8_pow2",
                              "x_fp8_pow2", "s_fp8_chan", "s_chan_multitile", "x_fp8_chan"])
def test_intermediate_matches_oracle(L, cfg, exact):
    """Gate|up GEMM, SwiGLU and the per-128 FP8 re-quantisation, row by row.
    The device's scales lie in the oracle's derived scale window and its E4M3
    codes (or BF16 values) equal the oracle's except where the derived bound
    of the device's a makes two values correct (reading R10), where they lie
    in that window.  On the exact-GEMM inputs the window is a few fp32 units
    of a wide, so codes and scales are bit-exact almost everywhere."""
    inp = (gen.make_exact_layer_inputs if exact else gen.make_inputs)(cfg, seed=6)
    out = L.forward(L.pack_weights(to_dev(inp)), cfg.k, mode="separate", inter_scale=cfg.scales)
    torch.cuda.synchronize()
    spec = gen.spec_of(cfg)
    ov = gen.oracle_view(inp)
    inter, isc = device_intermediate(L, out, cfg.weight)
    pw = cfg.scales == "pow2"
    perm = out["perm"].cpu().numpy()
    offs = out["expert_offsets"].cpu().numpy()
    xh = O.decode_activations(spec, ov["x"], ov["x_scales"])
    n_amb = n_tot = n_sdiff = n_blk = 0
    for e in range(cfg.E):
        rows = np.arange(offs[e], offs[e + 1])
        if rows.size == 0:
            continue
        toks = perm[rows] // cfg.k
        s1 = None if ov["w_gate_up_scales"] is None else ov["w_gate_up_scales"][e]
        pow2 = (cfg.act == "bf16" or O.powers_of_two(ov["x_scales"][toks])) and \
               (cfg.weight != "fp8" or O.powers_of_two(s1))
        if cfg.act == "fp8":
            assert pow2 == exact
        a, ea = O.intermediate_bound(spec, xh[toks], O.decode_weight(spec, ov["w_gate_up"][e], s1), pow2)
        if cfg.act == "bf16":
            lo, hi = O.bf16_window(a, ea)
            n_amb += int((lo != hi).sum())
            n_tot += a.size
            O.quantise_intermediate(spec, a, ea, inter[rows])      # raises outside the windows
            continue
        _, s_ref, _ = O.requant_fp8(a, pow2=pw)
        codes, s_dev, _ = O.requant_fp8(a, ea, resolve=inter[rows], resolve_scales=isc[rows], pow2=pw)   # raises
        _, lo, hi = O.requant_window(a, ea, s_dev, pw)
        n_amb += int((lo != hi).sum())
        n_tot += a.size
        n_sdiff += int((s_dev != s_ref).sum())
        n_blk += s_ref.size
    print(f"{cfg.name}: {n_amb} of {n_tot} positions in a rounding window, {n_sdiff} of {n_blk} scales "
          f"one fp32 step from the oracle's")
    # (a few ulps of SiLU error move fl32(amax/448) by an ulp in many blocks;
    # each such scale was checked against its window above)
    if exact:
        assert n_amb <= 1e-3 * n_tot


# ------------------------------------------------------------ weight layout
def _tiled_reference(w: np.ndarray, bs: int) -> np.ndarray:
    """The MFMA-tiled layout of moe_layer.h written out with numpy: w is the
    row-major [E][N][K-bytes] byte matrix; blocks (s, t), K step major, of
    BS/64 pieces of 1 KB, byte 16*l + j of piece p = row 16t + l%16, byte
    BS*s + 64p + 16*(l//16) + j."""
    E, N, KB = w.shape
    nsteps, npieces = KB // bs, bs // 64
    v = w.reshape(E, N // 16, 16, nsteps, npieces, 4, 16)      # e, t, row%16, s, p, l//16, j
    v = v.transpose(0, 3, 1, 4, 5, 2, 6)                        # e, s, t, p, l//16, row%16, j
    return np.ascontiguousarray(v).reshape(E, N, KB)


def _tiled_scales_reference(sc: np.ndarray, gate_up: bool) -> np.ndarray:
    """E8M0 scales [E][N][K/32] -> per (K step s, quad q) 256 bytes, byte
    4l + c = row 16t + l%16, group 4s + l//16, with t the quad's c-th tile:
    gate|up 2q + c (c < 2) or N/32 + 2q + c - 2, down 4q + c."""
    E, N, G = sc.shape
    S, nq = G // 4, N // 64
    q, c, l = np.arange(nq)[:, None, None], np.arange(4)[None, None, :], np.arange(64)[None, :, None]
    if gate_up:
        t = np.where(c < 2, 2 * q + c, N // 32 + 2 * q + c - 2)
    else:
        t = 4 * q + c
    rows = (t * 16 + l % 16)                                            # [q][l][c]
    out = np.empty((E, S, nq, 64, 4), dtype=sc.dtype)
    for s in range(S):
        out[:, s] = sc[:, rows, 4 * s + l // 16]
    return out.reshape(E, N, G)


@pytest.mark.parametrize("weight", ["fp8", "fp4", "bf16"])
def test_pack_weights_layout_bit_exact(L, weight):
    act = "bf16" if weight == "bf16" else "fp8"
    cfg = gen.LayerConfig("pack_" + weight, 8, 384, 3, 2, 256, act, weight)
    inp = to_dev(gen.make_inputs(cfg, seed=9))
    packed = L.pack_weights(inp)
    torch.cuda.synchronize()
    bs = {"fp8": 128, "fp4": 64, "bf16": 256}[weight]
    for w, sc in (("w_gate_up", "w_gate_up_scales"), ("w_down", "w_down_scales")):
        src = inp[w].cpu().contiguous().view(torch.uint8).numpy().reshape(cfg.E, inp[w].shape[1], -1)
        got = packed[w].cpu().contiguous().view(torch.uint8).numpy().reshape(src.shape)
        assert np.array_equal(got, _tiled_reference(src, bs)), w
        if weight == "fp4":
            s_src = inp[sc].cpu().numpy()
            assert np.array_equal(packed[sc].cpu().numpy(), _tiled_scales_reference(s_src, w == "w_gate_up")), sc
        elif weight == "fp8":
            assert packed[sc] is inp[sc]
