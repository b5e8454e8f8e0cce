"""fp64 reference of the fused MoE layer forward pass.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The layer, as the pages describe it:

* 机器之心, "DeepSeek悄悄更新：Mega MoE、FP4 Indexer来了", section
  "Mega MoE 是什么？": each token is dispatched to experts, passes a linear
  map, a SwiGLU activation and a second linear map, and the expert results
  are combined back per token; Mega MoE fuses all of these into one kernel.
  The same section names FP8 x FP4 mixed precision.
* youleyou, "DeepSeek 模型更新解读 Tile Kernels 与 DeepEP V2 新特性", section
  "Tile Kernels": gating is top-k expert selection with scoring; MoE routing
  maps tokens to experts with fused expand/reduce and weight normalisation;
  quantisation is per token / per block / per channel FP8 or FP4 and can be
  fused with SwiGLU.  Section "性能表现" fixes the benchmark shape (8K tokens,
  hidden 7168, top-8, FP8 dispatch, BF16).

Readings taken where the pages are silent (each is repeated where it is used):

R1  Scoring is a softmax over router logits; the k selected weights are the
    softmax restricted to the selected experts (equal to the full softmax
    renormalised over the selection, since the full denominator cancels).
R2  Selection orders experts by logit descending, ties to the lower expert
    index, and ids are emitted in that order.  Selection is on logits (the
    softmax is monotone).
R3  The router reads the dequantised activations; router weights are BF16;
    an optional per-expert fp32 bias is added to the logits before both
    selection and the softmax.
R4  No capacity limit: every token goes to exactly k experts.
R5  gate|up weights are one [2I, H] matrix per expert (stored K-contiguous):
    rows 0..I-1 are the gate projection, rows I..2I-1 the up projection.
    SwiGLU(g, u) = SiLU(g) * u with SiLU(z) = z / (1 + exp(-z)).
R6  The intermediate activation is re-quantised to FP8 E4M3 per row and per
    128 channels: s = fl32(amax / 448), q = E4M3_RNE_saturating(a / s), and a
    block of zeros gets s = 1.  (For all-BF16 layers the intermediate is
    rounded to BF16 instead.)
R7  FP8 weights carry one fp32 scale per 128 x 128 block of the stored [N, K]
    matrix; FP4 weights carry one E8M0 scale per 32 consecutive K elements of
    each output row, two E2M1 values per byte with the even K index in the low
    nibble.  FP8 activations carry one fp32 scale per token per 128 channels.
R8  The permuted (expert-contiguous) row order sorts the flat index
    p = t*k + j by expert, stably, so rows of one expert are in ascending token
    order.
R10 FP8 re-quantisation near-ties: the device forms a with fp32 (and
    MFMA-internal) accumulation, so its a / s differs from the fp64 value
    by up to a small amount relative to the row's largest element.  Where
    the window a / s +- TIE_EPS straddles an E4M3 rounding boundary, every
    value the window rounds to is a correct result of the method.  The
    oracle then accepts a code supplied by the caller, but only at such
    positions and only inside the window.
R9  The combine is the weighted sum over j of w[t, j] * expert_output.  The
    reference result is the unrounded fp64 sum; the device sums in fp32 in
    ascending j and rounds the result to BF16.
"""

from dataclasses import dataclass

import numpy as np

from . import formats as F


@dataclass(frozen=True)
class Spec:
    T: int
    H: int
    E: int
    k: int
    I: int
    act: str = "fp8"      # "fp8" or "bf16"
    weight: str = "fp8"   # "fp8", "fp4" or "bf16"


# ------------------------------------------------------------------ decoding
def decode_activations(spec: Spec, x, x_scales=None) -> np.ndarray:
    """Dequantise the input activations to fp64 [T, H] (reading R7).

    FP8: value = E4M3(x[t, h]) * x_scales[t, h // 128].  BF16: exact."""
    if spec.act == "bf16":
        return F.bf16_decode(x)
    q = np.asarray(x, dtype=np.uint8)
    s = np.asarray(x_scales, dtype=np.float32).astype(np.float64)
    T, H = q.shape
    v = F.E4M3_TABLE[q].reshape(T, H // 128, 128) * s[:, :, None]
    return v.reshape(T, H)


def decode_weight(spec: Spec, w, w_scales=None) -> np.ndarray:
    """Dequantise one expert's stored weight matrix [N, K] to fp64 (reading R7)."""
    if spec.weight == "bf16":
        return F.bf16_decode(w)
    if spec.weight == "fp8":
        q = np.asarray(w, dtype=np.uint8)
        N, K = q.shape
        s = np.asarray(w_scales, dtype=np.float32).astype(np.float64)
        v = F.E4M3_TABLE[q].reshape(N // 128, 128, K // 128, 128)
        v = v * s[:, None, :, None]
        return v.reshape(N, K)
    if spec.weight == "fp4":
        vals = F.e2m1_unpack(w)                      # [N, K]
        N, K = vals.shape
        sc = F.e8m0_decode(w_scales)                 # [N, K // 32]
        return (vals.reshape(N, K // 32, 32) * sc[:, :, None]).reshape(N, K)
    raise ValueError(spec.weight)


# ------------------------------------------------------------------- routing
def router_logits(xhat: np.ndarray, router_w, router_bias=None) -> np.ndarray:
    """Gate scores l[t, e] = sum_h xhat[t, h] * Wr[e, h] + b[e] in fp64
    (Tile Kernels section, gating bullet; readings R1, R3)."""
    wr = F.bf16_decode(router_w)
    logits = xhat @ wr.T
    if router_bias is not None:
        logits = logits + np.asarray(router_bias, dtype=np.float32).astype(np.float64)[None, :]
    return logits


def topk_select(logits: np.ndarray, k: int) -> np.ndarray:
    """Top-k expert ids per token, logit descending, ties to the lower index
    (reading R2).  A stable sort of -logit keeps equal logits in index order."""
    order = np.argsort(-logits, axis=1, kind="stable")
    return order[:, :k].astype(np.int64)


def topk_weights(logits: np.ndarray, ids: np.ndarray) -> np.ndarray:
    """Softmax over the selected logits (reading R1): w_j = exp(l_j - m) / sum."""
    sel = np.take_along_axis(logits, ids, axis=1)
    m = sel.max(axis=1, keepdims=True)
    e = np.exp(sel - m)
    return e / e.sum(axis=1, keepdims=True)


# --------------------------------------------------------------- permutation
def permutation(ids: np.ndarray, E: int):
    """Dispatch as a local permutation, counting-sort formulation (reading R8;
    'token to expert mapping', Tile Kernels section, MoE routing bullet).

    Returns (counts[E], offsets[E+1], perm[T*k], row_of[T*k]) where perm[r]
    is the flat index p = t*k + j held by permuted row r and row_of is its
    inverse."""
    flat = ids.reshape(-1)
    counts = np.zeros(E, dtype=np.int64)
    for e in flat:
        counts[e] += 1
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    cursor = offsets[:-1].copy()
    perm = np.empty(flat.size, dtype=np.int64)
    for p, e in enumerate(flat):       # p ascending, so each segment is stable
        perm[cursor[e]] = p
        cursor[e] += 1
    row_of = np.empty_like(perm)
    row_of[perm] = np.arange(perm.size)
    return counts, offsets, perm, row_of


# ------------------------------------------------------------ expert compute
def silu(z: np.ndarray) -> np.ndarray:
    """SiLU(z) = z / (1 + exp(-z)) (reading R5)."""
    return z / (1.0 + np.exp(-z))


def swiglu(g: np.ndarray, u: np.ndarray) -> np.ndarray:
    """SwiGLU activation between the two linear maps (Mega MoE section; R5)."""
    return silu(g) * u


# Half-width of the window around a / s (whose largest magnitude is 448)
# within which the device's own pre-quantisation value may lie (reading
# R10): 448 * 2**-13, about five times the largest device-versus-fp64
# difference of a / s observed with fp32 accumulation.
TIE_EPS = F.E4M3_MAX * 2.0 ** -13


def tie_window(v: np.ndarray):
    """For each value of a / s, the smallest and largest E4M3 value that the
    round-to-nearest-even encoding of any value within TIE_EPS of it can
    give.  Where they differ, every E4M3 value between them (inclusive) is a
    correct re-quantisation result (reading R10)."""
    lo = F.E4M3_TABLE[F.e4m3_encode(v - TIE_EPS)]
    hi = F.E4M3_TABLE[F.e4m3_encode(v + TIE_EPS)]
    return lo != hi, lo, hi


def requant_fp8(a: np.ndarray, resolve=None):
    """Per-row, per-128-channel FP8 re-quantisation of the intermediate
    (Tile Kernels section, quantisation bullet, fused with SwiGLU; reading R6).

    resolve: optional uint8 [m, C] codes chosen by another implementation;
    they replace the oracle's code only where the tie window of a / s holds
    more than one value (reading R10), and must there lie in the window.

    Returns (codes uint8 [m, C], scales fp32-valued float64 [m, C/128],
    dequantised float64 [m, C])."""
    m, C = a.shape
    blocks = a.reshape(m, C // 128, 128)
    amax = np.abs(blocks).max(axis=2)
    s = F.f32_round(amax / F.E4M3_MAX)
    s = np.where(amax == 0.0, 1.0, s)
    v = blocks / s[:, :, None]
    codes = F.e4m3_encode(v)
    if resolve is not None:
        amb, lo, hi = tie_window(v)
        r = np.asarray(resolve, dtype=np.uint8).reshape(m, C // 128, 128)
        rv = F.E4M3_TABLE[r]
        valid = (rv >= lo) & (rv <= hi)
        if not np.all(valid[amb]):
            raise ValueError("a supplied code at a re-quantisation near-tie lies outside its tie window")
        codes = np.where(amb, r, codes)
    deq = F.E4M3_TABLE[codes] * s[:, :, None]
    return codes.reshape(m, C), s, deq.reshape(m, C)


def quantise_intermediate(spec: Spec, a: np.ndarray, resolve=None) -> np.ndarray:
    """The value GEMM2 consumes: FP8 re-quantised (R6, R10), or BF16-rounded
    for all-BF16 layers."""
    if spec.act == "bf16":
        return F.bf16_round(a)
    return requant_fp8(a, resolve)[2]


def expert_intermediate(spec: Spec, xrows: np.ndarray, w_gu: np.ndarray) -> np.ndarray:
    """Linear 1 (gate|up) and SwiGLU of one expert's rows, before requant."""
    G = xrows @ w_gu.T                        # [m, 2I]
    return swiglu(G[:, : spec.I], G[:, spec.I:])


def expert_ffn(spec: Spec, xrows: np.ndarray, w_gu: np.ndarray, w_d: np.ndarray, resolve=None) -> np.ndarray:
    """One expert on its gathered rows: linear 1 (gate|up), SwiGLU, requant,
    linear 2 (Mega MoE section: 线性变换 -> SwiGLU -> 线性变换).

    xrows [m, H] fp64; w_gu [2I, H] and w_d [H, I] dequantised fp64."""
    a = expert_intermediate(spec, xrows, w_gu)
    ahat = quantise_intermediate(spec, a, resolve)
    return ahat @ w_d.T                       # [m, H]


# ----------------------------------------------------------------- the layer
def route(spec: Spec, inputs: dict):
    """Gating for all tokens: (xhat, logits, ids, weights)."""
    xhat = decode_activations(spec, inputs["x"], inputs.get("x_scales"))
    logits = router_logits(xhat, inputs["router_w"], inputs.get("router_bias"))
    ids = topk_select(logits, spec.k)
    w = topk_weights(logits, ids)
    return xhat, logits, ids, w


def layer(spec: Spec, inputs: dict, ids=None, tokens=None, inter_codes=None) -> dict:
    """The whole layer in fp64.

    inputs: dict with x, x_scales, router_w, router_bias, w_gate_up,
    w_gate_up_scales, w_down, w_down_scales (numpy arrays, or objects whose
    [e] indexing yields one expert's numpy array, so that weights can be
    fetched one expert at a time).

    ids: optional [T, k] expert ids to use instead of the oracle's own
    selection (weights are still the softmax of the oracle's logits over
    those ids).  tokens: optional sorted array of token indices; when given,
    y is computed only for those tokens (routing and permutation are always
    computed for all tokens).

    Returns dict(y, logits, ids, weights, counts, offsets, perm, row_of),
    y being the unrounded fp64 output rows (of `tokens` when given)."""
    xhat, logits, sel, _ = route(spec, inputs)
    if ids is None:
        ids = sel
    ids = np.asarray(ids, dtype=np.int64)
    w = topk_weights(logits, ids)
    counts, offsets, perm, row_of = permutation(ids, spec.E)

    T, k = spec.T, spec.k
    tok_list = np.arange(T) if tokens is None else np.asarray(tokens, dtype=np.int64)
    out_row = -np.ones(T, dtype=np.int64)
    out_row[tok_list] = np.arange(tok_list.size)
    y = np.zeros((tok_list.size, spec.H), dtype=np.float64)

    for e in range(spec.E):
        rows = perm[offsets[e]: offsets[e + 1]]
        toks = rows // k
        keep = out_row[toks] >= 0
        if not np.any(keep):
            continue
        rows, toks = rows[keep], toks[keep]
        resolve = None
        if inter_codes is not None:
            resolve = np.asarray(inter_codes[np.arange(offsets[e], offsets[e + 1])[keep]])
        wgu_s = None if inputs.get("w_gate_up_scales") is None else np.asarray(inputs["w_gate_up_scales"][e])
        wd_s = None if inputs.get("w_down_scales") is None else np.asarray(inputs["w_down_scales"][e])
        w_gu = decode_weight(spec, np.asarray(inputs["w_gate_up"][e]), wgu_s)
        w_d = decode_weight(spec, np.asarray(inputs["w_down"][e]), wd_s)
        O = expert_ffn(spec, xhat[toks], w_gu, w_d, resolve)
        wt = w.reshape(-1)[rows]
        # Tokens are distinct within one expert, so these row updates never
        # collide; the sum over j is formed across the expert loop.
        y[out_row[toks]] += wt[:, None] * O
    return dict(y=y, logits=logits, ids=ids, weights=w, counts=counts,
                offsets=offsets, perm=perm, row_of=row_of, xhat=xhat)
