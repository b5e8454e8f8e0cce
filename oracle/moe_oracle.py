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
    rounded to BF16 instead.)  The power-of-two variant of the quantisation
    options takes s = the smallest power of two >= amax / 448 (as R12), an
    E8M0 number that scaled matrix-core instructions apply exactly.
R7  FP8 weights carry one fp32 scale per 128 x 128 block of the stored [N, K]
    matrix; FP4 weights carry one E8M0 scale per 32 consecutive K elements of
    each output row, two E2M1 values per byte with the even K index in the low
    nibble.  FP8 activations carry one fp32 scale per token per 128 channels.
R8  The permuted (expert-contiguous) row order sorts the flat index
    p = t*k + j by expert, stably, so rows of one expert are in ascending token
    order.
R10 Where the device's result is one rounding step away from the oracle's
    (an FP8 code of the intermediate, its fp32 scale, a BF16 intermediate,
    or the order of two router logits), both are results of the method if
    the device's inputs to that rounding lie within a bound derived here
    from the arithmetic: fp32 accumulation (every product of a dot product
    passes through at most n additions, each erring by at most one unit in
    the last place of its fp32 result, u = 2**-23, so the sum is off by at
    most gamma_n * sum|x*w| with gamma_n = n*u/(1-n*u)), zero where every
    partial sum is exactly representable in fp32, plus the documented
    accuracy of the matrix core and of the exponential and reciprocal the
    SiLU uses (one unit in the last place each).  The oracle accepts a
    caller-supplied value only where that bound makes more than one value
    correct, and only inside that range.
R11 a / s is formed on the device as a times the correctly rounded fp32
    reciprocal of s; those two roundings (2**-24 relative each) are part of
    the R10 bound.  The oracle's own code is the E4M3 rounding of the exact
    a / s.
R12 Input quantisation (the per-token FP8 quantisation of the Tile Kernels
    section's quantisation bullet, in front of the router): per token and
    128 channels, amax = max |x|; s = fl32(amax / 448) (fp32 division), a
    zero block gets s = 1; or, for power-of-two scales, s = 2**e with e the
    smallest integer such that 448 * 2**e >= amax, clamped to [-127, 127]
    (an E8M0-representable scale).  Codes are E4M3_RNE_sat(x * fl32(1 / s))
    with the product rounded to fp32: the rounding decision is taken in the
    kernel's precision, so codes are bit-exact.  When the layer quantises its
    input, the router reads the unquantised BF16 activations and the experts
    the quantised ones.
R13 Per-channel weight scales (the per-channel option of the quantisation
    bullet): an FP8 weight matrix [N, K] may carry one fp32 scale per output
    channel (row n, all of K) instead of one per 128 x 128 block: value =
    E4M3(q[n, k]) * s[n].  Only FP8 weights take it (FP4 weights keep the
    E8M0-per-32 scaling of their format); activations keep their per-token
    per-128 scales.
R14 The backward pass (the training workload of the pages: trainable
    layers in the Tile Kernels section's model-layer bullet) is the exact
    gradient of the layer with the routing held fixed (the selection is
    piecewise constant) and every rounding of the forward pass (the
    intermediate's re-quantisation or BF16 rounding) passed straight through
    as the identity: y[t] = sum_j w[t, j] * SwiGLU(x[t] W_gu[e]^T) W_d[e]^T
    with e = ids[t, j] and w the softmax of the selected logits
    l = x_r W_r^T + b.  The router's gradient reaches x through the logits
    (x_r is the router's input, R3).
R15 E5M6 quantisation (the third format of the quantisation bullet, a
    conversion target: no matrix-core instruction takes it, and every E5M6
    value is exactly a BF16 and an fp32 number): the format of
    formats.py; per token and 128 channels as R12 with 65024 in place of
    448: s = fl32(amax / 65024) (a zero block gets s = 1), codes =
    E5M6_RNE_sat(fl32(x * fl32(1 / s))); or s = 2**e with e the smallest
    integer such that 65024 * 2**e >= amax (clamped to [-127, 127]) and codes
    of the exact x / s.  Dequantisation gives fl32(value(code) * s).
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
    act: str = "fp8"      # "fp8" (quantised input), "bf16" (all-BF16 layer) or
                          # "bf16_fp8" (BF16 input quantised to FP8 in the layer, R12)
    weight: str = "fp8"   # "fp8", "fp4" or "bf16"
    scales: str = "f32"   # scales of the layer's own FP8 quantisations: "f32" or "pow2"
    wscale: str = "block"  # FP8 weight scales: "block" (128 x 128) or "channel" (R13)


# ------------------------------------------------------------------ decoding
def decode_activations(spec: Spec, x, x_scales=None) -> np.ndarray:
    """The activations the expert GEMMs read, in fp64 [T, H] (readings R7,
    R12).

    FP8: value = E4M3(x[t, h]) * x_scales[t, h // 128].  BF16: exact.
    BF16 quantised in the layer: the per-token FP8 quantisation of x,
    dequantised."""
    if spec.act == "bf16":
        return F.bf16_decode(x)
    if spec.act == "bf16_fp8":
        codes, s = quantise_tokens_fp8(F.bf16_decode(x), spec.scales == "pow2")
        T, H = codes.shape
        return (F.E4M3_TABLE[codes].reshape(T, H // 128, 128) * s[:, :, None]).reshape(T, H)
    q = np.asarray(x, dtype=np.uint8)
    s = np.asarray(x_scales, dtype=np.float32).astype(np.float64)
    T, H = q.shape
    v = F.E4M3_TABLE[q].reshape(T, H // 128, 128) * s[:, :, None]
    return v.reshape(T, H)


def decode_weight(spec: Spec, w, w_scales=None) -> np.ndarray:
    """Dequantise one expert's stored weight matrix [N, K] to fp64 (readings
    R7, R13)."""
    if spec.weight == "bf16":
        return F.bf16_decode(w)
    if spec.weight == "fp8" and spec.wscale == "channel":
        q = np.asarray(w, dtype=np.uint8)
        s = np.asarray(w_scales, dtype=np.float32).astype(np.float64)     # [N]
        if s.shape != (q.shape[0],):
            raise ValueError(f"per-channel scales must have shape ({q.shape[0]},), got {s.shape}")
        return F.E4M3_TABLE[q] * s[:, None]
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


# --------------------------------------------------- input quantisation (R12)
def pow2_scale_exponent(amax: np.ndarray, fmax: float = F.E4M3_MAX) -> np.ndarray:
    """Smallest integer e with fmax * 2**e >= amax (amax > 0; fmax the
    format's largest finite value, 448 for E4M3), clamped to [-127, 127]; 0
    where amax == 0 (scale 1).  Exact: fmax * 2**e is exact in fp64 for every
    e in range."""
    amax = np.asarray(amax, dtype=np.float64)
    e = np.ceil(np.log2(np.where(amax > 0, amax, 1.0) / fmax)).astype(np.int64)
    # correct the floating-point log2 by one step either way, exactly
    e = np.where(np.ldexp(fmax, e - 1) >= amax, e - 1, e)
    e = np.where(np.ldexp(fmax, e) < amax, e + 1, e)
    e = np.clip(e, -127, 127)
    return np.where(amax > 0, e, 0)


def quantise_tokens_fp8(x: np.ndarray, pow2: bool = False):
    """Per-token, per-128-channel FP8 quantisation of activations (reading
    R12).  x: [T, H] values exactly representable in fp32 (BF16 or fp32
    inputs).  Returns (codes uint8 [T, H], scales float64 [T, H/128]
    (fp32 values; powers of two when pow2)).

    Steps in the kernel's precision (fp32, IEEE round to nearest even):
    s = fl32(amax / 448), inv = fl32(1 / s), v = fl32(x * inv), then E4M3
    round-to-nearest-even with saturation.  With pow2, s = 2**e and v = x / s
    is exact."""
    x = np.asarray(x, dtype=np.float64)
    T, H = x.shape
    b = x.reshape(T, H // 128, 128)
    if not np.all(np.isfinite(b)) or not np.array_equal(b, b.astype(np.float32).astype(np.float64)):
        raise ValueError("quantise_tokens_fp8 takes finite values representable in fp32")
    amax = np.abs(b).max(axis=2)
    if pow2:
        s = np.ldexp(1.0, pow2_scale_exponent(amax))
        v = b / s[:, :, None]                                   # exact (power-of-two scaling)
    else:
        a32 = amax.astype(np.float32)
        s32 = np.where(a32 > 0, a32 / np.float32(F.E4M3_MAX), np.float32(1.0)).astype(np.float32)
        inv = (np.float32(1.0) / s32).astype(np.float32)
        v = (b.astype(np.float32) * inv[:, :, None]).astype(np.float32).astype(np.float64)
        s = s32.astype(np.float64)
    codes = F.e4m3_encode(v)
    return codes.reshape(T, H), s


# ---------------------------------------------------- E5M6 quantisation (R15)
def quantise_tokens_e5m6(x: np.ndarray, pow2: bool = False):
    """Per-token, per-128-channel E5M6 quantisation (reading R15).  x: [T, H]
    values exactly representable in fp32.  Returns (codes uint16 [T, H] of
    12 bits, scales float64 [T, H/128] (fp32 values)).  The same steps as
    quantise_tokens_fp8 with the E5M6 maximum: s = fl32(amax / 65024),
    inv = fl32(1 / s), v = fl32(x * inv), E5M6 round-to-nearest-even with
    saturation; with pow2, s = 2**e and v = x / s exactly."""
    x = np.asarray(x, dtype=np.float64)
    T, H = x.shape
    b = x.reshape(T, H // 128, 128)
    if not np.all(np.isfinite(b)) or not np.array_equal(b, b.astype(np.float32).astype(np.float64)):
        raise ValueError("quantise_tokens_e5m6 takes finite values representable in fp32")
    amax = np.abs(b).max(axis=2)
    if pow2:
        s = np.ldexp(1.0, pow2_scale_exponent(amax, F.E5M6_MAX))
        v = b / s[:, :, None]                                   # exact (power-of-two scaling)
    else:
        a32 = amax.astype(np.float32)
        s32 = np.where(a32 > 0, a32 / np.float32(F.E5M6_MAX), np.float32(1.0)).astype(np.float32)
        inv = (np.float32(1.0) / s32).astype(np.float32)
        v = (b.astype(np.float32) * inv[:, :, None]).astype(np.float32).astype(np.float64)
        s = s32.astype(np.float64)
    return F.e5m6_encode(v).reshape(T, H), s


def dequantise_e5m6(codes: np.ndarray, s: np.ndarray) -> np.ndarray:
    """fl32(value(code) * s) per element (reading R15): codes [T, H], scales
    [T, H/128] -> fp32 values as float64."""
    codes = np.asarray(codes)
    T, H = codes.shape
    v = F.e5m6_decode(codes).reshape(T, H // 128, 128)
    out = (v.astype(np.float32) * np.asarray(s, dtype=np.float32)[:, :, None]).astype(np.float32)
    return out.reshape(T, H).astype(np.float64)


# --------------------------------------------- device deviation bounds (R10)
# One unit in the last place of an fp32 result, relative: the bound taken for
# every floating-point operation of the device (matrix-core additions, vector
# additions and multiplies, the exponential and the reciprocal).  Correctly
# rounded operations err by half of it.
U1 = 2.0 ** -23


def gamma(n) -> float:
    """gamma_n = n*u / (1 - n*u): the relative bound of n chained roundings
    of at most u each (the classic bound for recursive summation)."""
    return n * U1 / (1.0 - n * U1)


def _lowest_bit_exponent(v: np.ndarray) -> int:
    """Exponent of the lowest set bit over the nonzero values of v (all
    finite): every value of v is an integer multiple of 2**result."""
    v = np.asarray(v, dtype=np.float64).ravel()
    v = v[v != 0]
    if v.size == 0:
        return 1 << 20
    m, e = np.frexp(v)                                    # v = m * 2**e, 0.5 <= |m| < 1
    M = np.abs(np.ldexp(m, 53)).astype(np.int64)          # integer significand
    tz = np.zeros(M.shape, dtype=np.int64)
    rest = M.copy()
    while True:
        even = (rest & 1) == 0
        if not even.any():
            break
        tz += even
        rest = np.where(even, rest >> 1, rest)
    return int((e - 53 + tz).min())


def fp32_sums_exact(xrows: np.ndarray, w: np.ndarray, scales_pow2: bool) -> np.ndarray:
    """Whether every partial sum of the dot products xrows @ w.T is exactly
    representable in fp32, whatever the order and grouping of the additions:
    all products are integer multiples of 2**(qx + qw) (the lowest set bits of
    the two operands), and with power-of-two block scales every partial sum is
    a multiple of that bounded by sum|x*w| < 2**24 * 2**(qx + qw).  Returns a
    boolean [m, N] (all False unless scales_pow2)."""
    if not scales_pow2:
        return np.zeros((xrows.shape[0], w.shape[0]), dtype=bool)
    q = _lowest_bit_exponent(xrows) + _lowest_bit_exponent(w)
    S = np.abs(xrows) @ np.abs(w).T
    return S < np.ldexp(1.0, 24 + q)


def additions_per_product(spec: Spec, K: int) -> int:
    """How many roundings one product of a length-K dot product of the expert
    GEMMs can pass through on the device.  FP8 activations: up to 128 additions
    inside one block-scaled MFMA (one 128-wide K block), the fp32 product of
    the two block scales and the promotion FMA, then one addition per K block.
    BF16: up to 32 additions inside one MFMA and one per chained MFMA."""
    if spec.act == "bf16":
        return 32 + K // 32 + 1
    return 128 + 2 + K // 128


def accumulation_bound(spec: Spec, xrows: np.ndarray, w: np.ndarray, scales_pow2: bool) -> np.ndarray:
    """Absolute bound on |device - exact| of each element of xrows @ w.T
    (reading R10): gamma_n * sum_k |x_k * w_k|, and 0 where every partial sum
    is exact in fp32."""
    S = np.abs(xrows) @ np.abs(w).T
    e = gamma(additions_per_product(spec, xrows.shape[1])) * S
    return np.where(fp32_sums_exact(xrows, w, scales_pow2), 0.0, e)


# |SiLU'(z)| = |sigma(z) (1 + z (1 - sigma(z)))| is at most 1.0999 (at z ~ 2.4).
SILU_LIPSCHITZ = 1.1


def swiglu_bound(g, u, eg, eu):
    """Absolute bound on |device - exact| of a = SiLU(g) * u when the device's
    g and u are within eg and eu of the exact ones (reading R10).

    The device forms exp(-g) as 2**(-g * log2 e) (one rounded multiply by the
    rounded constant: relative argument error <= 2 * 2**-24 = U1, hence a
    relative error |g| * U1 of the exponential; the exponential instruction
    itself <= U1), adds 1 (<= U1/2), takes the reciprocal (<= U1) and
    multiplies by g and by u (<= U1/2 each): relative error <= (|g| + 4) U1 of
    its own result.  Below g = -80 the exponential overflows and the device's
    a is 0, which is within |a| of the exact value."""
    g, u, eg, eu = (np.asarray(v, dtype=np.float64) for v in (g, u, eg, eu))
    sg = silu(g)
    dsilu = SILU_LIPSCHITZ * eg
    prop = dsilu * (np.abs(u) + eu) + np.abs(sg) * eu        # from the inputs' error
    mag = (np.abs(sg) + dsilu) * (np.abs(u) + eu)             # bound on |device a|
    rnd = mag * (np.abs(g) + eg + 4.0) * U1 * (1 + 1e-6)      # the device's own evaluation
    ea = prop + rnd
    return np.where(g - eg < -80.0, np.maximum(ea, 2.0 * mag + 1e-300), ea)


def intermediate_bound(spec: Spec, xrows: np.ndarray, w_gu: np.ndarray, scales_pow2: bool):
    """(a, ea): the exact SwiGLU intermediate of one expert's rows and the
    bound on the device's deviation from it (R10)."""
    G = xrows @ w_gu.T
    eG = accumulation_bound(spec, xrows, w_gu, scales_pow2)
    g, u = G[:, : spec.I], G[:, spec.I:]
    return swiglu(g, u), swiglu_bound(g, u, eG[:, : spec.I], eG[:, spec.I:])


def requant_window(a: np.ndarray, ea: np.ndarray, s: np.ndarray, pow2: bool = False):
    """For the block scales s [m, C/128], the exact a / s [m, C/128, 128] and
    the smallest and largest E4M3 values that the device may produce there:
    the device's pre-rounding value lies within ea / s of a / s, plus the two
    roundings of the reciprocal multiply (R11; none for power-of-two scales,
    where the scaling is exact)."""
    m, C = a.shape
    A = a.reshape(m, C // 128, 128)
    EA = np.broadcast_to(np.asarray(ea, dtype=np.float64), a.shape).reshape(m, C // 128, 128)
    sc = s[:, :, None]
    v = A / sc
    ev = EA / sc + (0.0 if pow2 else 1.01 * U1) * (np.abs(A) + EA) / sc
    lo = F.E4M3_TABLE[F.e4m3_encode(v - ev)]
    hi = F.E4M3_TABLE[F.e4m3_encode(v + ev)]
    return v, lo, hi


def block_scale(amax: np.ndarray, pow2: bool = False) -> np.ndarray:
    """The re-quantisation scale of a block with maximum amax (R6 / R12):
    fl32(amax / 448), or the smallest power of two >= amax / 448; 1 for a
    zero block."""
    if pow2:
        return np.ldexp(1.0, pow2_scale_exponent(amax))
    return np.where(amax == 0.0, 1.0, F.f32_round(amax / F.E4M3_MAX))


def scale_window(a: np.ndarray, ea: np.ndarray, pow2: bool = False):
    """Smallest and largest block scale the device may compute from its own
    block maximum (within ea of the exact one), per row and 128-channel
    block; a zero maximum gives 1.  Returns (s_lo, s_hi, may_be_zero,
    must_be_zero)."""
    m, C = a.shape
    A = np.abs(a).reshape(m, C // 128, 128)
    EA = np.broadcast_to(np.asarray(ea, dtype=np.float64), a.shape).reshape(m, C // 128, 128)
    amax_lo = np.maximum(A - EA, 0.0).max(axis=2)
    amax_hi = (A + EA).max(axis=2)
    # a device maximum anywhere in [amax_lo, amax_hi]; where that range reaches
    # zero, any scale up to s_hi (or 1, for a maximum of exactly zero)
    s_lo = np.where(amax_lo > 0, block_scale(amax_lo, pow2), 0.0)
    s_hi = block_scale(amax_hi, pow2)
    return s_lo, s_hi, amax_lo == 0.0, amax_hi == 0.0


def requant_fp8(a: np.ndarray, a_err=None, resolve=None, resolve_scales=None, pow2: bool = False):
    """Per-row, per-128-channel FP8 re-quantisation of the intermediate
    (Tile Kernels section, quantisation bullet, fused with SwiGLU; reading R6).

    Without a_err: s = fl32(amax / 448) (1 for a zero block), or with pow2 the
    smallest power of two >= amax / 448 (R12's rule), codes =
    E4M3_RNE_sat(a / s).  With a_err (the R10 bound of another
    implementation's a) and its scales and codes:
    * resolve_scales [m, C/128] must lie within the scale window of each block
      (scale_window) and are then used as that block's s;
    * resolve [m, C] codes replace the oracle's where the value window of a / s
      holds more than one E4M3 value, and must lie in it; elsewhere they must
      equal the oracle's code (compared by value, so +0 and -0 agree).
    ValueError otherwise.

    Returns (codes uint8 [m, C], scales float64 [m, C/128] (fp32 values),
    dequantised float64 [m, C])."""
    m, C = a.shape
    blocks = a.reshape(m, C // 128, 128)
    amax = np.abs(blocks).max(axis=2)
    s = block_scale(amax, pow2)
    if a_err is not None and resolve_scales is not None:
        rs = np.asarray(resolve_scales, dtype=np.float64).reshape(m, C // 128)
        s_lo, s_hi, may_zero, must_zero = scale_window(a, a_err, pow2)
        ok = ((rs >= s_lo) & (rs <= s_hi) & ~must_zero) | ((rs == 1.0) & may_zero)
        if not np.all(ok):
            r, b = np.argwhere(~ok)[0]
            raise ValueError(f"a supplied scale {rs[r, b]!r} (row {r}, block {b}) lies outside "
                             f"[{s_lo[r, b]!r}, {s_hi[r, b]!r}]")
        s = rs
    v = blocks / s[:, :, None]
    codes = F.e4m3_encode(v)
    if a_err is not None and resolve is not None:
        _, lo, hi = requant_window(a, a_err, s, pow2)
        amb = lo != hi
        r = np.asarray(resolve, dtype=np.uint8).reshape(m, C // 128, 128)
        rv, cv = F.E4M3_TABLE[r], F.E4M3_TABLE[codes]
        inside = (rv >= lo) & (rv <= hi)
        if not np.all(inside[amb]):
            raise ValueError("a supplied code at a re-quantisation near-tie lies outside its window")
        if not np.all(rv[~amb] == cv[~amb]):
            bad = np.argwhere(~amb & (rv != cv))[0]
            raise ValueError(f"a supplied code differs from the oracle's away from a near-tie at "
                             f"(row, block, channel) {tuple(int(i) for i in bad)}")
        codes = np.where(amb, r, codes)
    deq = F.E4M3_TABLE[codes] * s[:, :, None]
    return codes.reshape(m, C), s, deq.reshape(m, C)


def bf16_window(a: np.ndarray, ea: np.ndarray):
    """Smallest and largest BF16 value the device's rounding of an a within ea
    of the exact one can give (R10)."""
    return F.bf16_round(a - ea), F.bf16_round(a + ea)


def quantise_intermediate(spec: Spec, a: np.ndarray, a_err=None, resolve=None, resolve_scales=None) -> np.ndarray:
    """The value GEMM2 consumes: FP8 re-quantised (R6, R10, R11), or
    BF16-rounded for all-BF16 layers.  With a_err and resolve (the device's
    BF16 values), those replace the oracle's where the BF16 window holds two
    values and must equal them elsewhere."""
    if spec.act == "bf16":
        r = F.bf16_round(a)
        if a_err is not None and resolve is not None:
            lo, hi = bf16_window(a, a_err)
            amb = lo != hi
            rv = F.bf16_decode(resolve)
            if not np.all(((rv >= lo) & (rv <= hi))[amb]):
                raise ValueError("a supplied BF16 intermediate at a rounding near-tie lies outside its window")
            if not np.all(rv[~amb] == r[~amb]):
                raise ValueError("a supplied BF16 intermediate differs from the oracle's away from a near-tie")
            r = np.where(amb, rv, r)
        return r
    return requant_fp8(a, a_err, resolve, resolve_scales, spec.scales == "pow2")[2]


def expert_intermediate(spec: Spec, xrows: np.ndarray, w_gu: np.ndarray) -> np.ndarray:
    """Linear 1 (gate|up) and SwiGLU of one expert's rows, before requant."""
    G = xrows @ w_gu.T                        # [m, 2I]
    return swiglu(G[:, : spec.I], G[:, spec.I:])


def expert_ffn(spec: Spec, xrows: np.ndarray, w_gu: np.ndarray, w_d: np.ndarray) -> np.ndarray:
    """One expert on its gathered rows: linear 1 (gate|up), SwiGLU, requant,
    linear 2 (Mega MoE section: 线性变换 -> SwiGLU -> 线性变换).

    xrows [m, H] fp64; w_gu [2I, H] and w_d [H, I] dequantised fp64."""
    a = expert_intermediate(spec, xrows, w_gu)
    ahat = quantise_intermediate(spec, a)
    return ahat @ w_d.T                       # [m, H]


def powers_of_two(v) -> bool:
    """True when every value of v is a positive power of two."""
    v = np.asarray(v, dtype=np.float64)
    m, _ = np.frexp(v)
    return bool(np.all(m == 0.5))


# ------------------------------------------------------------------- routing
def router_additions(H: int) -> int:
    """Roundings a product of the router's dot product can pass through on the
    device: up to 132 inside the four chained BF16 MFMAs of one 128-channel
    block, the multiply by the activation scale and one addition per block,
    up to 8 additions of channel-slice partial sums, and the bias."""
    return 132 + 2 + H // 128 + 8 + 1


def router_input(spec: Spec, inputs: dict) -> np.ndarray:
    """The activations the router reads: the dequantised FP8 input, or the
    BF16 input itself (all-BF16 layers, and layers that quantise their input:
    R3, R12)."""
    if spec.act in ("bf16", "bf16_fp8"):
        return F.bf16_decode(inputs["x"])
    return decode_activations(spec, inputs["x"], inputs.get("x_scales"))


def logit_bound(spec: Spec, inputs: dict) -> np.ndarray:
    """Absolute bound [T, E] on |device logit - exact logit| (R10):
    gamma_n * (sum_h |x_h Wr_h| + |b|), and 0 where every partial sum is exact
    in fp32 (power-of-two activation scales, grid-aligned operands and bias)."""
    xhat = router_input(spec, inputs)
    router_w, router_bias = inputs["router_w"], inputs.get("router_bias")
    x_scales = inputs.get("x_scales") if spec.act == "fp8" else None
    wr = F.bf16_decode(router_w)
    b = np.zeros(wr.shape[0]) if router_bias is None else np.asarray(router_bias, dtype=np.float32).astype(np.float64)
    S = np.abs(xhat) @ np.abs(wr).T + np.abs(b)[None, :]
    e = gamma(router_additions(xhat.shape[1])) * S
    pow2 = x_scales is None or powers_of_two(x_scales)
    if pow2:
        q = min(_lowest_bit_exponent(xhat) + _lowest_bit_exponent(wr), _lowest_bit_exponent(b))
        e = np.where(S < np.ldexp(1.0, 24 + q), 0.0, e)
    return e


# ----------------------------------------------------------------- the layer
def route(spec: Spec, inputs: dict):
    """Gating for all tokens: (xhat, logits, ids, weights).  xhat are the
    activations the experts read; the router reads the BF16 input itself
    when the layer quantises it (R12)."""
    xhat = decode_activations(spec, inputs["x"], inputs.get("x_scales"))
    xr = router_input(spec, inputs) if spec.act == "bf16_fp8" else xhat
    logits = router_logits(xr, inputs["router_w"], inputs.get("router_bias"))
    ids = topk_select(logits, spec.k)
    w = topk_weights(logits, ids)
    return xhat, logits, ids, w


def layer(spec: Spec, inputs: dict, ids=None, tokens=None, inter=None, inter_scales=None) -> dict:
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

    inter, inter_scales: another implementation's intermediate in permuted
    row order (E4M3 codes [T*k, I] with fp32 scales [T*k, I/128], or BF16 bit
    patterns [T*k, I]).  Where the R10 bound of that implementation makes more
    than one value correct, its value is used (it must lie in the window);
    elsewhere it must equal the oracle's (ValueError otherwise).

    Returns dict(y, logits, ids, weights, counts, offsets, perm, row_of),
    y being the unrounded fp64 output rows (of `tokens` when given)."""
    xhat, logits, sel, _ = route(spec, inputs)
    if ids is None:
        ids = sel
    ids = np.asarray(ids, dtype=np.int64)
    w = topk_weights(logits, ids)
    counts, offsets, perm, row_of = permutation(ids, spec.E)
    # the scales of the activations the experts read (None for BF16 layers)
    x_scales = inputs.get("x_scales")
    if spec.act == "bf16_fp8":
        x_scales = quantise_tokens_fp8(F.bf16_decode(inputs["x"]), spec.scales == "pow2")[1]

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
        wgu_s = None if inputs.get("w_gate_up_scales") is None else np.asarray(inputs["w_gate_up_scales"][e])
        wd_s = None if inputs.get("w_down_scales") is None else np.asarray(inputs["w_down_scales"][e])
        w_gu = decode_weight(spec, np.asarray(inputs["w_gate_up"][e]), wgu_s)
        w_d = decode_weight(spec, np.asarray(inputs["w_down"][e]), wd_s)
        xr = xhat[toks]
        if inter is None:
            a = expert_intermediate(spec, xr, w_gu)
            ahat = quantise_intermediate(spec, a)
        else:
            prow = np.arange(offsets[e], offsets[e + 1])[keep]
            pow2 = (spec.act == "bf16" or powers_of_two(np.asarray(x_scales)[toks])) and \
                   (spec.weight != "fp8" or powers_of_two(wgu_s))
            a, ea = intermediate_bound(spec, xr, w_gu, pow2)
            sc = None if inter_scales is None else np.asarray(inter_scales[prow])
            ahat = quantise_intermediate(spec, a, ea, np.asarray(inter[prow]), sc)
        O = ahat @ w_d.T
        wt = w.reshape(-1)[rows]
        # Tokens are distinct within one expert, so these row updates never
        # collide; the sum over j is formed across the expert loop.
        y[out_row[toks]] += wt[:, None] * O
    return dict(y=y, logits=logits, ids=ids, weights=w, counts=counts,
                offsets=offsets, perm=perm, row_of=row_of, xhat=xhat)


# ------------------------------------------------------------------ backward
def silu_grad(z: np.ndarray) -> np.ndarray:
    """d/dz SiLU(z) = sigma(z) * (1 + z * (1 - sigma(z)))."""
    sg = 1.0 / (1.0 + np.exp(-z))
    return sg * (1.0 + z * (1.0 - sg))


def forward_exact(xh, xr, wr, b, w_gu, w_d, ids, I: int) -> np.ndarray:
    """The layer as a function of fp64 parameters, no rounding anywhere (R14):
    xh [T, H] the experts' input, xr [T, H] the router's input, wr [E, H],
    b [E], w_gu [E, 2I, H], w_d [E, H, I], ids [T, k] fixed."""
    logits = xr @ wr.T + b[None, :]
    w = topk_weights(logits, ids)
    T, k = ids.shape
    y = np.zeros((T, w_d.shape[1]))
    for t in range(T):
        for j in range(k):
            e = ids[t, j]
            gu = w_gu[e] @ xh[t]
            y[t] += w[t, j] * (w_d[e] @ swiglu(gu[:I], gu[I:]))
    return y


def backward_exact(xh, xr, wr, b, w_gu, w_d, ids, dy, I: int) -> dict:
    """Gradients of sum(dy * forward_exact(...)) (R14), token by token:

    dw[t, j]  = <dy[t], o>,  o = SwiGLU(g, u) W_d[e]^T
    dW_d[e]  += w[t, j] dy[t]^T a             (a = SwiGLU(g, u))
    da        = w[t, j] dy[t] W_d[e]
    dg        = da * u * SiLU'(g),  du = da * SiLU(g)
    dW_gu[e] += [dg; du]^T xh[t],  dx[t] += [dg; du] W_gu[e]
    dl[t, j]  = w[t, j] (dw[t, j] - sum_i w[t, i] dw[t, i])   (softmax over the selection)
    dW_r[e]  += dl[t, j] xr[t],  db[e] += dl[t, j],  dxr[t] += dl[t, j] W_r[e]

    dx is the gradient of the layer's input: the experts' and the router's
    parts added (any quantisation between the input and either reader passes
    straight through, R14)."""
    logits = xr @ wr.T + b[None, :]
    w = topk_weights(logits, ids)
    T, k = ids.shape
    H = xh.shape[1]
    dx = np.zeros_like(xh)
    dxr = np.zeros_like(xr)
    dw_gu = np.zeros_like(w_gu)
    dw_d = np.zeros_like(w_d)
    dwr = np.zeros_like(wr)
    db = np.zeros_like(b)
    dws = np.zeros((T, k))
    for t in range(T):
        for j in range(k):
            e = ids[t, j]
            gu = w_gu[e] @ xh[t]
            g, u = gu[:I], gu[I:]
            a = swiglu(g, u)
            dws[t, j] = dy[t] @ (w_d[e] @ a)
            dw_d[e] += w[t, j] * np.outer(dy[t], a)
            da = w[t, j] * (dy[t] @ w_d[e])
            dgu = np.concatenate([da * u * silu_grad(g), da * silu(g)])
            dw_gu[e] += np.outer(dgu, xh[t])
            dx[t] += dgu @ w_gu[e]
        dl = w[t] * (dws[t] - w[t] @ dws[t])
        for j in range(k):
            e = ids[t, j]
            dwr[e] += dl[j] * xr[t]
            db[e] += dl[j]
            dxr[t] += dl[j] * wr[e]
    return dict(dx=dx + dxr, dx_experts=dx, dx_router=dxr, dw_gate_up=dw_gu, dw_down=dw_d, dw_router=dwr, dbias=db, dweights=dws)


def weight_grad_elements(xh, xr, wr, b, w_gu_e, w_d_e, e: int, ids, dy, I: int, chans, cols) -> dict:
    """Elements of one expert's weight gradients (R14) from their
    definition, for the channels `chans` (indices into 0..I-1) and the model
    columns `cols`: dW_gate_up[e][i][h] (gate rows i, up rows I + i) and
    dW_down[e][h][i], summed over the (token, slot) pairs routed to e:

    dG = dA_i u_i SiLU'(g_i),  dU = dA_i SiLU(g_i),  dA_i = w <dy, W_d[e][:, i]>
    dW_gate[i][h] += dG x[h],  dW_up[i][h] += dU x[h],
    dW_down[h][i] += w dy[h] SiLU(g_i) u_i

    with g_i = <W_gu[e][i], x>, u_i = <W_gu[e][I + i], x> and w the pair's
    routing weight (softmax over the token's selected logits).  Only rows i
    and I + i of W_gu[e] and column i of W_d[e] are read, so the cost is
    three dot products of length H per pair and channel."""
    ids = np.asarray(ids, dtype=np.int64)
    chans = np.asarray(chans, dtype=np.int64)
    cols = np.asarray(cols, dtype=np.int64)
    gate = np.zeros((chans.size, cols.size))
    up = np.zeros((chans.size, cols.size))
    down = np.zeros((cols.size, chans.size))
    toks, slots = np.nonzero(ids == e)
    for t, j in zip(toks, slots):
        logits = xr[t] @ wr.T + b
        w = topk_weights(logits[None, :], ids[t][None, :])[0, j]
        for c, i in enumerate(chans):
            g = w_gu_e[i] @ xh[t]
            u = w_gu_e[I + i] @ xh[t]
            da = w * (dy[t] @ w_d_e[:, i])
            gate[c] += da * u * silu_grad(np.array(g)) * xh[t, cols]
            up[c] += da * silu(np.array(g)) * xh[t, cols]
            down[:, c] += w * dy[t, cols] * silu(np.array(g)) * u
    return dict(dw_gate=gate, dw_up=up, dw_down=down)


def layer_backward(spec: Spec, inputs: dict, ids, dy) -> dict:
    """The backward pass of the layer (R14) for routing ids [T, k] and the
    output gradient dy [T, H]: gradients of x, W_gate_up, W_down, W_r and
    the bias, in fp64, taken at the decoded values the forward pass reads
    (BF16 layers: the values themselves)."""
    xh = decode_activations(spec, inputs["x"], inputs.get("x_scales"))
    xr = router_input(spec, inputs)
    wr = F.bf16_decode(inputs["router_w"])
    b = np.zeros(wr.shape[0]) if inputs.get("router_bias") is None else \
        np.asarray(inputs["router_bias"], dtype=np.float32).astype(np.float64)
    E = spec.E
    sc = lambda key, e: None if inputs.get(key) is None else np.asarray(inputs[key][e])
    w_gu = np.stack([decode_weight(spec, np.asarray(inputs["w_gate_up"][e]), sc("w_gate_up_scales", e)) for e in range(E)])
    w_d = np.stack([decode_weight(spec, np.asarray(inputs["w_down"][e]), sc("w_down_scales", e)) for e in range(E)])
    return backward_exact(xh, xr, wr, b, w_gu, w_d, np.asarray(ids, dtype=np.int64),
                          np.asarray(dy, dtype=np.float64), spec.I)
