"""CPU oracle of the routed-expert MoE FFN on packed low-bit expert weights.

TEST INFRASTRUCTURE.  This module is the slow, plain reference that the GPU
library is checked against.  Only the test-suite, the smoke check and the
benchmark's CPU-baseline leg may import it; the GPU product path never calls it,
and it shares no code, table or helper with the HIP sources.

Everything is NumPy in float64 (products of bf16 / fp16 / E2M1 / E4M3 values with
power-of-two scales are exact in float64), written from the pages' definitions:

* Hy4 layer shape and the routed/shared split -- "Hy4-preview Flash-MoE STQ1_0"
  (anemll), Package details table (256 routed experts, 8 selected per token, one
  shared expert, embedding 6144, MoE intermediate 2048).
* STQ1_0 -- "Hy4-preview-GGUF" (AngelSlim), section 3 "STQ1_0 and the
  mixed-precision strategy", The format; and "Hy4-preview Flash-MoE STQ1_0",
  "How the STQ1_0 packing works": 256-weight blocks of 64 groups of four, exactly
  one zero and three values in {-d, +d} per group, 4 x 2^3 = 32 patterns, 5 bits a
  group, one fp16 scale per block, 42 bytes per 256 weights.  The bit layout is our
  own (the pages' codebook ABI is not on them): pattern p = 8*z + s, z the zero
  lane, bit i of s the sign of the i-th non-zero lane in ascending lane order;
  byte i of the 32-byte nibble area holds p(2i) & 15 in its low and p(2i+1) & 15 in
  its high nibble; the 8-byte high-bit area is a little-endian 64-bit word whose
  bit g is p(g) >> 4.  Blocks run over the row-major [out][in] matrix, flattened.
* MXFP4 x FP8 -- "Hy4-preview-SF-WFP4AFP8" (siliconflow), Quant Diff table
  (recipe weight_fp4_activation_fp8, group 32, ue8m0 / e4m3; routed experts FP4
  E2M1 weights with FP8 E4M3 activations, group 32).  The pages name the formats
  only; the value sets and the scale rule are the OCP Microscaling v1.0 ones.
* Router kept in BF16 -- same table, BF16 row (router mlp.gate).
* SwiGLU expert MLP (gate_proj, up_proj, down_proj) -- same table, and the
  Hy4-preview-GGUF tensor families ffn_gate_exps / ffn_up_exps / ffn_down_exps.

Readings where the pages are silent (routing function, tie order, combine rule,
norm placement, scale rule) are stated next to the function that takes them.
"""
from __future__ import annotations

import numpy as np

# =============================================================================
# Scalar number formats
# =============================================================================


def bf16_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns -> float64 (bf16 is the top half of an IEEE binary32)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def fp16_to_f64(bits) -> np.ndarray:
    """IEEE binary16 bit patterns -> float64 (the STQ1_0 block scale d)."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def f64_to_bf16_bits(x) -> np.ndarray:
    """Round float64 values to bf16 (8 significant bits), nearest-even, finite only.

    Written from the format: a normal bf16 is m * 2^(e-7) with m an 8-bit integer
    in [128, 255]; below 2^-126 the quantum stays 2^-133.
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    _, e = np.frexp(a)                      # a = f * 2^e, f in [0.5, 1)
    e = np.maximum(e - 1, -126)             # floor(log2 a), clamped to the normal floor
    q = np.ldexp(1.0, e - 7)                # quantum of the binade
    r = np.rint(a / q) * q                  # rint is round-half-to-even
    r = np.where(a == 0, 0.0, r)
    v = np.copysign(r, x).astype(np.float32)   # exact: r has <= 8 significant bits
    return (v.view(np.uint32) >> 16).astype(np.uint16)


def e2m1_value(code) -> np.ndarray:
    """FP4 E2M1: bit 3 sign, bits 2..1 exponent (bias 1), bit 0 mantissa."""
    c = np.asarray(code, dtype=np.int64) & 15
    s = np.where(c & 8, -1.0, 1.0)
    e = (c >> 1) & 3
    m = c & 1
    mag = np.where(e == 0, 0.5 * m, np.ldexp(1.0 + 0.5 * m, e - 1))
    return s * mag


def e4m3_value(code) -> np.ndarray:
    """FP8 E4M3 ("fn" variant): bias 7, no infinities, S.1111.111 is NaN."""
    c = np.asarray(code, dtype=np.int64) & 255
    s = np.where(c & 128, -1.0, 1.0)
    e = (c >> 3) & 15
    m = c & 7
    mag = np.where(e == 0, np.ldexp(m.astype(np.float64), -9),
                   np.ldexp(1.0 + m / 8.0, e - 7))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return s * mag


def ue8m0_value(code) -> np.ndarray:
    """UE8M0 scale byte v: 2^(v-127); 255 is NaN."""
    c = np.asarray(code, dtype=np.int64) & 255
    return np.where(c == 255, np.nan, np.ldexp(1.0, c - 127))


E4M3_MAX = 448.0   # 1.75 * 2^8, the largest finite E4M3 magnitude
E4M3_EMAX = 8      # exponent of the largest E4M3 binade


def e4m3_encode(y) -> np.ndarray:
    """Encode float64 values into E4M3 codes: round to nearest (ties to even) on the
    unbounded E4M3 grid, then saturate the magnitude to 448.  The sign bit is the
    input's sign bit, so a negative value that rounds to zero gives 0x80."""
    y = np.asarray(y, dtype=np.float64)
    a = np.abs(y)
    _, e = np.frexp(a)
    e = e - 1                                  # floor(log2 a) for a > 0
    q = np.where(a < 2.0 ** -6, 2.0 ** -9, np.ldexp(1.0, e - 3))
    r = np.rint(a / q) * q
    r = np.where(a == 0, 0.0, np.minimum(r, E4M3_MAX))
    _, er = np.frexp(r)
    er = er - 1
    sub = r < 2.0 ** -6
    mant_sub = np.rint(r / 2.0 ** -9).astype(np.int64)
    exp_field = np.where(sub, 0, er + 7)
    mant_norm = np.rint(np.ldexp(r, -np.where(sub, 0, er) + 3)).astype(np.int64) - 8
    code = np.where(sub, mant_sub, (exp_field.astype(np.int64) << 3) | mant_norm)
    sign = np.signbit(y).astype(np.int64) << 7
    return (code | sign).astype(np.uint8)


def mx_quantize_e4m3(v) -> tuple[np.ndarray, np.ndarray]:
    """MX (OCP Microscaling) quantisation of the last axis in groups of 32 into
    E4M3 elements with one UE8M0 scale per group.

    Reading of the group-32 ue8m0 / e4m3 activation recipe: the shared exponent is
    X = floor(log2(amax)) - 8 (8 = exponent of E4M3's largest binade), clamped to
    [-127, 127] and stored as X + 127; elements are v / 2^X rounded to nearest even
    and saturated to +-448.  A group whose amax is 0 stores scale byte 0 and zero
    elements.
    """
    v = np.asarray(v, dtype=np.float64)
    K = v.shape[-1]
    assert K % 32 == 0, "MX groups are 32 elements along the last axis"
    g = v.reshape(v.shape[:-1] + (K // 32, 32))
    amax = np.abs(g).max(axis=-1)
    _, e = np.frexp(amax)
    X = np.clip(e - 1 - E4M3_EMAX, -127, 127)
    X = np.where(amax == 0, -127, X)
    codes = e4m3_encode(g / np.ldexp(1.0, X)[..., None])
    codes = np.where((amax == 0)[..., None], np.uint8(0), codes).astype(np.uint8)
    return codes.reshape(v.shape), (X + 127).astype(np.uint8)


def mx_dequantize_e4m3(codes, scales) -> np.ndarray:
    c = np.asarray(codes)
    K = c.shape[-1]
    vals = e4m3_value(c).reshape(c.shape[:-1] + (K // 32, 32))
    return (vals * ue8m0_value(scales)[..., None]).reshape(c.shape)


# =============================================================================
# STQ1_0 (our bit layout of the pages' 5-bit pattern, 42 bytes / 256 weights)
# =============================================================================

STQ_BLOCK = 256
STQ_GROUPS = 64
STQ_CODE_BYTES = 40   # 32 nibble bytes + 8 high-bit bytes
STQ_SCALE_BYTES = 2   # one binary16 scale


def stq1_pattern(p: int) -> list[int]:
    """The four ternary lanes (in units of d) of 5-bit pattern p = 8*z + s."""
    z, s = p >> 3, p & 7
    lanes = [0, 0, 0, 0]
    nz = [j for j in range(4) if j != z]          # ascending lane order
    for i, j in enumerate(nz):
        lanes[j] = -1 if (s >> i) & 1 else 1
    return lanes


_PATTERNS = np.array([stq1_pattern(p) for p in range(32)], dtype=np.float64)


def stq1_pack(z, s, d_bits) -> tuple[np.ndarray, np.ndarray]:
    """Pack per-group zero lanes z (0..3) and sign fields s (0..7) with per-block
    fp16 scales into (code bytes [n_blk*40], scale bits [n_blk])."""
    z = np.asarray(z, dtype=np.uint8)
    s = np.asarray(s, dtype=np.uint8)
    n_groups = z.size
    assert n_groups % STQ_GROUPS == 0 and s.size == n_groups
    n_blk = n_groups // STQ_GROUPS
    p = ((z.astype(np.uint16) << 3) | s).reshape(n_blk, STQ_GROUPS)
    lo = (p & 15).astype(np.uint8)
    qs = lo[:, 0::2] | (lo[:, 1::2] << 4)                   # [n_blk, 32]
    hi = (p >> 4).astype(np.uint64)
    word = np.zeros(n_blk, dtype=np.uint64)
    for g in range(STQ_GROUPS):
        word |= hi[:, g] << np.uint64(g)
    qh = word.astype('<u8').view(np.uint8).reshape(n_blk, 8)
    codes = np.concatenate([qs, qh], axis=1).reshape(-1)
    d = np.asarray(d_bits, dtype=np.uint16).reshape(-1)
    assert d.size == n_blk
    return codes, d.copy()


def stq1_patterns_of(codes) -> np.ndarray:
    """Recover the 5-bit pattern of every group: [n_blk, 64] ints."""
    c = np.asarray(codes, dtype=np.uint8).reshape(-1, STQ_CODE_BYTES)
    qs, qh = c[:, :32], c[:, 32:]
    lo = np.empty((c.shape[0], STQ_GROUPS), dtype=np.int64)
    lo[:, 0::2] = qs & 15
    lo[:, 1::2] = qs >> 4
    # little-endian 64-bit word: byte j holds groups 8j..8j+7, lowest bit first
    hi = np.unpackbits(np.ascontiguousarray(qh), axis=1, bitorder='little')
    return lo | (hi.astype(np.int64) << 4)


def stq1_decode(codes, scales, n_weights: int | None = None) -> np.ndarray:
    """Decode packed STQ1_0 to float64 weights in flattened order."""
    p = stq1_patterns_of(codes)                               # [n_blk, 64]
    w = _PATTERNS[p].reshape(p.shape[0], STQ_BLOCK)           # units of d
    d = fp16_to_f64(scales).reshape(-1, 1)
    out = (w * d).reshape(-1)
    if n_weights is not None:
        assert n_weights == out.size
    return out


def stq1_matrix(codes, scales, N: int, K: int) -> np.ndarray:
    """One expert matrix [N, K] (row-major, blocks over the flattened matrix)."""
    return stq1_decode(codes, scales, N * K).reshape(N, K)


# -----------------------------------------------------------------------------
# STQ1_0 encoders ("Hy4-preview-GGUF" (AngelSlim), section 3, Our encoder)
# -----------------------------------------------------------------------------
# A float matrix is encoded per 256-weight block of its flattened row-major order (the
# blocks stq1_decode reads), with importance w per weight: the imatrix entry of the
# weight's input column (column = flat index mod K), or 1 without an imatrix.
#  * upstream: d = the block's largest magnitude; in every group the lane of smallest |x|
#    is zeroed.
#  * wls (the pages' encoder): alternate (i) the weighted least-squares scale
#    d = sum(w sel x) / sum(w sel^2) for the current selection and (ii) in every group the
#    zero at the lane of smallest incremental cost w_j (x_j^2 - (|x_j| - d)^2), 3 rounds.
# Readings (the pages leave these open): the rounds start from the upstream zero placement;
# a round is (i) then (ii), and a final (i) fits d to the final selection; a kept lane
# takes the sign of x (x = 0 counts as positive); ties go to the lowest lane; a block whose
# kept lanes all have w = 0 keeps d = amax; d is rounded to fp16 (nearest even) once, at the
# end.

STQ_ENC_ROUNDS = 3


def _stq_blocks(x, K: int, imatrix):
    """x and its importance as [n_blk, 64, 4] float64."""
    x = np.asarray(x, dtype=np.float64).reshape(-1)
    assert x.size % STQ_BLOCK == 0
    if imatrix is None:
        w = np.ones_like(x)
    else:
        w = np.asarray(imatrix, dtype=np.float64).reshape(-1)[np.arange(x.size) % K]
    shp = (x.size // STQ_BLOCK, STQ_GROUPS, 4)
    return x.reshape(shp), w.reshape(shp)


def stq1_ls_scale(xb, wb, z):
    """Weighted least-squares d of each block for zero lanes z [n_blk, 64], the kept lanes
    carrying sign(x): sel x = |x| and sel^2 = 1 on them."""
    kept = np.arange(4)[None, None, :] != np.asarray(z)[:, :, None]
    num = (wb * np.abs(xb) * kept).sum(axis=(1, 2))
    den = (wb * kept).sum(axis=(1, 2))
    amax = np.abs(xb).max(axis=(1, 2))
    return np.where(den > 0, num / np.where(den > 0, den, 1.0), amax)


def stq1_zero_placement(xb, wb, d):
    """Zero lane of every group: the smallest incremental cost w (x^2 - (|x| - d)^2) of
    zeroing it instead of keeping it at sign(x) d (first lane on ties)."""
    cost = wb * (xb * xb - (np.abs(xb) - np.asarray(d)[:, None, None]) ** 2)
    return np.argmin(cost, axis=2)


def stq1_encode_parts(x, K: int, imatrix=None, method: str = "wls", rounds: int = STQ_ENC_ROUNDS):
    """(zero lanes [n_blk*64], sign fields [n_blk*64], d [n_blk] float64 before rounding)."""
    xb, wb = _stq_blocks(x, K, imatrix)
    z = np.argmin(np.abs(xb), axis=2)
    if method == "upstream":
        d = np.abs(xb).max(axis=(1, 2))
    else:
        assert method == "wls"
        for _ in range(rounds):
            d = stq1_ls_scale(xb, wb, z)
            z = stq1_zero_placement(xb, wb, d)
        d = stq1_ls_scale(xb, wb, z)
    neg = xb < 0
    s = np.zeros(z.shape, dtype=np.int64)
    for zz in range(4):
        nz = [j for j in range(4) if j != zz]
        sz = sum(neg[:, :, j].astype(np.int64) << i for i, j in enumerate(nz))
        s = np.where(z == zz, sz, s)
    return z.reshape(-1).astype(np.uint8), s.reshape(-1).astype(np.uint8), d


def stq1_encode(x, K: int, imatrix=None, method: str = "wls", rounds: int = STQ_ENC_ROUNDS):
    """Encode a float matrix (flattened row-major, K columns) into STQ1_0 (code bytes, fp16
    scale bits)."""
    z, s, d = stq1_encode_parts(x, K, imatrix, method, rounds)
    return stq1_pack(z, s, d.astype(np.float16).view(np.uint16))


def stq1_weighted_ssd(x, K: int, codes, scales, imatrix=None):
    """Weighted squared error sum w (x - decode)^2 of every 256-weight block."""
    xb, wb = _stq_blocks(x, K, imatrix)
    y = stq1_decode(codes, scales).reshape(xb.shape)
    return (wb * (xb - y) ** 2).sum(axis=(1, 2))


# =============================================================================
# MXFP4 weights
# =============================================================================


def mxfp4_matrix(codes, scales, N: int, K: int) -> np.ndarray:
    """Weights [N, K]: E2M1 code pairs [N, K/2] (element 2i in the low nibble) times
    UE8M0 group-32 scales [N, K/32] along K."""
    c = np.asarray(codes, dtype=np.uint8).reshape(N, K // 2)
    el = np.empty((N, K), dtype=np.int64)
    el[:, 0::2] = c & 15
    el[:, 1::2] = c >> 4
    v = e2m1_value(el).reshape(N, K // 32, 32)
    sc = ue8m0_value(np.asarray(scales).reshape(N, K // 32))
    return (v * sc[..., None]).reshape(N, K)


# =============================================================================
# The layer
# =============================================================================


def route(k: int, x_bits=None, wr_bits=None, bias=None, logits_in=None):
    """Router logits, top-k selection and routing weights.

    The router is a BF16 linear layer (Hy4-preview-SF-WFP4AFP8, BF16 row of the
    Quant Diff table); selection keeps the token's k largest logits (Flash-MoE
    page: 8 selected experts per token).  The pages do not give the routing
    function; reading: softmax over all experts, keep the top k, renormalise over
    them -- which equals the softmax over the k selected logits, since the full
    denominator cancels.  Order: descending logit, ties to the lower expert index.
    A per-expert bias, when given, is added to the logits before everything else.
    A NaN logit (a NaN in the token's activations makes its whole row NaN) has no
    place in that order; reading: NaN ranks above every number and all NaNs are
    equal, so a NaN row selects experts 0 .. k-1, and the weights of a selection
    holding a NaN are NaN.

    Returns (logits [T, E] float64, ids [T, k] int32, w [T, k] float64).
    """
    if logits_in is not None:
        logits = np.asarray(logits_in, dtype=np.float64).copy()
    else:
        logits = bf16_to_f64(x_bits) @ bf16_to_f64(wr_bits).T
    if bias is not None:
        logits = logits + np.asarray(bias, dtype=np.float64)[None, :]
    T, E = logits.shape
    ids = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float64)
    for t in range(T):
        nan = np.isnan(logits[t])
        # NaN first, then by -logit, then by index (lexsort's last key is the primary one)
        order = np.lexsort((np.arange(E), np.where(nan, 0.0, -logits[t]), ~nan))
        sel = order[:k]
        ids[t] = sel
        ex = np.exp(logits[t, sel] - logits[t, sel].max())
        w[t] = ex / ex.sum()
    return logits, ids, w


def permute(ids, E: int):
    """Group the T*k (token, slot) pairs by expert, stably.

    Pair f = t*k + j.  Counting sort: offsets[e] = number of pairs whose expert is
    below e; within one expert, pairs keep increasing f.  sorted_pair[pos] = f and
    pair_pos[f] = pos.  The result is unique.

    A pair whose id is not an expert (outside [0, E): the library's rule for ids it
    cannot route) takes no position: pair_pos[f] = -1, offsets[E] counts the routed
    pairs only, and sorted_pair holds -1 from offsets[E] on.
    """
    flat = np.asarray(ids, dtype=np.int64).reshape(-1)
    P = flat.size
    counts = np.zeros(E, dtype=np.int64)
    for f in range(P):
        if 0 <= flat[f] < E:
            counts[flat[f]] += 1
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    fill = offsets[:-1].copy()
    sorted_pair = np.full(P, -1, dtype=np.int64)
    pair_pos = np.full(P, -1, dtype=np.int64)
    for f in range(P):
        e = flat[f]
        if not 0 <= e < E:
            continue
        sorted_pair[fill[e]] = f
        pair_pos[f] = fill[e]
        fill[e] += 1
    return sorted_pair.astype(np.int32), offsets.astype(np.int32), pair_pos.astype(np.int32)


def silu(g):
    """SiLU of the SwiGLU gate: g * sigmoid(g) = g / (1 + exp(-g))."""
    g = np.asarray(g, dtype=np.float64)
    return g / (1.0 + np.exp(-g))


def swiglu_expert(a, Wg, Wu, Wd, mx_h: bool = False):
    """One SwiGLU expert on rows a [n, K]: h = silu(a Wg^T) * (a Wu^T), y = h Wd^T.

    With mx_h the intermediate h is MX-quantised (E4M3, group 32 along the
    intermediate axis) before the down projection: every routed-expert linear of the
    WFP4AFP8 checkpoint takes FP8 E4M3 group-32 activations.
    Returns (h as fed to the down projection, y)."""
    g = a @ Wg.T
    u = a @ Wu.T
    h = silu(g) * u
    if mx_h:
        hq, hs = mx_quantize_e4m3(h)
        h = mx_dequantize_e4m3(hq, hs)
    return h, h @ Wd.T


def expert_ffn(x_bits, ids, sorted_pair, offsets, get_w, fmt: str):
    """Routed-expert outputs in sorted-pair order.

    get_w(e, m) returns expert e's float64 matrix m (0 gate [I,H], 1 up [I,H],
    2 down [H,I]).  fmt "stq1": inputs are the bf16 activations, h stays float64.
    fmt "mxfp4": the activations are MX-quantised to E4M3 (group 32 along H) first
    and h is MX-quantised before the down projection.
    Returns (y_pairs [P, H], h [P, I]) float64.
    """
    x = bf16_to_f64(x_bits)
    if fmt == "mxfp4":
        xq, xs = mx_quantize_e4m3(x)
        x = mx_dequantize_e4m3(xq, xs)
    k = ids.shape[1]
    E = len(offsets) - 1
    P = len(sorted_pair)
    H = x.shape[1]
    y = np.zeros((P, H))
    h_all = None
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        toks = np.asarray(sorted_pair[lo:hi]) // k
        h, ye = swiglu_expert(x[toks], get_w(e, 0), get_w(e, 1), get_w(e, 2), fmt == "mxfp4")
        if h_all is None:
            h_all = np.zeros((P, h.shape[1]))
        h_all[lo:hi] = h
        y[lo:hi] = ye
    return y, h_all


def shared_expert(x_bits, wg_bits, wu_bits, wd_bits):
    """The always-on shared expert (one per MoE block, Flash-MoE package table), in
    bf16 weights on the bf16 activations."""
    x = bf16_to_f64(x_bits)
    _, y = swiglu_expert(x, bf16_to_f64(wg_bits), bf16_to_f64(wu_bits), bf16_to_f64(wd_bits))
    return y


def shared_expert_mxfp8(x_bits, wg, wu, wd):
    """The shared expert in MXFP8 W8A8 group 32 ("Hy4-preview-SF-WFP4AFP8", Quant Diff
    table: mlp.shared_experts.{gate,up,down}_proj MXFP8 W8A8 g32): E4M3 weights with UE8M0
    scales per 32 along the input axis, x MX-quantised to E4M3 along H and h along I (the
    same rule as the routed experts' activations).  wg, wu, wd are (codes, scale bytes)."""
    a = mx_dequantize_e4m3(*mx_quantize_e4m3(bf16_to_f64(x_bits)))
    W = [mx_dequantize_e4m3(c, sc) for c, sc in (wg, wu, wd)]
    _, y = swiglu_expert(a, W[0], W[1], W[2], mx_h=True)
    return y


def combine(y_pairs, w, pair_pos, y_shared=None, residual=None):
    """out[t] = y_shared[t] + sum_j w[t, j] * y_pairs[pair_pos[t*k + j]] (+ residual).

    The pages show no gate on the shared expert, so it is added unweighted.  A pair
    that permute left unrouted (pair_pos -1) adds nothing."""
    T, k = w.shape
    H = y_pairs.shape[1]
    out = np.zeros((T, H)) if y_shared is None else np.array(y_shared, dtype=np.float64)
    for t in range(T):
        for j in range(k):
            if pair_pos[t * k + j] >= 0:
                out[t] += w[t, j] * y_pairs[pair_pos[t * k + j]]
    if residual is not None:
        out = out + residual
    return out


def rmsnorm_bf16(r, eps: float = 1e-6):
    """a = bf16(r / sqrt(mean(r^2) + eps)) per row (norm weight 1)."""
    r = np.asarray(r, dtype=np.float64)
    a = r / np.sqrt(np.mean(r * r, axis=-1, keepdims=True) + eps)
    return f64_to_bf16_bits(a)


def moe_layer(x_bits, k, get_w, fmt, wr_bits=None, bias=None, logits_in=None,
              shared=None, residual=None, shared_fmt: str = "bf16"):
    """Whole layer: route -> permute -> routed experts (+ shared, bf16 or MXFP8) ->
    combine.  Returns a dict of every stage."""
    logits, ids, w = route(k, x_bits, wr_bits, bias, logits_in)
    E = logits.shape[1]
    sp, off, pp = permute(ids, E)
    y_pairs, h = expert_ffn(x_bits, ids, sp, off, get_w, fmt)
    y_sh = None
    if shared is not None:
        y_sh = shared_expert(x_bits, *shared) if shared_fmt == "bf16" else shared_expert_mxfp8(x_bits, *shared)
    out = combine(y_pairs, w, pp, y_sh, residual)
    return dict(logits=logits, ids=ids, w=w, sorted_pair=sp, offsets=off, pair_pos=pp,
                y_pairs=y_pairs, h=h, y_shared=y_sh, out=out)
