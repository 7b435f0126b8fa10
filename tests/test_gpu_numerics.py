"""GPU checks of the numeric edges of the path, through the C ABI:

* routing of NaN logits (a NaN in x), out-of-range expert ids through permute / expert FFN /
  combine, and activation rows of wide dynamic range (one huge element among tiny ones,
  all-zero rows, bf16 subnormals) through the STQ1_0 prefill GEMMs and the fused decode;
* the E4M3 encoder of the MXFP4 gate/up epilogue (the scaled hardware conversion) against
  the integer rule and the oracle on chosen values;
* the accumulation error of the scaled FP8 x FP4 MFMA, measured on the down projection
  against an exact reference, and the FP8 code-flip rate of h that it causes.

Every reference comes from the CPU oracle or from exact arithmetic on the GPU's own
operands; nothing here reads an expected value from the HIP path."""
import math
import sys

import numpy as np
import pytest
import torch

import bit_quantized_moe_softmax_amd as M
import synth
from bit_quantized_moe_softmax_amd.layer import LayerBuffers, bf16_experts, run_layer
from oracle import moe_oracle as O
from tests.helpers import TOL, layer_inputs, oracle_weights, row_err, shapes

pytestmark = pytest.mark.gpu

# Bound on the scaled MFMA's error per dot product, relative to the sum of the magnitudes of
# its products: twice the largest value test_mx_scaled_mfma_accumulation_error measured
# (2^-16.15 over 262144 dot products of K = 2048; median 2^-19.9), which prints it on every
# run.  A sequential fp32 sum of the same products stays below 2^-23.8.
MFMA_REL_BOUND = 2.0 ** -15


def say(*a):
    print("[gpu-numerics]", *a, file=sys.__stderr__, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    M.lib()
    yield
    torch.cuda.synchronize()


def dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


def host(t, dtype=None):
    a = t.detach().cpu().numpy()
    return a.view(dtype) if dtype is not None else a


# ----------------------------------------------------------------------------- routing edges
def test_topk_nan_rows_bitexact():
    """Rows with NaN logits (some, all, next to +-inf): ids bit-exact with the oracle's rule
    (NaN above every number, NaNs tie), every id a real expert, NaN weights where the
    selection holds a NaN and the oracle's weights elsewhere."""
    g = np.random.default_rng(61)
    T, E, k = 9, 256, 8
    logits = g.standard_normal((T, E)).astype(np.float32)
    logits[0, :] = np.nan
    logits[1, [5, 77, 200]] = np.nan
    logits[2, 3] = np.inf
    logits[2, 9] = -np.inf
    logits[3, ::2] = np.nan
    logits[4, 250] = np.nan
    logits[4, 251] = np.inf
    logits[5, :] = -np.inf
    logits[6, 10] = -0.0
    logits[6, 11] = 0.0
    logits[6, 12:] = -1.0
    logits[7, :] = np.float32(-np.nan)            # NaN with the sign bit set
    d = M.Dims(T, 32, 32, E, k)
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    M.moe_route(d, None, None, None, dev(logits), None, ids, w)
    _, rid, rw = O.route(k, logits_in=logits.astype(np.float64))
    gi, gw = host(ids), host(w)
    assert ((gi >= 0) & (gi < E)).all()
    assert (gi == rid).all()
    assert (np.isnan(gw) == np.isnan(rw)).all()
    ok = ~np.isnan(rw)
    assert np.allclose(gw[ok], rw[ok], rtol=1e-6, atol=0)
    assert list(gi[0]) == list(range(k))


def test_permute_unroutable_ids_bitexact():
    """Ids outside [0, E) (-1 from the slot bank for an expert without a slot, E, large
    values) are dropped by the permutation exactly as the oracle drops them."""
    g = np.random.default_rng(62)
    for T, k, E in [(37, 8, 256), (5, 2, 8), (300, 4, 16), (2048, 8, 256)]:   # the last chunk-parallel
        ids = g.integers(0, E, (T, k)).astype(np.int32)
        bad = g.random((T, k)) < 0.2
        ids[bad] = g.choice(np.array([-1, -7, E, E + 5, 1 << 20], dtype=np.int32), bad.sum())
        d = M.Dims(T, 32, 32, E, k)
        sp = torch.empty(T * k, dtype=torch.int32, device="cuda")
        off = torch.empty(E + 1, dtype=torch.int32, device="cuda")
        pp = torch.empty(T * k, dtype=torch.int32, device="cuda")
        M.moe_permute(d, dev(ids), sp, off, pp)
        rsp, roff, rpp = O.permute(ids, E)
        say("permute with unroutable ids", T, k, E, "dropped", int(bad.sum()))
        assert (host(sp) == rsp).all() and (host(off) == roff).all() and (host(pp) == rpp).all()


def test_layer_with_unroutable_pairs():
    """A layer whose ids (as the slot bank's remap gives them) hold -1 for some pairs: permute
    drops them, the expert FFN runs only the routed pairs, and the combine adds nothing for
    the dropped ones -- against the oracle's layer with those pairs dropped."""
    c = synth.LayerCfg("unroutable", 13, 512, 256, 8, 2, True, "stq1", False, True, 1, 63)
    inp = layer_inputs(c)
    d = M.Dims(c.T, c.H, c.I, c.E, c.k)
    fmt = M.MOE_W_STQ1_0
    routed = M.Experts(fmt, *[(dev(cd), dev(sc)) for cd, sc in inp["routed"]])
    shared = bf16_experts(*(dev(w) for w in inp["shared"]))
    bufs = LayerBuffers(d, fmt, True)
    M.moe_route(d, None, None, None, dev(inp["logits_in"]), bufs.logits, bufs.topk_ids, bufs.topk_w)
    ids = host(bufs.topk_ids).copy()
    ids[ids == 3] = -1                                  # expert 3 has no slot
    ids[5, 1] = -1
    M.moe_permute(d, dev(ids), bufs.sorted_pair, bufs.offsets, bufs.pair_pos)
    x = dev(inp["x"])
    M.moe_expert_ffn(d, routed, shared, x, bufs.sorted_pair, bufs.offsets, bufs.y_pairs, bufs.y_shared, bufs.ws)
    M.moe_combine(d, bufs.y_pairs, bufs.topk_w, bufs.pair_pos, bufs.y_shared, None, bufs.out, None)
    torch.cuda.synchronize()
    _, _, rw = O.route(c.k, logits_in=inp["logits_in"])
    sp, off, pp = O.permute(ids, c.E)
    assert (host(bufs.sorted_pair) == sp).all() and (host(bufs.pair_pos) == pp).all()
    yp, _ = O.expert_ffn(inp["x"], ids, sp[:off[-1]], off, oracle_weights(c, inp["routed"]), "stq1")
    ysh = O.shared_expert(inp["x"], *inp["shared"])
    n = int(off[-1])
    assert row_err(host(bufs.y_pairs)[:n], yp).max() <= TOL
    yfull = np.zeros((d.P, c.H))
    yfull[:n] = yp
    ref = O.combine(yfull, rw, pp, ysh)
    err = row_err(host(bufs.out), ref)
    say("layer with unroutable pairs: routed", n, "of", d.P, "max row err", float(err.max()))
    assert err.max() <= TOL


def _run_fused(c, x, wr, routed_np, shared_np, bias=None):
    d = M.Dims(c.T, c.H, c.I, c.E, c.k)
    routed = M.Experts(M.MOE_W_STQ1_0, *[(dev(cd), dev(sc)) for cd, sc in routed_np])
    shared = bf16_experts(*(dev(w) for w in shared_np)) if shared_np is not None else None
    f32, i32 = torch.float32, torch.int32
    o = dict(logits=torch.empty((c.T, c.E), dtype=f32, device="cuda"),
             ids=torch.empty((c.T, c.k), dtype=i32, device="cuda"),
             w=torch.empty((c.T, c.k), dtype=f32, device="cuda"),
             sp=torch.empty(d.P, dtype=i32, device="cuda"),
             off=torch.empty(c.E + 1, dtype=i32, device="cuda"),
             pp=torch.empty(d.P, dtype=i32, device="cuda"),
             yp=torch.empty((d.P, c.H), dtype=f32, device="cuda"),
             ysh=torch.empty((c.T, c.H), dtype=f32, device="cuda") if shared is not None else None,
             out=torch.empty((c.T, c.H), dtype=f32, device="cuda"))
    ws = torch.zeros(M.moe_layer_decode_workspace_size(d, shared is not None), dtype=torch.uint8, device="cuda")
    M.moe_layer_decode(d, routed, shared, dev(x), dev(wr), dev(bias) if bias is not None else None,
                       o["logits"], o["ids"], o["w"], o["sp"], o["off"], o["pp"], o["yp"], o["ysh"],
                       None, o["out"], None, ws)
    torch.cuda.synchronize()
    return o


@pytest.mark.parametrize("T", [1, 3, 9])
def test_fused_decode_nan_token(T):
    """A token whose x holds a NaN routes to experts 0 .. k-1 in the fused decode (as in the
    oracle), and the other tokens of the batch keep their results."""
    c = synth.LayerCfg("nan", T, 512, 256, 16, 4, True, "stq1", False, False, 1, 64)
    inp = layer_inputs(c)
    x = inp["x"].copy()
    x[0, 17] = 0x7FC0                                   # bf16 NaN
    o = _run_fused(c, x, inp["wr"], inp["routed"], inp["shared"])
    rl, rid, _ = O.route(c.k, x, inp["wr"])
    gi = host(o["ids"])
    assert ((gi >= 0) & (gi < c.E)).all()
    assert list(gi[0]) == list(range(c.k))
    assert np.isnan(host(o["out"])[0]).all()
    if T > 1:
        ref = O.moe_layer(x[1:], c.k, oracle_weights(c, inp["routed"]), "stq1", wr_bits=inp["wr"],
                          shared=inp["shared"])
        assert (gi[1:] == ref["ids"]).all()
        err = row_err(host(o["out"])[1:], ref["out"])
        say("fused decode, NaN token beside", T - 1, "others: max row err", float(err.max()))
        assert err.max() <= TOL


def _wide_rows(T, H, seed):
    """bf16 activation rows of wide dynamic range: one huge element among tiny ones, an
    all-zero row, bf16 subnormals beside normal values, mixed magnitudes over 2^-40 .. 2^40,
    plus plain rows.  (A row of subnormals only would give outputs below fp32's range.)"""
    g = np.random.default_rng(seed)
    x = g.standard_normal((T, H)).astype(np.float32)
    x[0] = g.standard_normal(H) * 1e-6
    x[0, 123] = 3.0e4                                   # one huge element, 2^-34 .. row max
    x[1] = 0.0
    x[2] = g.standard_normal(H) * 1e-3
    x[2, ::3] = g.standard_normal((H + 2) // 3) * 1e-39   # bf16 subnormals (below 2^-126)
    x[3] = g.standard_normal(H) * np.exp2(g.integers(-40, 41, H))
    x[4, ::97] *= 1e8
    return synth.f32_to_bf16_bits(x)


def test_wide_range_rows_stq_prefill_gemm():
    """Rows of wide dynamic range through the STQ1_0 prefill GEMMs (x scaled per row by a power
    of two into fp16, h as fp16 hi + lo): every row within the tolerance, zero rows exactly
    zero."""
    c = synth.LayerCfg("wide", 160, 512, 256, 8, 2, True, "stq1", False, True, 1, 65)
    inp = layer_inputs(c)
    x = _wide_rows(c.T, c.H, 65)
    d = M.Dims(c.T, c.H, c.I, c.E, c.k)
    routed = M.Experts(M.MOE_W_STQ1_0, *[(dev(cd), dev(sc)) for cd, sc in inp["routed"]])
    shared = bf16_experts(*(dev(w) for w in inp["shared"]))
    bufs = LayerBuffers(d, M.MOE_W_STQ1_0, True)
    M.moe_reset_counters()
    run_layer(d, bufs, dev(x), routed, shared, logits_in=dev(inp["logits_in"]))
    torch.cuda.synchronize()
    assert M.moe_get_counters()["stq_gemm"] == 2
    ref = O.moe_layer(x, c.k, oracle_weights(c, inp["routed"]), "stq1", logits_in=inp["logits_in"],
                      shared=inp["shared"])
    out = host(bufs.out)
    assert (out[1] == 0).all() and np.isfinite(out).all()
    keep = [t for t in range(c.T) if t != 1]
    err = row_err(out[keep], ref["out"][keep])
    yp_err = row_err(host(bufs.y_pairs), ref["y_pairs"])
    say("wide-range rows, STQ1_0 prefill GEMMs: max row err", float(err.max()),
        "rows 0/2/3/4", [float(e) for e in err[[0, 1, 2, 3]]], "y_pairs", float(np.nanmax(yp_err)))
    assert err.max() <= TOL


@pytest.mark.parametrize("T", [1, 4, 7])
def test_wide_range_rows_fused_decode(T):
    """The same rows through the fused decode (bf16 MFMA on x, h as bf16 hi + lo)."""
    c = synth.LayerCfg("wide", T, 512, 256, 16, 4, True, "stq1", False, False, 1, 66)
    inp = layer_inputs(c)
    x = _wide_rows(max(T, 5), c.H, 66)[:T]
    o = _run_fused(c, x, inp["wr"], inp["routed"], inp["shared"])
    ref = O.moe_layer(x, c.k, oracle_weights(c, inp["routed"]), "stq1", wr_bits=inp["wr"],
                      shared=inp["shared"])
    from tests.helpers import near_tie_tokens
    tie = near_tie_tokens(ref["logits"], c.k)
    gi = host(o["ids"])
    assert (gi[~tie] == ref["ids"][~tie]).all()
    out = host(o["out"])
    assert np.isfinite(out).all()
    if T > 1:
        assert (out[1] == 0).all()
    keep = [t for t in range(T) if not tie[t] and not (t == 1)]
    err = row_err(out[keep], ref["out"][keep])
    say("wide-range rows, fused decode T", T, "max row err", float(err.max()), "near-ties", int(tie.sum()))
    assert err.max() <= TOL


# ----------------------------------------------------------------------------- MX encoders
def _encoder_rows():
    """fp32 rows (K = 256, 8 groups each) covering every group exponent the MX rule produces
    (-127 .. 119), E4M3 rounding ties, the saturating band, zeros, -0, tiny values and fp32
    subnormals."""
    g = np.random.default_rng(67)
    rows = []
    for X in range(-127, 120):
        base = 2.0 ** (X + 8)                           # amax in [2^(X+8), 2^(X+9))
        grp = []
        # random magnitudes spread down to 2^-12 of the group max
        v = g.uniform(1, 2, 32) * base * np.exp2(-g.integers(0, 13, 32)) * g.choice([-1, 1], 32)
        v[0] = 1.99 * base
        grp.append(v)
        # exact ties: (n + 1/2) quanta at several binades, with the group max pinned
        q = np.exp2(g.integers(-9, 6, 32)) * 2.0 ** X
        t = (2 * g.integers(4, 15, 32) + 1) * q / 2
        t[0] = 1.5 * base
        grp.append(t * g.choice([-1, 1], 32))
        # saturating band: 448 .. 512 (x 2^X) round or saturate to 448
        s = g.uniform(440, 511.9, 32) * 2.0 ** X
        s[1] = 464 * 2.0 ** X                            # the tie at the top of the grid
        grp.append(s * g.choice([-1, 1], 32))
        # zeros, -0 and values that underflow to zero or to E4M3 subnormals
        z = g.uniform(0, 2 ** -9, 32) * 2.0 ** X * 4
        z[:4] = [0.0, -0.0, 2.0 ** (X - 10), -(2.0 ** (X - 10))]
        z[4] = 1.2 * base
        grp.append(z)
        row = np.concatenate(grp + grp[::-1])
        rows.append(row)
    x = np.array(rows)
    x = np.where(np.abs(x) < 2.0 ** -149, np.copysign(0.0, x), x)
    return x.astype(np.float32)


def test_mx_hw_encoder_equals_integer_rule():
    """The scaled hardware conversion of the MXFP4 gate/up epilogue gives, on every chosen
    value, the codes of the integer rule (moe_mx_quant_act) and of the oracle, bit for bit."""
    x = _encoder_rows()
    R, K = x.shape
    say("mx encoders on", R, "rows of", K, "values, group exponents -127 .. 119")
    rq, rs = O.mx_quantize_e4m3(x.astype(np.float64))
    outs = {}
    for name in ("integer", "hwcvt"):
        q = torch.empty((R, K), dtype=torch.uint8, device="cuda")
        s = torch.empty((R, K // 32), dtype=torch.uint8, device="cuda")
        if name == "integer":
            M.moe_mx_quant_act(R, K, None, dev(x), q, s)
        else:
            M.moe_mx_quant_f32_hwcvt(R, K, dev(x), q, s)
        torch.cuda.synchronize()
        outs[name] = (host(q), host(s))
    scales = sorted(set(rs.ravel().tolist()))
    say("scale bytes covered", scales[0], "..", scales[-1], "(", len(scales), "values )")
    assert scales[0] == 0 and scales[-1] == 246
    for name, (q, s) in outs.items():
        nq = int((q != rq).sum())
        say(name, "codes differing from the oracle:", nq, "of", q.size)
        assert (s == rs).all(), name
        assert nq == 0, name


# ----------------------------------------------------------------------------- scaled MFMA
def _mx_cfg():
    return synth.LayerCfg("mfma", 64, 512, 2048, 4, 2, False, "mxfp4", False, True, 1, 68)


def test_mx_scaled_mfma_accumulation_error():
    """Measure the error of the scaled FP8 x FP4 MFMA on the MXFP4 down projection: the GPU's
    y_pairs against the exact dot products of the GPU's own FP8 h with the E2M1 weights
    (products exact in float64; the float64 sum's error is below 1e-15 of the sum of |terms|).
    Reported relative to sum |terms| and to the row RMS, next to what a sequential fp32 sum
    in K order gives; the bound MFMA_REL_BOUND is asserted."""
    c = _mx_cfg()
    inp = layer_inputs(c)
    d = M.Dims(c.T, c.H, c.I, c.E, c.k)
    for tiled in (False, True):
        fmt = M.MOE_W_MXFP4
        tens = [(dev(cd), dev(sc)) for cd, sc in inp["routed"]]
        if tiled:
            packed = []
            for (cd, sc), (codes, _) in zip(tens, inp["routed"]):
                rows = codes.shape[0] * codes.shape[1]
                tc, ts = torch.empty_like(cd), torch.empty_like(sc)
                M.moe_mxfp4_pack_tiles(cd, sc, rows, 2 * codes.shape[-1], tc, ts)
                packed.append((tc, ts))
            tens, fmt = packed, M.MOE_W_MXFP4_TILED
        routed = M.Experts(fmt, *tens)
        bufs = LayerBuffers(d, M.MOE_W_MXFP4, False)
        run_layer(d, bufs, dev(inp["x"]), routed, None, logits_in=dev(inp["logits_in"]))
        torch.cuda.synchronize()
        offs = M.moe_workspace_offsets(d, M.MOE_W_MXFP4, False)
        ws = host(bufs.ws)
        P, I, H = d.P, c.I, c.H
        hq = ws[offs[4]:offs[4] + P * I].reshape(P, I)
        hs = ws[offs[5]:offs[5] + P * I // 32].reshape(P, I // 32)
        hv = O.mx_dequantize_e4m3(hq, hs)
        off = host(bufs.offsets)
        yp = host(bufs.y_pairs).astype(np.float64)
        get_w = oracle_weights(c, inp["routed"])
        rel, rel_rms, rel32 = [], [], []
        for e in range(c.E):
            lo, hi = int(off[e]), int(off[e + 1])
            if hi == lo:
                continue
            W = get_w(e, 2)                                   # [H, I]
            for pos in range(lo, hi):
                terms = W * hv[pos][None, :]                  # exact products
                exact = terms.sum(axis=1)
                mag = np.abs(terms).sum(axis=1)
                seq32 = np.cumsum(terms.astype(np.float32), axis=1, dtype=np.float32)[:, -1]
                ok = mag > 0
                rel.append(np.abs(yp[pos] - exact)[ok] / mag[ok])
                rel32.append(np.abs(seq32.astype(np.float64) - exact)[ok] / mag[ok])
                rms = math.sqrt(float((exact ** 2).mean()))
                if rms > 0:
                    rel_rms.append(float(np.abs(yp[pos] - exact).max()) / rms)
        rel = np.concatenate(rel)
        rel32 = np.concatenate(rel32)
        say(f"MEASURE scaled-MFMA ({'tiled' if tiled else 'row-major'}) K={I}: error / sum|terms| "
            f"max {rel.max():.3e} (2^{math.log2(rel.max()):.2f}) p99 {np.quantile(rel, 0.99):.3e} "
            f"median {np.median(rel):.3e}; sequential fp32 max {rel32.max():.3e} median {np.median(rel32):.3e}; "
            f"max |err| / row RMS {max(rel_rms):.3e}")
        assert rel.max() <= MFMA_REL_BOUND
