"""GPU parity of every hot-path step against the CPU oracle, through the C ABI.

Bit-exact: STQ1_0 packing and decoding, MXFP4 decoding, MX activation quantisation,
top-k ids and slot order from given logits, the permutation.  Tolerance (max |err| /
RMS of the reference row <= 2e-3): expert outputs and the combined layer output.
Where floating point decides an integer (top-k from x-computed logits, the FP8 codes of
h) near-ties are allowed to differ and are counted instead."""
import math
import sys

import numpy as np
import pytest
import torch

import bit_quantized_moe_softmax_amd as M
import synth
from bit_quantized_moe_softmax_amd.layer import LayerBuffers, bf16_experts, run_layer
from oracle import moe_oracle as O
from tests.helpers import (TOL, layer_inputs, near_tie_tokens, oracle_weights, row_err, shapes,
                           valid_selection)

pytestmark = pytest.mark.gpu


def say(*a):
    print("[gpu-parity]", *a, file=sys.__stderr__, flush=True)


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


def routed_experts(c, routed, tiled=False):
    """Device copies of the routed families; with tiled=True (MXFP4 only) each family is
    repacked on the GPU into the tiled layout and the row-major copy is dropped."""
    fmt = M.MOE_W_STQ1_0 if c.fmt == "stq1" else M.MOE_W_MXFP4
    tens = [(dev(codes), dev(scales)) for codes, scales in routed]
    if tiled:
        assert fmt == M.MOE_W_MXFP4
        out = []
        for (cd, sc), (codes, _) in zip(tens, routed):
            rows = codes.shape[0] * codes.shape[1] if codes.ndim == 3 else codes.shape[0]
            K = 2 * codes.shape[-1]
            tc, ts = torch.empty_like(cd), torch.empty_like(sc)
            M.moe_mxfp4_pack_tiles(cd, sc, rows, K, tc, ts)
            out.append((tc, ts))
        torch.cuda.synchronize()
        return M.Experts(M.MOE_W_MXFP4_TILED, *out)
    return M.Experts(fmt, *tens)


def tiled_reference(codes, scales):
    """The tiled MXFP4 layout by its definition: tile t, K step j, lane l = 16 g + r holds
    row 16 t + r, code bytes 64 j + 16 g .. + 15; the step's scale block holds 4 bytes per row."""
    R, KB = codes.shape
    t, S = R // 16, KB // 64
    tc = codes.reshape(t, 16, S, 4, 16).transpose(0, 2, 3, 1, 4).reshape(-1)
    ts = scales.reshape(t, 16, S, 4).transpose(0, 2, 1, 3).reshape(-1)
    return tc, ts


def shared_experts(shared):
    if shared is None:
        return None
    return bf16_experts(*(dev(w) for w in shared))


# ----------------------------------------------------------------------------- formats
def test_stq1_pack_dequant_bitexact():
    n_blk = 1237
    say("stq1_pack/dequant n_blk", n_blk)
    z, s, d = synth.stq1_pattern_fields(21, 0, 0, 0, n_blk * 64)
    codes_ref, scales_ref = O.stq1_pack(z, s, d)
    codes = torch.empty(n_blk * 40, dtype=torch.uint8, device="cuda")
    scales = torch.empty(n_blk, dtype=torch.int16, device="cuda")
    M.moe_stq1_pack(dev(z), dev(s), dev(d), n_blk, codes, scales)
    assert (host(codes) == codes_ref).all()
    assert (host(scales, np.uint16) == scales_ref).all()
    out = torch.empty(n_blk * 256, dtype=torch.float32, device="cuda")
    M.moe_stq1_dequant(codes, scales, n_blk, out)
    ref = O.stq1_decode(codes_ref, scales_ref).astype(np.float32)
    assert (host(out).view(np.uint32) == ref.view(np.uint32)).all()
    # uniform code bytes of a Hy4-shaped matrix
    codes2, scales2 = synth.stq1_matrix(1, 0, 3, 2, 2048 * 6144)
    nb = scales2.size
    out2 = torch.empty(nb * 256, dtype=torch.float32, device="cuda")
    M.moe_stq1_dequant(dev(codes2), dev(scales2), nb, out2)
    ref2 = O.stq1_decode(codes2, scales2).astype(np.float32)
    assert (host(out2).view(np.uint32) == ref2.view(np.uint32)).all()


def test_mxfp4_dequant_bitexact():
    rows, K = 96, 512
    say("mxfp4_dequant", rows, K)
    codes, scales = synth.mxfp4_matrix(3, 0, 0, 0, rows, K)
    scales = scales.copy()
    scales[0] = np.arange(K // 32, dtype=np.uint8) * 15 + 10     # wide exponent range
    out = torch.empty((rows, K), dtype=torch.float32, device="cuda")
    M.moe_mxfp4_dequant(dev(codes), dev(scales), rows, K, out)
    ref = O.mxfp4_matrix(codes, scales, rows, K).astype(np.float32)
    assert (host(out).view(np.uint32) == ref.view(np.uint32)).all()


@pytest.mark.parametrize("rows,K", [(48, 384), (2048 * 3, 6144), (6144, 2048)])
def test_mxfp4_pack_tiles_bitexact(rows, K):
    say("mxfp4_pack_tiles", rows, K)
    g = np.random.default_rng(rows + K)
    codes = g.integers(0, 256, size=(rows, K // 2), dtype=np.uint8)
    scales = g.integers(0, 256, size=(rows, K // 32), dtype=np.uint8)
    tc = torch.empty(rows * K // 2, dtype=torch.uint8, device="cuda")
    ts = torch.empty(rows * K // 32, dtype=torch.uint8, device="cuda")
    M.moe_mxfp4_pack_tiles(dev(codes), dev(scales), rows, K, tc, ts)
    rc, rs = tiled_reference(codes, scales)
    assert (host(tc) == rc).all() and (host(ts) == rs).all()
    # lane 17 of tile 0, step 1: row 1, code bytes 64 + 16 .. 64 + 31
    if K >= 256:
        assert (host(tc)[1024 + 16 * 17:1024 + 16 * 18] == codes[1, 80:96]).all()


def _mx_case_rows(K):
    g = np.random.default_rng(7)
    x = synth.activations(3, 0, 40, K).astype(np.uint16)
    rows = [x]
    e = np.zeros((8, K), dtype=np.float32)
    e[0] = 0.0                                           # amax 0
    e[1] = g.standard_normal(K) * 1e-30                  # tiny, bf16 subnormal range
    e[2] = g.standard_normal(K) * 3e30                   # huge
    e[3] = np.where(np.arange(K) % 2 == 0, 256.0, -17.0)  # exact ties after scaling
    e[4] = g.integers(-512, 512, K).astype(np.float32) / 64.0
    e[5] = -np.abs(g.standard_normal(K)) * 1e-3
    e[6, ::32] = 1.0
    e[7] = g.standard_normal(K) * 448.0
    rows.append(synth.f32_to_bf16_bits(e))
    return np.concatenate(rows)


def test_mx_quant_act_bitexact_bf16_and_f32():
    K = 512
    xb = _mx_case_rows(K)
    say("mx_quant_act bf16 rows", xb.shape)
    q = torch.empty(xb.shape, dtype=torch.uint8, device="cuda")
    s = torch.empty((xb.shape[0], K // 32), dtype=torch.uint8, device="cuda")
    M.moe_mx_quant_act(xb.shape[0], K, dev(xb), None, q, s)
    rq, rs = O.mx_quantize_e4m3(O.bf16_to_f64(xb))
    assert (host(s) == rs).all()
    assert (host(q) == rq).all()
    g = np.random.default_rng(8)
    xf = (g.standard_normal((33, K)) * np.exp(g.uniform(-20, 20, (33, 1)))).astype(np.float32)
    xf[0, :5] = [1e-40, -1e-41, 0.0, -0.0, 3e-39]            # fp32 subnormals
    say("mx_quant_act f32 rows", xf.shape)
    q2 = torch.empty(xf.shape, dtype=torch.uint8, device="cuda")
    s2 = torch.empty((xf.shape[0], K // 32), dtype=torch.uint8, device="cuda")
    M.moe_mx_quant_act(xf.shape[0], K, None, dev(xf), q2, s2)
    rq2, rs2 = O.mx_quantize_e4m3(xf.astype(np.float64))
    assert (host(s2) == rs2).all()
    assert (host(q2) == rq2).all()


# ----------------------------------------------------------------------------- routing
@pytest.mark.parametrize("T,E,k", [(37, 256, 8), (5, 8, 2), (3, 1024, 32), (9, 64, 64 // 2), (1, 7, 7)])
def test_topk_from_logits_bitexact(T, E, k):
    say("topk", T, E, k)
    g = np.random.default_rng(T * 1000 + E)
    logits = g.standard_normal((T, E)).astype(np.float32)
    logits[0] = np.round(logits[0] * 2) / 2                  # many exact ties
    bias = (g.standard_normal(E) * 0.1).astype(np.float32) if T % 2 else None
    d = M.Dims(T, 32, 32, E, k)
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    lo = torch.empty((T, E), dtype=torch.float32, device="cuda")
    M.moe_route(d, None, None, dev(bias) if bias is not None else None, dev(logits), lo, ids, w)
    # the biased logits are fp32 sums; the oracle takes that same fp32 value
    lref = logits if bias is None else (logits + bias[None, :]).astype(np.float32)
    assert (host(lo) == lref).all()
    _, rid, rw = O.route(k, logits_in=lref.astype(np.float64))
    assert (host(ids) == rid).all()
    assert np.allclose(host(w), rw, rtol=1e-6, atol=0)


def test_route_from_x():
    c = synth.cfg(2)
    T = 70
    say("route gemv T", T)
    x = synth.activations(5, 0, T, c.H)
    wr = synth.router_weights(5, 0, c.E, c.H)
    bias = synth.zipf_bias(5, 0, c.E)
    d = M.Dims(T, c.H, c.I, c.E, c.k)
    ids = torch.empty((T, c.k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, c.k), dtype=torch.float32, device="cuda")
    lo = torch.empty((T, c.E), dtype=torch.float32, device="cuda")
    M.moe_route(d, dev(x), dev(wr), dev(bias), None, lo, ids, w)
    rl, rid, rw = O.route(c.k, x, wr, bias)
    assert np.abs(host(lo) - rl).max() < 2e-5
    tie = near_tie_tokens(rl, c.k)
    gi = host(ids)
    assert (gi[~tie] == rid[~tie]).all()
    for t in np.flatnonzero(tie):
        assert valid_selection(rl[t], gi[t], c.k)
    say("near-tie tokens", int(tie.sum()), "of", T)
    ok = ~tie
    assert np.allclose(host(w)[ok], rw[ok], rtol=2e-5, atol=1e-7)


# from 8192 pairs (and chunks of 1024 x E <= pairs) the permutation runs chunk-parallel:
# 4096 x 8, 4100 x 8 (a ragged last chunk, Zipf load) and 8192 x 1 take that path, 1100 x 8
# with E = 1024 (9 chunks x 1024 > 8800 pairs) the single-workgroup one
@pytest.mark.parametrize("T,k,E,mode", [(1, 8, 256, "rand"), (7, 2, 8, "rand"), (64, 8, 256, "zipf"),
                                        (4096, 8, 256, "rand"), (300, 3, 4, "rand"),
                                        (129, 8, 256, "one"), (50, 1, 1024, "rand"),
                                        (4100, 8, 512, "zipf"), (8192, 1, 8, "rand"),
                                        (1100, 8, 1024, "rand")])
def test_permute_bitexact(T, k, E, mode):
    say("permute", T, k, E, mode)
    g = np.random.default_rng(T + k + E)
    if mode == "one":
        ids = np.stack([np.r_[5, g.choice(np.r_[0:5, 6:E], k - 1, replace=False)] for _ in range(T)])
    elif mode == "zipf":
        p = 1.0 / np.arange(1, E + 1) ** 1.1
        ids = np.stack([g.choice(E, k, replace=False, p=p / p.sum()) for _ in range(T)])
    else:
        ids = np.stack([g.choice(E, k, replace=False) for _ in range(T)])
    ids = ids.astype(np.int32)
    d = M.Dims(T, 32, 32, E, k)
    sp = torch.empty(T * k, dtype=torch.int32, device="cuda")
    off = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    pp = torch.empty(T * k, dtype=torch.int32, device="cuda")
    M.moe_permute(d, dev(ids), sp, off, pp)
    rsp, roff, rpp = O.permute(ids, E)
    assert (host(sp) == rsp).all() and (host(off) == roff).all() and (host(pp) == rpp).all()


# ----------------------------------------------------------------------------- whole layers
SMALL = {
    "cfg0": synth.cfg(0),
    "h512-i256-e8-top2-t37-shared": synth.LayerCfg("t", 37, 512, 256, 8, 2, True, "stq1", False, False, 1, 11),
    "h768-i512-e16-top4-t21-zipf": synth.LayerCfg("t", 21, 768, 512, 16, 4, True, "stq1", True, False, 1, 12),
}


def _check_layer(c, inp, bufs, d, ref, sample=None):
    gi = host(bufs.topk_ids)
    tie = near_tie_tokens(ref["logits"], c.k)
    assert (gi[~tie] == ref["ids"][~tie]).all()
    toks = np.arange(c.T) if sample is None else np.asarray(sample)
    out = host(bufs.out)
    if tie.any():
        say("near-tie tokens", np.flatnonzero(tie))
    keep = [t for t in toks if not tie[t]]
    err = row_err(out[keep], ref["out"][keep])
    say("layer max row err", float(err.max()))
    assert err.max() <= TOL
    return err


@pytest.mark.parametrize("name", list(SMALL))
def test_layer_stq_small(name):
    c = SMALL[name]
    say("layer", name)
    inp = layer_inputs(c)
    d = M.Dims(c.T, c.H, c.I, c.E, c.k)
    routed = routed_experts(c, inp["routed"])
    shared = shared_experts(inp["shared"])
    bufs = LayerBuffers(d, M.MOE_W_STQ1_0, shared is not None)
    bias = dev(inp["bias"]) if inp["bias"] is not None else None
    M.moe_reset_counters()
    run_layer(d, bufs, dev(inp["x"]), routed, shared, wr_bf16=dev(inp["wr"]), logit_bias=bias)
    torch.cuda.synchronize()
    ref = O.moe_layer(inp["x"], c.k, oracle_weights(c, inp["routed"]), "stq1", wr_bits=inp["wr"],
                      bias=inp["bias"], shared=inp["shared"])
    _check_layer(c, inp, bufs, d, ref)
    cnt = M.moe_get_counters()
    if c.H % 256 == 0:
        assert cnt["stq_gateup_mfma"] == 1
    if c.I % 256 == 0:
        assert cnt["stq_down_mfma"] == 1
    # per-stage: h and y_pairs of the pairs
    yp = host(bufs.y_pairs)
    if (host(bufs.topk_ids) == ref["ids"]).all():
        assert row_err(yp, ref["y_pairs"]).max() <= TOL
        if shared is not None:
            assert row_err(host(bufs.y_shared), ref["y_shared"]).max() <= TOL


STQ_PREFILL = {
    # about 75 pairs per expert (one ragged M block each); shared expert in three M blocks
    "h512-i256-e8-top2-t300-shared": synth.LayerCfg("p", 300, 512, 256, 8, 2, True, "stq1", False, False, 1, 21),
    # Zipf-skewed load: a few experts with several M blocks; down output in three N tiles
    "h768-i512-e4-top2-t400-zipf": synth.LayerCfg("p", 400, 768, 512, 4, 2, True, "stq1", True, False, 1, 22),
    # a few pairs per expert, idle experts, given logits, no shared expert
    "h256-i256-e64-top4-t128-logits": synth.LayerCfg("p", 128, 256, 256, 64, 4, False, "stq1", False, True, 1, 23),
    # routed experts on the GEMMs, the shared expert (under 256 tokens) on the decode kernels
    "h512-i256-e8-top2-t150-shared": synth.LayerCfg("p", 150, 512, 256, 8, 2, True, "stq1", False, False, 1, 24),
}


@pytest.mark.parametrize("name", list(STQ_PREFILL))
def test_layer_stq_prefill_gemm(name):
    """STQ1_0 routed experts and the bf16 shared expert at prefill token counts: the tiled
    grouped GEMMs (fp16 / bf16 MFMA) against the float64 oracle, stage by stage."""
    c = STQ_PREFILL[name]
    say("stq prefill layer", name)
    inp = layer_inputs(c)
    d = M.Dims(c.T, c.H, c.I, c.E, c.k)
    routed = routed_experts(c, inp["routed"])
    shared = shared_experts(inp["shared"])
    bufs = LayerBuffers(d, M.MOE_W_STQ1_0, shared is not None)
    M.moe_reset_counters()
    if c.logits_given:
        run_layer(d, bufs, dev(inp["x"]), routed, shared, logits_in=dev(inp["logits_in"]))
        ref = O.moe_layer(inp["x"], c.k, oracle_weights(c, inp["routed"]), "stq1",
                          logits_in=inp["logits_in"], shared=inp["shared"])
    else:
        bias = dev(inp["bias"]) if inp["bias"] is not None else None
        run_layer(d, bufs, dev(inp["x"]), routed, shared, wr_bf16=dev(inp["wr"]), logit_bias=bias)
        ref = O.moe_layer(inp["x"], c.k, oracle_weights(c, inp["routed"]), "stq1", wr_bits=inp["wr"],
                          bias=inp["bias"], shared=inp["shared"])
    torch.cuda.synchronize()
    cnt = M.moe_get_counters()
    assert cnt["stq_gemm"] == 2 and cnt["stq_gateup_mfma"] == 0 and cnt["stq_down_mfma"] == 0
    sh_gemm = shared is not None and c.T >= 256      # the shared expert's GEMMs start at 256 tokens
    assert cnt["bf16_gemm"] == (2 if sh_gemm else 0)
    assert cnt["bf16_gateup"] == (1 if shared is not None and not sh_gemm else 0)
    _check_layer(c, inp, bufs, d, ref)
    if (host(bufs.topk_ids) == ref["ids"]).all():
        offs = M.moe_workspace_offsets(d, M.MOE_W_STQ1_0, shared is not None)
        h = host(bufs.ws)[offs[0]:offs[0] + d.P * c.I * 4].view(np.float32).reshape(d.P, c.I)
        eh = row_err(h, ref["h"]).max()
        ey = row_err(host(bufs.y_pairs), ref["y_pairs"]).max()
        say("h max row err", float(eh), "y_pairs max row err", float(ey))
        assert eh <= TOL and ey <= TOL
        if shared is not None:
            es = row_err(host(bufs.y_shared), ref["y_shared"]).max()
            say("y_shared max row err", float(es))
            assert es <= TOL


def _stq_rows(codes_e, scales_e, K, rows):
    """Rows `rows` of one STQ1_0 matrix with K columns (each row is K/256 whole blocks)."""
    nb = K // 256
    c = np.concatenate([codes_e[r * nb * 40:(r + 1) * nb * 40] for r in rows])
    sc = np.concatenate([scales_e[r * nb:(r + 1) * nb] for r in rows])
    return O.stq1_decode(c, sc).reshape(len(rows), K)


def _mx_rows(codes_e, scales_e, K, rows):
    """Rows `rows` of one row-major MXFP4 matrix with K columns."""
    rows = np.asarray(rows)
    return O.mxfp4_matrix(codes_e[rows], scales_e[rows], len(rows), K)


def _expert_samples(c, off, seed):
    """For every expert with pairs: its first and last pair (the first and last M block of a
    split expert), two h groups of 32 columns from different gate/up N tiles (128 columns
    each), and one output row from each down N tile (256 rows each)."""
    g = np.random.default_rng(seed)
    out = []
    n_ht = c.I // 128
    for e in range(c.E):
        lo, hi = int(off[e]), int(off[e + 1])
        if hi == lo:
            continue
        poss = sorted({lo, hi - 1})
        t0, t1 = g.choice(n_ht, 2, replace=False) if n_ht > 1 else (0, 0)
        grp = [4 * t0 + int(g.integers(4)), 4 * t1 + int(g.integers(4))]
        if grp[0] == grp[1]:
            grp[1] = (grp[1] + 1) % (c.I // 32)
        hcols = np.concatenate([np.arange(32 * q, 32 * q + 32) for q in grp])
        orow = np.array([256 * t + int(g.integers(256)) for t in range(c.H // 256)])
        out.append((e, poss, grp, hcols, orow))
    return out


def _sampled_err(got, ref):
    """max |got - ref| / RMS(ref) over a sample of one row's entries."""
    ref = np.asarray(ref, dtype=np.float64)
    rms = math.sqrt(float((ref * ref).mean()))
    return float(np.abs(np.asarray(got, dtype=np.float64) - ref).max()) / max(rms, 1e-300)


def test_stq_prefill_hy4_t4096_sampled():
    """Hy4-shaped STQ1_0 layer at 4096 tokens (256 experts, top-8, bf16 shared expert) on the
    prefill GEMMs: routing and permutation in full; on EVERY expert, the first and last pair
    (both M blocks of a split expert): h on two 32-column groups from different N tiles
    against the oracle, and the down projection of the GPU's h on one output row per N tile;
    the combined output of sampled tokens against the oracle's own layer (its h, its y_pairs,
    its shared expert)."""
    c = synth.LayerCfg("hy4-stq1-prefill-t4096", 4096, 6144, 2048, 256, 8, True, "stq1", False, True, 1, 31)
    say("stq prefill t4096 generate")
    inp = layer_inputs(c)
    d = M.Dims(c.T, c.H, c.I, c.E, c.k)
    routed = routed_experts(c, inp["routed"])
    shared = shared_experts(inp["shared"])
    bufs = LayerBuffers(d, M.MOE_W_STQ1_0, True)
    say("stq prefill t4096 run")
    M.moe_reset_counters()
    run_layer(d, bufs, dev(inp["x"]), routed, shared, logits_in=dev(inp["logits_in"]))
    torch.cuda.synchronize()
    cnt = M.moe_get_counters()
    assert cnt["stq_gemm"] == 2 and cnt["bf16_gemm"] == 2
    _, rid, rw = O.route(c.k, logits_in=inp["logits_in"])
    rsp, roff, rpp = O.permute(rid, c.E)
    assert (host(bufs.sorted_pair) == rsp).all() and (host(bufs.offsets) == roff).all()
    assert (host(bufs.pair_pos) == rpp).all()
    offs = M.moe_workspace_offsets(d, M.MOE_W_STQ1_0, True)
    P = d.P
    h_gpu = host(bufs.ws[offs[0]:offs[0] + P * c.I * 4]).view(np.float32).reshape(P, c.I)
    yp = host(bufs.y_pairs)
    xf = O.bf16_to_f64(inp["x"])
    (gc, gs), (uc, us), (dc, ds) = inp["routed"]
    worst_h = worst_y = 0.0
    samples = _expert_samples(c, roff, 131)
    for e, poss, grp, hcols, orow in samples:
        a = xf[rsp[poss] // c.k]
        h = O.silu(a @ _stq_rows(gc[e], gs[e], c.H, hcols).T) * (a @ _stq_rows(uc[e], us[e], c.H, hcols).T)
        Wd = _stq_rows(dc[e], ds[e], c.I, orow)
        for i, pos in enumerate(poss):
            worst_h = max(worst_h, _sampled_err(h_gpu[pos, hcols], h[i]))
            worst_y = max(worst_y, _sampled_err(yp[pos, orow], Wd @ h_gpu[pos].astype(np.float64)))
    say("stq prefill t4096:", len(samples), "experts checked, h max err", worst_h, "down max err", worst_y)
    assert len(samples) == int((np.diff(roff) > 0).sum())
    assert worst_h <= TOL and worst_y <= TOL
    # two sampled tokens through the oracle's own layer (independent of every GPU stage)
    toks = synth.sample_tokens(c.seed, c.T, 2)
    get_w = oracle_weights(c, inp["routed"])
    ysh = O.shared_expert(inp["x"][toks], *inp["shared"])
    assert row_err(host(bufs.y_shared)[toks], ysh).max() <= TOL
    out_ref = ysh.copy()
    for i, t in enumerate(toks):
        for j in range(c.k):
            e = int(rid[t, j])
            _, y = O.swiglu_expert(xf[t:t + 1], get_w(e, 0), get_w(e, 1), get_w(e, 2))
            out_ref[i] += rw[t, j] * y[0]
    err = row_err(host(bufs.out)[toks], out_ref)
    say("stq prefill t4096 combined output vs the oracle's layer on tokens", list(toks), float(err.max()))
    assert err.max() <= TOL


def test_layer_cfg1_hy4_decode():
    c = synth.cfg(1)
    say("layer cfg1 generate")
    inp = layer_inputs(c)
    d = M.Dims(c.T, c.H, c.I, c.E, c.k)
    routed = routed_experts(c, inp["routed"])
    shared = shared_experts(inp["shared"])
    bufs = LayerBuffers(d, M.MOE_W_STQ1_0, True)
    say("layer cfg1 run")
    run_layer(d, bufs, dev(inp["x"]), routed, shared, wr_bf16=dev(inp["wr"]))
    torch.cuda.synchronize()
    say("layer cfg1 oracle")
    ref = O.moe_layer(inp["x"], c.k, oracle_weights(c, inp["routed"]), "stq1", wr_bits=inp["wr"],
                      shared=inp["shared"])
    _check_layer(c, inp, bufs, d, ref)
    assert row_err(host(bufs.y_pairs), ref["y_pairs"]).max() <= TOL
    assert row_err(host(bufs.y_shared), ref["y_shared"]).max() <= TOL


def test_layer_cfg2_hy4_decode_zipf_sampled():
    c = synth.cfg(2)
    say("layer cfg2 generate")
    inp = layer_inputs(c)
    d = M.Dims(c.T, c.H, c.I, c.E, c.k)
    routed = routed_experts(c, inp["routed"])
    shared = shared_experts(inp["shared"])
    bufs = LayerBuffers(d, M.MOE_W_STQ1_0, True)
    say("layer cfg2 run")
    run_layer(d, bufs, dev(inp["x"]), routed, shared, wr_bf16=dev(inp["wr"]),
              logit_bias=dev(inp["bias"]))
    torch.cuda.synchronize()
    # routing of every token, then the full layer for a sample of tokens
    rl, rid, rw = O.route(c.k, inp["x"], inp["wr"], inp["bias"])
    tie = near_tie_tokens(rl, c.k)
    gi = host(bufs.topk_ids)
    assert (gi[~tie] == rid[~tie]).all()
    sample = [t for t in synth.sample_tokens(c.seed, c.T, 6) if not tie[t]]
    say("layer cfg2 oracle tokens", sample, "unique experts", len(np.unique(rid)))
    get_w = oracle_weights(c, inp["routed"])
    ref = O.moe_layer(inp["x"][sample], c.k, get_w, "stq1", wr_bits=inp["wr"], bias=inp["bias"],
                      shared=inp["shared"])
    err = row_err(host(bufs.out)[sample], ref["out"])
    say("cfg2 sampled max row err", float(err.max()))
    assert err.max() <= TOL


MX_SMALL = synth.LayerCfg("mx", 150, 512, 256, 8, 2, True, "mxfp4", False, True, 1, 13)


# FP8 requantisation of h (R11 stage ii): codes of h may differ from the oracle's by one E4M3
# step where the scaled MFMA's reduced-precision sums (about 2^-16 of the sum of |products|,
# measured by test_mx_scaled_mfma_accumulation_error) move a value across a rounding
# boundary.  Measured rates, on samples of 32768 .. 307200 codes: 3.1e-4 .. 4.9e-4.  The
# budget is twice the largest, plus a Poisson margin (three standard deviations and two codes)
# so that configs with a few thousand codes do not fail on counting noise.
MX_FLIP_RATE = 1e-3


def _mx_flip_budget(n_tot):
    mean = MX_FLIP_RATE * n_tot
    return mean + 3.0 * math.sqrt(mean) + 2.0


def _mx_flip_count(hq, hs, hq_ref, hs_ref):
    """Codes of h that differ from the oracle's; each must stay within one E4M3 step of the
    oracle's value (a flip at a rounding boundary, or an amax on either side of a power of
    two)."""
    diff = hq != hq_ref
    if diff.any():
        vg = O.mx_dequantize_e4m3(hq, hs)
        vr = O.mx_dequantize_e4m3(hq_ref, hs_ref)
        step = np.abs(vr) * 2.0 ** -3 + O.ue8m0_value(hs_ref).repeat(32, axis=1) * 2.0 ** -9
        assert (np.abs(vg - vr)[diff] <= step[diff] * 1.0001).all()
    return int(diff.sum())


def _mx_h_down_check(c, get_w, a, hq, hs, yp, sp, off, experts):
    """h codes of the pairs the GPU routed against the oracle's MX quantisation of
    SiLU(x W_g^T) * (x W_u^T) (a = dequantised E4M3 x), and the down projection fed the GPU's
    FP8 h.  A code may flip where the GPU's fp32 h and the oracle's float64 h fall on either
    side of an E4M3 rounding boundary: flips are counted and must stay one step wide."""
    n_flip = n_tot = 0
    worst = 0.0
    for e in experts:
        lo, hi = int(off[e]), int(off[e + 1])
        if hi == lo:
            continue
        toks = sp[lo:hi] // c.k
        g = a[toks] @ get_w(e, 0).T
        u = a[toks] @ get_w(e, 1).T
        h = O.silu(g) * u
        hq_ref, hs_ref = O.mx_quantize_e4m3(h)
        n_flip += _mx_flip_count(hq[lo:hi], hs[lo:hi], hq_ref, hs_ref)
        n_tot += hq_ref.size
        y_ref = O.mx_dequantize_e4m3(hq[lo:hi], hs[lo:hi]) @ get_w(e, 2).T
        worst = max(worst, float(row_err(yp[lo:hi], y_ref).max()))
    say(f"mx h code flips {n_flip} of {n_tot} (rate {n_flip / max(1, n_tot):.2e}, budget "
        f"{MX_FLIP_RATE:.1e}), down-stage max row err {worst:.3e}")
    assert n_flip <= _mx_flip_budget(n_tot)
    assert worst <= TOL


def _mx_stage_check(c, inp, bufs, d, experts_check=None):
    offs = M.moe_workspace_offsets(d, M.MOE_W_MXFP4, bool(c.shared))
    ws = host(bufs.ws)
    T, H, I, P = c.T, c.H, c.I, c.T * c.k
    xq = ws[offs[2]:offs[2] + T * H].reshape(T, H)
    xs = ws[offs[3]:offs[3] + T * H // 32].reshape(T, H // 32)
    rq, rs = O.mx_quantize_e4m3(O.bf16_to_f64(inp["x"]))
    assert (xq == rq).all() and (xs == rs).all()
    hq = ws[offs[4]:offs[4] + P * I].reshape(P, I)
    hs = ws[offs[5]:offs[5] + P * I // 32].reshape(P, I // 32)
    # reference h from the oracle's pieces on the pairs the GPU routed
    sp = host(bufs.sorted_pair)
    off = host(bufs.offsets)
    _, rid, _ = O.route(c.k, logits_in=inp["logits_in"])
    assert (host(bufs.topk_ids) == rid).all()
    get_w = oracle_weights(c, inp["routed"])
    a = O.mx_dequantize_e4m3(rq, rs)
    experts = range(c.E) if experts_check is None else experts_check
    _mx_h_down_check(c, get_w, a, hq, hs, host(bufs.y_pairs), sp, off, experts)


MX_MORE = {
    # about 300 pairs per expert: three M blocks each
    "h512-i256-e4-top2-t600": synth.LayerCfg("mx", 600, 512, 256, 4, 2, True, "mxfp4", False, True, 1, 17),
    # most experts idle, ragged blocks of one to two pairs
    "h512-i384-e64-top2-t3": synth.LayerCfg("mx", 3, 512, 384, 64, 2, False, "mxfp4", False, True, 1, 18),
    # wide down projection with a partial last N tile (H = 640 = 2.5 tiles of 256)
    "h640-i256-e8-top2-t70": synth.LayerCfg("mx", 70, 640, 256, 8, 2, False, "mxfp4", False, True, 1, 19),
}


@pytest.mark.parametrize("tiled", [False, True], ids=["rowmajor", "tiled"])
@pytest.mark.parametrize("name", list(MX_MORE))
def test_mx_layer_blocks_and_tails(name, tiled):
    c = MX_MORE[name]
    say("mx layer", name, "tiled" if tiled else "row-major")
    inp = layer_inputs(c)
    d = M.Dims(c.T, c.H, c.I, c.E, c.k)
    routed = routed_experts(c, inp["routed"], tiled)
    shared = shared_experts(inp["shared"])
    bufs = LayerBuffers(d, M.MOE_W_MXFP4, shared is not None)
    run_layer(d, bufs, dev(inp["x"]), routed, shared, logits_in=dev(inp["logits_in"]))
    torch.cuda.synchronize()
    _mx_stage_check(c, inp, bufs, d)


def test_mx_layer_cfg3_hy4_prefill_sampled():
    """Full-size MXFP4 prefill (4096 tokens, 256 experts, top-8): routing, permutation and
    activation quantisation in full; on EVERY expert, the first and last pair (both M blocks
    of a split expert): h codes on two 32-column groups from different N tiles by the
    stage-(ii) rule, and the down projection of the GPU's FP8 h on one output row per N tile;
    the shared expert and the combined output of sampled tokens against the oracle's y_pairs
    (the oracle's down projection of the GPU's FP8 h, whole rows)."""
    c = synth.cfg(3)
    say("mx cfg3 generate")
    inp = layer_inputs(c)
    d = M.Dims(c.T, c.H, c.I, c.E, c.k)
    routed = routed_experts(c, inp["routed"], tiled=True)   # the layout the prefill timing uses
    shared = shared_experts(inp["shared"])
    bufs = LayerBuffers(d, M.MOE_W_MXFP4, True)
    say("mx cfg3 run")
    run_layer(d, bufs, dev(inp["x"]), routed, shared, logits_in=dev(inp["logits_in"]))
    torch.cuda.synchronize()
    _, rid, rw = O.route(c.k, logits_in=inp["logits_in"])
    rsp, roff, rpp = O.permute(rid, c.E)
    assert (host(bufs.sorted_pair) == rsp).all() and (host(bufs.offsets) == roff).all()
    assert (host(bufs.pair_pos) == rpp).all()
    offs = M.moe_workspace_offsets(d, M.MOE_W_MXFP4, True)
    ws = host(bufs.ws)
    T, H, I, P = c.T, c.H, c.I, d.P
    xq = ws[offs[2]:offs[2] + T * H].reshape(T, H)
    xs = ws[offs[3]:offs[3] + T * H // 32].reshape(T, H // 32)
    rq, rs = O.mx_quantize_e4m3(O.bf16_to_f64(inp["x"]))
    assert (xq == rq).all() and (xs == rs).all()
    hq = ws[offs[4]:offs[4] + P * I].reshape(P, I)
    hs = ws[offs[5]:offs[5] + P * I // 32].reshape(P, I // 32)
    a = O.mx_dequantize_e4m3(rq, rs)
    yp = host(bufs.y_pairs)
    (gc, gs), (uc, us), (dc, ds) = inp["routed"]
    n_flip = n_tot = 0
    worst_y = 0.0
    samples = _expert_samples(c, roff, 133)
    for e, poss, grp, hcols, orow in samples:
        at = a[rsp[poss] // c.k]
        h = O.silu(at @ _mx_rows(gc[e], gs[e], H, hcols).T) * (at @ _mx_rows(uc[e], us[e], H, hcols).T)
        hq_ref, hs_ref = O.mx_quantize_e4m3(h)
        hq_g = hq[poss][:, hcols]
        hs_g = hs[poss][:, grp]
        n_flip += _mx_flip_count(hq_g, hs_g, hq_ref, hs_ref)
        n_tot += hq_g.size
        hv = O.mx_dequantize_e4m3(hq[poss], hs[poss])
        Wd = _mx_rows(dc[e], ds[e], I, orow)
        for i, pos in enumerate(poss):
            worst_y = max(worst_y, _sampled_err(yp[pos, orow], Wd @ hv[i]))
    rate = n_flip / max(1, n_tot)
    say(f"mx cfg3: {len(samples)} experts checked; h code flips {n_flip} of {n_tot} "
        f"(rate {rate:.2e}, budget {MX_FLIP_RATE:.1e}); down-stage max err {worst_y:.3e}")
    assert len(samples) == int((np.diff(roff) > 0).sum())
    assert n_flip <= _mx_flip_budget(n_tot)
    assert worst_y <= TOL
    toks = synth.sample_tokens(c.seed, c.T, 3)
    ysh = O.shared_expert(inp["x"][toks], *inp["shared"])
    assert row_err(host(bufs.y_shared)[toks], ysh).max() <= TOL
    get_w = oracle_weights(c, inp["routed"])
    hv_all = {}
    out_ref = ysh.copy()
    for i, t in enumerate(toks):
        for j in range(c.k):
            pos = int(rpp[t * c.k + j])
            e = int(rid[t, j])
            y = O.mx_dequantize_e4m3(hq[pos:pos + 1], hs[pos:pos + 1]) @ get_w(e, 2).T
            out_ref[i] += rw[t, j] * y[0]
    err = row_err(host(bufs.out)[toks], out_ref)
    say("mx cfg3 combined output vs the oracle's y_pairs on tokens", list(toks), float(err.max()))
    assert err.max() <= TOL


@pytest.mark.parametrize("tiled", [False, True], ids=["rowmajor", "tiled"])
def test_mx_layer_small_stages(tiled):
    c = MX_SMALL
    say("mx layer small", "tiled" if tiled else "row-major")
    inp = layer_inputs(c)
    d = M.Dims(c.T, c.H, c.I, c.E, c.k)
    routed = routed_experts(c, inp["routed"], tiled)
    shared = shared_experts(inp["shared"])
    bufs = LayerBuffers(d, M.MOE_W_MXFP4, True)
    run_layer(d, bufs, dev(inp["x"]), routed, shared, logits_in=dev(inp["logits_in"]))
    torch.cuda.synchronize()
    _mx_stage_check(c, inp, bufs, d)
    ref = O.moe_layer(inp["x"], c.k, oracle_weights(c, inp["routed"]), "mxfp4",
                      logits_in=inp["logits_in"], shared=inp["shared"])
    assert row_err(host(bufs.y_shared), ref["y_shared"]).max() <= TOL
    say("mx end-to-end max row err (reported, FP8 re-quantisation of h is discontinuous)",
        float(row_err(host(bufs.out), ref["out"]).max()))


# ----------------------------------------------------------------------------- fused decode layer
FUSED = {
    "h512-i256-e8-top2-t37-shared": synth.LayerCfg("t", 37, 512, 256, 8, 2, True, "stq1", False, False, 1, 11),
    "h1024-i512-e16-top4-t21-zipf": synth.LayerCfg("t", 21, 1024, 512, 16, 4, True, "stq1", True, False, 1, 14),
    "h512-i256-e40-top8-t64-noshared": synth.LayerCfg("t", 64, 512, 256, 40, 8, False, "stq1", True, False, 1, 15),
    # beyond 4 tokens: every expert takes all 64 tokens (four full units each, two 8-pair
    # halves per unit in the down items; four shared token tiles); the smallest large batch;
    # two token tiles, the second of one token
    "h512-i256-e4-top4-t64-shared": synth.LayerCfg("t", 64, 512, 256, 4, 4, True, "stq1", False, False, 1, 17),
    "h512-i256-e16-top8-t5-shared": synth.LayerCfg("t", 5, 512, 256, 16, 8, True, "stq1", False, False, 1, 18),
    "h2048-i1024-e16-top4-t17-zipf": synth.LayerCfg("t", 17, 2048, 1024, 16, 4, True, "stq1", True, False, 1, 19),
    # the widest supported H beyond 4 tokens (gate/up workgroups of 4 waves: 8 x rows of
    # 16 KB and 8 waves' code staging would not fit the LDS together)
    "h8192-i2048-e8-top2-t9-shared": synth.LayerCfg("t", 9, 8192, 2048, 8, 2, True, "stq1", False, False, 1, 20),
    "h512-i256-e8-top2-t1-shared": synth.LayerCfg("t", 1, 512, 256, 8, 2, True, "stq1", False, False, 1, 16),
    # 2..4 tokens: the per-workgroup routing path, experts shared by several tokens
    "h512-i256-e8-top2-t4-shared": synth.LayerCfg("t", 4, 512, 256, 8, 2, True, "stq1", False, False, 1, 23),
    "h1024-i512-e16-top4-t3-zipf": synth.LayerCfg("t", 3, 1024, 512, 16, 4, True, "stq1", True, False, 1, 24),
    "h512-i256-e4-top4-t2-noshared": synth.LayerCfg("t", 2, 512, 256, 4, 4, False, "stq1", False, False, 1, 25),
    "h512-i256-e64-top32-t4-shared": synth.LayerCfg("t", 4, 512, 256, 64, 32, True, "stq1", False, False, 1, 26),
    # one token at H a multiple of 2048: the K-quarter table path of the gate/up kernel
    "h2048-i1024-e16-top4-t1-shared": synth.LayerCfg("t", 1, 2048, 1024, 16, 4, True, "stq1", False, False, 1, 27),
    "h4096-i2048-e32-top8-t1-zipf-noshared": synth.LayerCfg("t", 1, 4096, 2048, 32, 8, False, "stq1", True, False, 1, 28),
}


def run_fused(c, inp, residual=None, with_bf16=False, ws=None, tiled=False):
    d = M.Dims(c.T, c.H, c.I, c.E, c.k)
    routed = routed_experts(c, inp["routed"], tiled)
    shared = shared_experts(inp["shared"])
    f32, i32 = torch.float32, torch.int32
    o = dict(logits=torch.empty((c.T, c.E), dtype=f32, device="cuda"),
             ids=torch.empty((c.T, c.k), dtype=i32, device="cuda"),
             w=torch.empty((c.T, c.k), dtype=f32, device="cuda"),
             sp=torch.empty(d.P, dtype=i32, device="cuda"),
             off=torch.empty(c.E + 1, dtype=i32, device="cuda"),
             pp=torch.empty(d.P, dtype=i32, device="cuda"),
             yp=torch.empty((d.P, c.H), dtype=f32, device="cuda"),
             ysh=torch.empty((c.T, c.H), dtype=f32, device="cuda") if shared is not None else None,
             out=torch.empty((c.T, c.H), dtype=f32, device="cuda"),
             obf=torch.empty((c.T, c.H), dtype=torch.int16, device="cuda") if with_bf16 else None)
    if ws is None:
        ws = torch.zeros(M.moe_layer_decode_workspace_size(d, shared is not None), dtype=torch.uint8,
                         device="cuda")
    bias = dev(inp["bias"]) if inp["bias"] is not None else None
    M.moe_layer_decode(d, routed, shared, dev(inp["x"]), dev(inp["wr"]), bias, o["logits"], o["ids"],
                       o["w"], o["sp"], o["off"], o["pp"], o["yp"], o["ysh"],
                       residual, o["out"], o["obf"], ws)
    torch.cuda.synchronize()
    o["ws"] = ws
    return o


@pytest.mark.parametrize("name", list(FUSED))
def test_fused_decode_small(name):
    c = FUSED[name]
    say("fused decode", name)
    inp = layer_inputs(c)
    res = synth.activations(c.seed + 100, 0, c.T, c.H).astype(np.uint16)
    resid = O.bf16_to_f64(res).astype(np.float32)
    M.moe_reset_counters()
    o = run_fused(c, inp, residual=dev(resid), with_bf16=True)
    assert M.moe_get_counters()["decode_fused"] == 1
    ref = O.moe_layer(inp["x"], c.k, oracle_weights(c, inp["routed"]), "stq1", wr_bits=inp["wr"],
                      bias=inp["bias"], shared=inp["shared"], residual=resid.astype(np.float64))
    assert np.abs(host(o["logits"]) - ref["logits"]).max() < 2e-5
    tie = near_tie_tokens(ref["logits"], c.k)
    gi = host(o["ids"])
    assert (gi[~tie] == ref["ids"][~tie]).all()
    for t in np.flatnonzero(tie):
        assert valid_selection(ref["logits"][t], gi[t], c.k)
    # the permutation is exact for the ids the kernel chose
    rsp, roff, rpp = O.permute(gi, c.E)
    assert (host(o["sp"]) == rsp).all() and (host(o["off"]) == roff).all() and (host(o["pp"]) == rpp).all()
    ok = ~tie
    out = host(o["out"])
    err = row_err(out[ok], ref["out"][ok])
    say("fused max row err", float(err.max()), "near ties", int(tie.sum()))
    assert err.max() <= TOL
    if not tie.any():
        assert row_err(host(o["yp"]), ref["y_pairs"]).max() <= TOL
        if inp["shared"] is not None:
            assert row_err(host(o["ysh"]), ref["y_shared"]).max() <= TOL
    assert (host(o["obf"], np.uint16) == O.f64_to_bf16_bits(out.astype(np.float64))).all()
    # the counters were left zero: a second call on the same workspace gives the same bits
    o2 = run_fused(c, inp, residual=dev(resid), ws=o["ws"])
    assert (host(o2["out"]).view(np.uint32) == out.view(np.uint32)).all()


MX_FUSED = {
    "h512-i256-e8-top2-t1-shared": synth.LayerCfg("t", 1, 512, 256, 8, 2, True, "mxfp4", False, False, 1, 41),
    "h1024-i512-e16-top4-t3-zipf": synth.LayerCfg("t", 3, 1024, 512, 16, 4, True, "mxfp4", True, False, 1, 42),
    "h512-i256-e64-top8-t4-shared": synth.LayerCfg("t", 4, 512, 256, 64, 8, True, "mxfp4", False, False, 1, 43),
    # experts shared by both tokens
    "h512-i256-e4-top4-t2-noshared": synth.LayerCfg("t", 2, 512, 256, 4, 4, False, "mxfp4", False, False, 1, 44),
    # one pair: the staged h run (264 bytes) is not a whole number of 16-byte pieces
    "h512-i256-e8-top1-t1-noshared": synth.LayerCfg("t", 1, 512, 256, 8, 1, False, "mxfp4", False, False, 1, 45),
    # beyond four tokens: the item-list kernels (one token tile; two with Zipf routing and
    # experts over 16 pairs, split into several units; three tiles, every expert in 10 units)
    "h512-i256-e16-top4-t9-shared": synth.LayerCfg("t", 9, 512, 256, 16, 4, True, "mxfp4", False, False, 1, 47),
    "h1024-i512-e32-top8-t17-zipf": synth.LayerCfg("t", 17, 1024, 512, 32, 8, True, "mxfp4", True, False, 1, 48),
    "h512-i256-e8-top2-t40-noshared": synth.LayerCfg("t", 40, 512, 256, 8, 2, False, "mxfp4", False, False, 1, 49),
}


def _fused_mx_check(c, inp, o, resid, experts=None):
    d = M.Dims(c.T, c.H, c.I, c.E, c.k)
    T, H, I, P = c.T, c.H, c.I, d.P
    rl, rid, _ = O.route(c.k, inp["x"], inp["wr"], inp["bias"])
    assert np.abs(host(o["logits"]) - rl).max() < 2e-5
    tie = near_tie_tokens(rl, c.k)
    gi = host(o["ids"])
    assert (gi[~tie] == rid[~tie]).all()
    for t in np.flatnonzero(tie):
        assert valid_selection(rl[t], gi[t], c.k)
    rsp, roff, rpp = O.permute(gi, c.E)
    sp, off = host(o["sp"]), host(o["off"])
    assert (sp == rsp).all() and (off == roff).all() and (host(o["pp"]) == rpp).all()
    offs = M.moe_layer_decode_workspace_offsets(d, inp["shared"] is not None)
    ws = host(o["ws"])
    xq = ws[offs[9]:offs[9] + T * H].reshape(T, H)
    xs = ws[offs[9] + T * H:offs[9] + T * H + T * H // 32].reshape(T, H // 32)
    rq, rs = O.mx_quantize_e4m3(O.bf16_to_f64(inp["x"]))
    assert (xq == rq).all() and (xs == rs).all()
    hq = ws[offs[6]:offs[6] + P * I].reshape(P, I)
    hs = ws[offs[6] + P * I:offs[6] + P * I + P * I // 32].reshape(P, I // 32)
    yp = host(o["yp"])
    _mx_h_down_check(c, oracle_weights(c, inp["routed"]), O.mx_dequantize_e4m3(rq, rs), hq, hs, yp,
                     sp, off, range(c.E) if experts is None else experts)
    ysh = None
    if inp["shared"] is not None:
        ysh = host(o["ysh"])
        assert row_err(ysh, O.shared_expert(inp["x"], *inp["shared"])).max() <= TOL
    w = host(o["w"])
    out_ref = O.combine(yp, w, host(o["pp"]), ysh, None if resid is None else resid.astype(np.float64))
    err = row_err(host(o["out"]), out_ref)
    say("fused mx combine max row err", float(err.max()))
    assert err.max() <= TOL


@pytest.mark.parametrize("tiled", [False, True], ids=["rowmajor", "tiled"])
@pytest.mark.parametrize("name", list(MX_FUSED))
def test_fused_decode_mx_small(name, tiled):
    """Fused decode with MXFP4 routed experts: x and h codes bit-exact / within one E4M3
    step of the oracle on the GPU's routing, y_pairs from the GPU's h, shared expert, combine."""
    c = MX_FUSED[name]
    say("fused decode mx", name, "tiled" if tiled else "row-major")
    inp = layer_inputs(c)
    res = synth.activations(c.seed + 100, 0, c.T, c.H).astype(np.uint16)
    resid = O.bf16_to_f64(res).astype(np.float32)
    M.moe_reset_counters()
    o = run_fused(c, inp, residual=dev(resid), with_bf16=True, tiled=tiled)
    assert M.moe_get_counters()["decode_fused"] == 1
    _fused_mx_check(c, inp, o, resid)
    out = host(o["out"])
    assert (host(o["obf"], np.uint16) == O.f64_to_bf16_bits(out.astype(np.float64))).all()
    o2 = run_fused(c, inp, residual=dev(resid), ws=o["ws"], tiled=tiled)
    assert (host(o2["out"]).view(np.uint32) == out.view(np.uint32)).all()


def test_fused_decode_mx_hy4_t1():
    """Hy4 shape, one token, MXFP4 (tiled) routed experts and the bf16 shared expert."""
    c = synth.LayerCfg("hy4-mxfp4-decode-t1", 1, 6144, 2048, 256, 8, True, "mxfp4", False, False, 1, 46)
    say("fused decode mx hy4 generate")
    inp = layer_inputs(c)
    o = run_fused(c, inp, tiled=True)
    _fused_mx_check(c, inp, o, None, experts=sorted(set(host(o["ids"]).ravel().tolist())))


def test_fused_decode_mx_hy4_t64_zipf():
    """Hy4 shape, 64 tokens with Zipf(1.1) routing, MXFP4 (tiled) routed experts and the bf16
    shared expert: routing, permutation and x codes in full; h codes and the down stage on the
    experts with the most and the fewest pairs plus one more; shared expert and combine in full."""
    c = synth.LayerCfg("hy4-mxfp4-decode-t64-zipf", 64, 6144, 2048, 256, 8, True, "mxfp4", True, False, 1, 50)
    say("fused decode mx hy4 t64 generate")
    inp = layer_inputs(c)
    o = run_fused(c, inp, tiled=True)
    ids = host(o["ids"]).ravel()
    cnt = np.bincount(ids, minlength=c.E)
    used = np.flatnonzero(cnt)
    pick = sorted({int(used[np.argmax(cnt[used])]), int(used[np.argmin(cnt[used])]), int(used[len(used) // 2])})
    say("fused decode mx hy4 t64 experts", pick, "pairs", cnt[pick].tolist())
    _fused_mx_check(c, inp, o, None, experts=pick)


def test_fused_decode_cfg1_hy4():
    c = synth.cfg(1)
    say("fused decode cfg1 generate")
    inp = layer_inputs(c)
    o = run_fused(c, inp)
    say("fused decode cfg1 oracle")
    ref = O.moe_layer(inp["x"], c.k, oracle_weights(c, inp["routed"]), "stq1", wr_bits=inp["wr"],
                      shared=inp["shared"])
    assert (host(o["ids"]) == ref["ids"]).all()
    err = row_err(host(o["out"]), ref["out"])
    say("fused cfg1 max row err", float(err.max()))
    assert err.max() <= TOL
    assert row_err(host(o["yp"]), ref["y_pairs"]).max() <= TOL


def test_fused_decode_cfg2_hy4_zipf_sampled():
    c = synth.cfg(2)
    say("fused decode cfg2 generate")
    inp = layer_inputs(c)
    o = run_fused(c, inp)
    rl, rid, _ = O.route(c.k, inp["x"], inp["wr"], inp["bias"])
    tie = near_tie_tokens(rl, c.k)
    gi = host(o["ids"])
    assert (gi[~tie] == rid[~tie]).all()
    rsp, roff, rpp = O.permute(gi, c.E)
    assert (host(o["sp"]) == rsp).all() and (host(o["pp"]) == rpp).all()
    sample = [t for t in synth.sample_tokens(c.seed, c.T, 6) if not tie[t]]
    say("fused cfg2 oracle tokens", sample)
    ref = O.moe_layer(inp["x"][sample], c.k, oracle_weights(c, inp["routed"]), "stq1", wr_bits=inp["wr"],
                      bias=inp["bias"], shared=inp["shared"])
    err = row_err(host(o["out"])[sample], ref["out"])
    say("fused cfg2 sampled max row err", float(err.max()))
    assert err.max() <= TOL


# ----------------------------------------------------------------------------- norm, combine, chain
def test_rmsnorm_bf16_matches_oracle():
    g = np.random.default_rng(21)
    T, H = 19, 6144
    r = (g.standard_normal((T, H)) * np.exp(g.uniform(-6, 6, (T, 1)))).astype(np.float32)
    r[3] = 0.0                                     # all-zero row: eps keeps it finite
    say("rmsnorm", T, H)
    a = torch.empty((T, H), dtype=torch.int16, device="cuda")
    M.moe_rmsnorm_bf16(T, H, 1e-6, dev(r), a)
    got = host(a, np.uint16)
    ref = O.rmsnorm_bf16(r.astype(np.float64))
    # the GPU sums squares in fp32 in another order, so a value lying within an fp32 rounding
    # of a bf16 rounding boundary may round the other way: one bf16 step at most, rarely
    gi = got.astype(np.int32)
    ri = ref.astype(np.int32)
    assert (np.abs(gi - ri) <= 1).all()
    assert (gi != ri).mean() <= 1e-3
    assert (got[3] == 0).all()


def test_combine_with_residual_and_bf16():
    g = np.random.default_rng(22)
    T, H, k = 37, 768, 4
    P = T * k
    yp = g.standard_normal((P, H)).astype(np.float32)
    w = g.random((T, k)).astype(np.float32)
    w /= w.sum(axis=1, keepdims=True)
    pp = g.permutation(P).astype(np.int32)
    ysh = g.standard_normal((T, H)).astype(np.float32)
    res = g.standard_normal((T, H)).astype(np.float32)
    d = M.Dims(T, H, 256, 16, k)
    out = torch.empty((T, H), dtype=torch.float32, device="cuda")
    obf = torch.empty((T, H), dtype=torch.int16, device="cuda")
    M.moe_combine(d, dev(yp), dev(w), dev(pp), dev(ysh), dev(res), out, obf)
    ref = O.combine(yp, w, pp, ysh, res)
    got = host(out)
    assert row_err(got, ref).max() <= 1e-6
    assert (host(obf, np.uint16) == O.f64_to_bf16_bits(got.astype(np.float64))).all()
    # residual may alias the output
    r2 = dev(res)
    M.moe_combine(d, dev(yp), dev(w), dev(pp), dev(ysh), r2, r2, None)
    assert row_err(host(r2), ref).max() <= 1e-6


def test_combine_more_tokens_than_a_y_grid_dimension():
    """70000 tokens, more than the 65535 blocks a y or z grid dimension holds (the combine
    puts tokens on x)."""
    g = np.random.default_rng(23)
    T, H, k = 70000, 64, 2
    P = T * k
    yp = g.standard_normal((P, H)).astype(np.float32)
    w = g.random((T, k)).astype(np.float32)
    pp = g.permutation(P).astype(np.int32)
    d = M.Dims(T, H, 256, 16, k)
    out = torch.empty((T, H), dtype=torch.float32, device="cuda")
    M.moe_combine(d, dev(yp), dev(w), dev(pp), None, None, out, None)
    ref = O.combine(yp, w, pp, None, None)
    assert row_err(host(out), ref).max() <= 1e-6


def test_chain_cfg4_hy4_29_layers_sampled():
    """29 STQ1_0 Hy4 layers at 16 tokens with Zipf-skewed routing, chained through
    pre-norm residual adds: a = bf16(RMSNorm(r)), r <- r + MoE(a).  Two sampled tokens are
    checked at every layer, teacher-forced (the oracle takes the GPU's r of that layer)."""
    from concurrent.futures import ThreadPoolExecutor
    from tests.helpers import oracle_weights_regen
    c = synth.cfg(4)
    d = M.Dims(c.T, c.H, c.I, c.E, c.k)
    toks = synth.sample_tokens(c.seed, c.T, 2)
    x0 = synth.activations(c.seed, 0, c.T, c.H)
    r = torch.from_numpy(O.bf16_to_f64(x0).astype(np.float32)).cuda()
    r_next = torch.empty_like(r)
    a = torch.empty((c.T, c.H), dtype=torch.int16, device="cuda")
    f32, i32 = torch.float32, torch.int32
    o = dict(logits=torch.empty((c.T, c.E), dtype=f32, device="cuda"),
             ids=torch.empty((c.T, c.k), dtype=i32, device="cuda"),
             w=torch.empty((c.T, c.k), dtype=f32, device="cuda"),
             sp=torch.empty(d.P, dtype=i32, device="cuda"),
             off=torch.empty(c.E + 1, dtype=i32, device="cuda"),
             pp=torch.empty(d.P, dtype=i32, device="cuda"),
             yp=torch.empty((d.P, c.H), dtype=f32, device="cuda"),
             ysh=torch.empty((c.T, c.H), dtype=f32, device="cuda"))
    ws = torch.zeros(M.moe_layer_decode_workspace_size(d, True), dtype=torch.uint8, device="cuda")
    worst, n_tie, n_flip_a = 0.0, 0, 0
    pool = ThreadPoolExecutor(16)
    for layer in range(c.layers):
        inp = layer_inputs(c, layer)
        routed = routed_experts(c, inp["routed"])
        shared = shared_experts(inp["shared"])
        M.moe_rmsnorm_bf16(c.T, c.H, 1e-6, r, a)
        M.moe_layer_decode(d, routed, shared, a, dev(inp["wr"]), dev(inp["bias"]), o["logits"],
                           o["ids"], o["w"], o["sp"], o["off"], o["pp"], o["yp"], o["ysh"],
                           r, r_next, None, ws)
        torch.cuda.synchronize()
        r_l = host(r)[toks]
        a_l = host(a, np.uint16)[toks]
        delta = host(r_next)[toks].astype(np.float64) - r_l
        del routed, shared, inp
        # the norm: teacher-forced on the GPU's r
        a_ref = O.rmsnorm_bf16(r_l.astype(np.float64))
        assert (np.abs(a_l.astype(np.int32) - a_ref.astype(np.int32)) <= 1).all()
        n_flip_a += int((a_l != a_ref).sum())
        # the MoE layer on the GPU's normed input
        wr = synth.router_weights(c.seed, layer, c.E, c.H)
        bias = synth.zipf_bias(c.seed, layer, c.E)
        logits, rid, _ = O.route(c.k, a_l, wr, bias)
        tie = near_tie_tokens(logits, c.k)
        n_tie += int(tie.sum())
        assert (host(o["ids"])[toks][~tie] == rid[~tie]).all()
        regen = oracle_weights_regen(c, layer)
        need = sorted({(int(e), m) for e in rid.ravel() for m in range(3)})
        cache = dict(zip(need, pool.map(lambda em: regen(*em), need)))
        ref = O.moe_layer(a_l, c.k, lambda e, m: cache[(e, m)], "stq1", wr_bits=wr, bias=bias,
                          shared=synth.shared_weights(c.seed, layer, c.I, c.H))
        err = row_err(delta[~tie], ref["out"][~tie]) if (~tie).any() else np.zeros(1)
        worst = max(worst, float(err.max()))
        say(f"chain layer {layer}: max row err {float(err.max()):.2e}, near-ties {int(tie.sum())}")
        assert err.max() <= TOL
        r, r_next = r_next, r
    say("chain: worst", worst, "near-tie token-layers", n_tie, "bf16 norm flips", n_flip_a)


# ----------------------------------------------------------------------------- STQ1_0 encoders
def _encode_gpu(x, K, imat, method):
    n = x.size
    c = torch.empty(n // 256 * 40, dtype=torch.uint8, device="cuda")
    sc = torch.empty(n // 256, dtype=torch.int16, device="cuda")
    M.moe_stq1_encode(dev(np.ascontiguousarray(x, dtype=np.float32)),
                      None if imat is None else dev(np.ascontiguousarray(imat, dtype=np.float32)),
                      n, K, method, c, sc)
    torch.cuda.synchronize()
    return host(c), host(sc).view(np.uint16)


def _encode_inputs():
    g = np.random.default_rng(51)
    ties = (g.integers(-3, 4, 64 * 512) * 0.01).astype(np.float32)   # many equal |x| and zeros
    ties[::7] = -0.0
    return {
        "normal-n48-k512": (g.standard_normal(48 * 512).astype(np.float32) * 0.02, 512),
        "straddle-n64-k128": (g.standard_normal(64 * 128).astype(np.float32) * 0.02, 128),
        "ties-n64-k512": (ties, 512),
        "student3-n512-k6144": (g.standard_t(3, 512 * 6144).astype(np.float32) * 0.02, 6144),
    }


@pytest.mark.parametrize("name", ["normal-n48-k512", "straddle-n64-k128", "ties-n64-k512", "student3-n512-k6144"])
def test_stq1_encode_upstream_bitexact(name):
    """Upstream STQ1_0 encoder (block amax, zero at the smallest |x|): codes and scales equal
    the oracle's bit for bit (max and comparisons are exact in any order)."""
    x, K = _encode_inputs()[name]
    say("stq1 encode upstream", name)
    gc, gs = _encode_gpu(x, K, None, M.MOE_STQ1_ENC_UPSTREAM)
    oc, osc = O.stq1_encode(x.astype(np.float64), K, method="upstream")
    assert (gc == oc).all() and (gs == osc).all()


@pytest.mark.parametrize("imat", [False, True], ids=["no-imatrix", "imatrix"])
@pytest.mark.parametrize("name", ["normal-n48-k512", "straddle-n64-k128", "student3-n512-k6144"])
def test_stq1_encode_wls_matches_oracle(name, imat):
    """Weighted least-squares STQ1_0 encoder: the GPU sums in fp32, the oracle in float64.
    Blocks whose zero placement matches take d within one fp16 step; a block may place a zero
    differently only at a near-tie, so such blocks are rare and their weighted error equals
    the oracle's to 1e-3."""
    x, K = _encode_inputs()[name]
    w = np.exp(np.random.default_rng(52).standard_normal(K)).astype(np.float32) if imat else None
    say("stq1 encode wls", name, "imatrix" if imat else "")
    gc, gs = _encode_gpu(x, K, w, M.MOE_STQ1_ENC_WLS)
    xd = x.astype(np.float64)
    wd = None if w is None else w.astype(np.float64)
    oc, osc = O.stq1_encode(xd, K, imatrix=wd, method="wls")
    same = (O.stq1_patterns_of(gc) == O.stq1_patterns_of(oc)).all(axis=1)
    step = np.abs(gs.astype(np.int64) - osc.astype(np.int64))
    eg = O.stq1_weighted_ssd(xd, K, gc, gs, wd)
    eo = O.stq1_weighted_ssd(xd, K, oc, osc, wd)
    say("blocks", same.size, "with another zero placement", int((~same).sum()),
        "max fp16 step on matching blocks", int(step[same].max()) if same.any() else None)
    assert (step[same] <= 1).all()
    assert (~same).mean() <= 0.02
    assert (np.abs(eg - eo) <= 1e-3 * eo).all()
    # and the encoder does what it is for: far less weighted error than the upstream one
    uc, us = O.stq1_encode(xd, K, method="upstream")
    assert eg.sum() < 0.5 * O.stq1_weighted_ssd(xd, K, uc, us, wd).sum()


def test_stq1_encode_grid_inputs_exact():
    """Weights already on the ternary grid come back exactly from both GPU encoders."""
    g = np.random.default_rng(53)
    n_blk = 64
    z = g.integers(0, 4, n_blk * 64)
    s = g.integers(0, 8, n_blk * 64)
    d = np.abs(g.standard_normal(n_blk) * 0.02).astype(np.float16)
    d[d == 0] = np.float16(0.01)
    lanes = np.array([O.stq1_pattern(int(p)) for p in (8 * z + s)], dtype=np.float64)
    x = (lanes.reshape(n_blk, 256) * d.astype(np.float64)[:, None]).reshape(-1).astype(np.float32)
    want = O.stq1_pack(z, s, d.view(np.uint16))
    for method in (M.MOE_STQ1_ENC_UPSTREAM, M.MOE_STQ1_ENC_WLS):
        gc, gs = _encode_gpu(x, 1024, np.exp(g.standard_normal(1024)), method)
        assert (gc == want[0]).all() and (gs == want[1]).all()


# ----------------------------------------------------------------------------- MXFP8 shared expert
MX8_SHARED = {
    # a few tokens: routed STQ1_0 on the decode kernels, the MXFP8 shared expert on its GEMMs
    "stq-h512-i256-e8-top2-t5": synth.LayerCfg("s8", 5, 512, 256, 8, 2, True, "stq1", False, False, 1, 61),
    # several M blocks of the shared expert (300 tokens: three blocks of 100), MXFP4 routed
    "mx-h512-i256-e8-top2-t300": synth.LayerCfg("s8", 300, 512, 256, 8, 2, True, "mxfp4", False, True, 1, 62),
    # three down N tiles, full blocks (256 tokens: two blocks of 128)
    "stq-h768-i512-e4-top2-t256": synth.LayerCfg("s8", 256, 768, 512, 4, 2, True, "stq1", False, True, 1, 63),
}


def _mx8_shared_check(c, inp, bufs, d, sh8, toks=None):
    """h of the shared expert against the oracle's SiLU(a Wg^T) * (a Wu^T) with a the MX
    E4M3 values of x, and y_shared against the oracle's down projection of the MX E4M3
    values of the GPU's own h (so the discontinuous requantisation is taken the same way)."""
    fmt = M.MOE_W_STQ1_0 if c.fmt == "stq1" else M.MOE_W_MXFP4
    offs = M.moe_workspace_offsets(d, fmt, True)
    T, H, I = c.T, c.H, c.I
    toks = np.arange(T) if toks is None else np.asarray(toks)
    h_gpu = host(bufs.ws[offs[1]:offs[1] + T * I * 4]).view(np.float32).reshape(T, I)[toks]
    a = O.mx_dequantize_e4m3(*O.mx_quantize_e4m3(O.bf16_to_f64(inp["x"][toks])))
    Wg, Wu, Wd = [O.mx_dequantize_e4m3(cd, sc) for cd, sc in sh8]
    h_ref = O.silu(a @ Wg.T) * (a @ Wu.T)
    eh = row_err(h_gpu, h_ref).max()
    y_ref = O.mx_dequantize_e4m3(*O.mx_quantize_e4m3(h_gpu.astype(np.float64))) @ Wd.T
    ey = row_err(host(bufs.y_shared)[toks], y_ref).max()
    say("mxfp8 shared: h max row err", float(eh), "y_shared max row err", float(ey))
    assert eh <= TOL and ey <= TOL


@pytest.mark.parametrize("name", list(MX8_SHARED))
def test_shared_expert_mxfp8(name):
    """MXFP8 W8A8 shared expert (E4M3 weights decoded with the gfx950 scaled conversion, x and
    h MX-quantised) through moe_expert_ffn, next to STQ1_0 or MXFP4 routed experts."""
    c = MX8_SHARED[name]
    say("mxfp8 shared", name)
    inp = layer_inputs(c)
    d = M.Dims(c.T, c.H, c.I, c.E, c.k)
    sh8 = synth.shared_weights_mxfp8(c.seed, 0, c.I, c.H)
    shared = M.Experts(M.MOE_W_MXFP8, *[(dev(cd), dev(sc)) for cd, sc in sh8])
    routed = routed_experts(c, inp["routed"])
    fmt = M.MOE_W_STQ1_0 if c.fmt == "stq1" else M.MOE_W_MXFP4
    bufs = LayerBuffers(d, fmt, True)
    M.moe_reset_counters()
    if c.logits_given:
        run_layer(d, bufs, dev(inp["x"]), routed, shared, logits_in=dev(inp["logits_in"]))
    else:
        run_layer(d, bufs, dev(inp["x"]), routed, shared, wr_bf16=dev(inp["wr"]))
    torch.cuda.synchronize()
    cnt = M.moe_get_counters()
    assert cnt["mxfp8_shared"] == 2 and cnt["bf16_gateup"] == 0 and cnt["bf16_gemm"] == 0
    _mx8_shared_check(c, inp, bufs, d, sh8)
    out_ref = O.combine(host(bufs.y_pairs), host(bufs.topk_w), host(bufs.pair_pos), host(bufs.y_shared))
    assert row_err(host(bufs.out), out_ref).max() <= TOL
    # the whole layer against the oracle, printed (h requantisation is discontinuous)
    ref = O.moe_layer(inp["x"], c.k, oracle_weights(c, inp["routed"]), c.fmt,
                      wr_bits=None if c.logits_given else inp["wr"],
                      logits_in=inp["logits_in"] if c.logits_given else None,
                      shared=sh8, shared_fmt="mxfp8")
    say("mxfp8 shared: y_shared vs the oracle end to end",
        float(row_err(host(bufs.y_shared), ref["y_shared"]).max()))


def test_shared_expert_mxfp8_hy4_t4096_sampled():
    """Hy4 MXFP4 routed + MXFP8 shared layer at 4096 tokens (the WFP4AFP8 recipe's formats):
    the shared expert checked on sampled tokens."""
    c = synth.LayerCfg("hy4-wfp4afp8-prefill-t4096", 4096, 6144, 2048, 256, 8, True, "mxfp4", False, True, 1, 64)
    say("mxfp8 shared t4096 generate")
    inp = layer_inputs(c)
    d = M.Dims(c.T, c.H, c.I, c.E, c.k)
    sh8 = synth.shared_weights_mxfp8(c.seed, 0, c.I, c.H)
    shared = M.Experts(M.MOE_W_MXFP8, *[(dev(cd), dev(sc)) for cd, sc in sh8])
    routed = routed_experts(c, inp["routed"], tiled=True)
    bufs = LayerBuffers(d, M.MOE_W_MXFP4, True)
    run_layer(d, bufs, dev(inp["x"]), routed, shared, logits_in=dev(inp["logits_in"]))
    torch.cuda.synchronize()
    _mx8_shared_check(c, inp, bufs, d, sh8, toks=synth.sample_tokens(c.seed, c.T, 4))


# ----------------------------------------------------------------------------- graph capture
@pytest.mark.parametrize("fmt", ["stq1", "mxfp4"])
def test_fused_decode_graph_replays(fmt):
    """moe_layer_decode captured once into a HIP graph and replayed with new tokens copied into
    the captured input buffer, eager work and synchronisations between the replays: every
    replay equals the eager call on the same token, bit for bit."""
    c = synth.LayerCfg("g", 1, 512, 256, 8, 2, True, fmt, False, False, 1, 71)
    inp = layer_inputs(c)
    d = M.Dims(c.T, c.H, c.I, c.E, c.k)
    routed = routed_experts(c, inp["routed"], tiled=(fmt == "mxfp4"))
    shared = shared_experts(inp["shared"])
    f32, i32 = torch.float32, torch.int32
    bufs = [torch.empty((1, c.E), dtype=f32, device="cuda"), torch.empty((1, c.k), dtype=i32, device="cuda"),
            torch.empty((1, c.k), dtype=f32, device="cuda"), torch.empty(d.P, dtype=i32, device="cuda"),
            torch.empty(c.E + 1, dtype=i32, device="cuda"), torch.empty(d.P, dtype=i32, device="cuda"),
            torch.empty((d.P, c.H), dtype=f32, device="cuda"), torch.empty((1, c.H), dtype=f32, device="cuda")]
    out = torch.empty((1, c.H), dtype=f32, device="cuda")
    ws = torch.zeros(M.moe_layer_decode_workspace_size(d, True), dtype=torch.uint8, device="cuda")
    x_in = torch.empty((1, c.H), dtype=torch.int16, device="cuda")
    wr = dev(inp["wr"])
    tokens = dev(synth.activations(c.seed, 5, 4, c.H))

    def call(stream):
        M.moe_layer_decode(d, routed, shared, x_in, wr, None, *bufs, None, out, None, ws, stream)

    x_in.copy_(tokens[0:1])
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):          # warm the library's one-time set-up off the capture
        call(side.cuda_stream)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    for r in range(4):
        x_in.copy_(tokens[r:r + 1])
        call(torch.cuda.current_stream().cuda_stream)          # eager reference
        torch.cuda.synchronize()
        want = out.clone()
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int32), want.view(torch.int32)), f"replay {r} differs"


@pytest.mark.parametrize("fmt", ["stq1", "mxfp4"])
def test_prefill_layer_graph_replays(fmt):
    """The four calls of a prefill layer (router GEMV and top-k from x, the chunk-parallel
    permutation of 8200 pairs, the grouped GEMMs of the routed and the shared expert, combine)
    captured once into a HIP graph and replayed with new tokens copied into the captured
    input, eager calls and synchronisations between the replays: every replay equals the
    eager layer on the same tokens, bit for bit (routing, permutation and output)."""
    c = synth.LayerCfg("gp", 4100, 512, 256, 16, 2, True, fmt, True, False, 1, 72)
    say("prefill graph replays", fmt, "T", c.T)
    inp = layer_inputs(c)
    d = M.Dims(c.T, c.H, c.I, c.E, c.k)
    routed = routed_experts(c, inp["routed"], tiled=(fmt == "mxfp4"))
    shared = shared_experts(inp["shared"])
    bufs = LayerBuffers(d, M.MOE_W_MXFP4 if fmt == "mxfp4" else M.MOE_W_STQ1_0, True)
    wr, bias = dev(inp["wr"]), dev(inp["bias"])
    x_in = torch.empty((c.T, c.H), dtype=torch.int16, device="cuda")
    tokens = [dev(synth.activations(c.seed, 10 + r, c.T, c.H)) for r in range(3)]

    def call(stream):
        run_layer(d, bufs, x_in, routed, shared, wr_bf16=wr, logit_bias=bias, stream=stream)

    x_in.copy_(tokens[0])
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):          # warm the library's one-time set-up off the capture
        call(side.cuda_stream)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    for r in range(3):
        x_in.copy_(tokens[r])
        call(torch.cuda.current_stream().cuda_stream)          # eager reference
        torch.cuda.synchronize()
        want = [t.clone() for t in (bufs.topk_ids, bufs.sorted_pair, bufs.offsets, bufs.out)]
        bufs.out.zero_()
        bufs.sorted_pair.fill_(-7)
        g.replay()
        torch.cuda.synchronize()
        got = (bufs.topk_ids, bufs.sorted_pair, bufs.offsets, bufs.out)
        for name, a, b in zip(("ids", "sorted_pair", "offsets", "out"), got, want):
            assert torch.equal(a.view(torch.int32), b.view(torch.int32)), f"replay {r}: {name} differs"
    assert not torch.equal(want[3], torch.zeros_like(want[3]))


# ----------------------------------------------------------------------------- expert slot bank
def test_slot_bank_layer_equals_direct():
    """A layer whose 16 routed experts live in pinned host memory and run from an 8-slot
    device bank (plan, chunked fetch, id remap, then permute / FFN / combine over the slots)
    gives the same bits as the layer run on all 16 experts in device memory, step after step
    with new tokens (hits and misses both occur), also when a step is planned twice before its
    fetch."""
    E, S = 16, 8
    c = synth.LayerCfg("sb", 4, 512, 256, E, 2, True, "stq1", False, False, 1, 81)
    inp = layer_inputs(c)
    d = M.Dims(c.T, c.H, c.I, E, c.k)
    dS = M.Dims(c.T, c.H, c.I, S, c.k)
    routed = routed_experts(c, inp["routed"])
    shared = shared_experts(inp["shared"])
    wr = dev(inp["wr"])
    fams = inp["routed"]                                    # (codes [E, n], scales [E, m]) x 3
    host = [tuple(torch.from_numpy(np.ascontiguousarray(a).view(np.uint8)).pin_memory() for a in f) for f in fams]
    per = []
    for cd, sc in host:
        per += [cd.numel() // E, sc.numel() // E]
    slots = [(torch.empty(S * per[2 * i], dtype=torch.uint8, device="cuda"),
              torch.empty(S * per[2 * i + 1], dtype=torch.uint8, device="cuda")) for i in range(3)]
    host_src = M.Experts(M.MOE_W_STQ1_0, *host)
    dev_slots = M.Experts(M.MOE_W_STQ1_0, *slots)
    bank = M.SlotBank(E, S, per, io_split=4)
    ref_bufs = LayerBuffers(d, M.MOE_W_STQ1_0, True)
    sb = LayerBuffers(dS, M.MOE_W_STQ1_0, True)
    slot_of_dev = torch.empty(E, dtype=torch.int32, device="cuda")
    slot_ids = torch.empty((c.T, c.k), dtype=torch.int32, device="cuda")
    tokens = synth.activations(c.seed, 9, 8 * c.T, c.H)
    for step in range(8):
        x = dev(tokens[step * c.T:(step + 1) * c.T])
        ref = run_layer(d, ref_bufs, x, routed, shared, wr_bf16=wr)
        M.moe_route(d, x, wr, None, None, sb.logits, sb.topk_ids, sb.topk_w)
        slot_of, n_copies = bank.plan(host_t(sb.topk_ids))
        if step % 2:
            # planned again before the fetch: all hits now, and the first plan's copies must
            # still be fetched
            again, n2 = bank.plan(host_t(sb.topk_ids))
            assert n2 == 0 and (again == slot_of).all()
        slot_of_dev.copy_(torch.from_numpy(slot_of))
        bank.fetch(host_src, dev_slots, torch.cuda.current_stream().cuda_stream)
        M.moe_remap_ids(sb.topk_ids, d.P, slot_of_dev, slot_ids)
        M.moe_permute(dS, slot_ids, sb.sorted_pair, sb.offsets, sb.pair_pos)
        M.moe_expert_ffn(dS, dev_slots, shared, x, sb.sorted_pair, sb.offsets, sb.y_pairs, sb.y_shared, sb.ws)
        M.moe_combine(dS, sb.y_pairs, sb.topk_w, sb.pair_pos, sb.y_shared, None, sb.out, None)
        torch.cuda.synchronize()
        assert torch.equal(sb.out.view(torch.int32), ref.view(torch.int32)), f"step {step}"
    hits, misses = bank.stats()
    say("slot bank hits", hits, "misses", misses)
    assert hits > 0 and misses > S


def host_t(t):
    return t.detach().cpu().numpy()
