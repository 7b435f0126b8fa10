"""Pins of the CPU oracle to facts that do not come from the oracle itself:
sizes the pages print, hand-written layout examples, closed forms, independent
library routines (torch's float8 / bfloat16 conversions, scipy's expit, Python's
stable sort) and brute force on tiny inputs.  CPU only."""
import itertools
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import synth
from oracle import moe_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _kv(name):
    out = {}
    for line in open(os.path.join(GOLDEN, name)):
        line = line.split("#")[0].strip()
        if line:
            k, *v = line.split()
            out.setdefault(k, []).append(v)
    return out


# ----------------------------------------------------------------------------- STQ1_0 format
def test_stq1_patterns_exhaustive():
    """All 32 patterns: exactly one zero and three +-1 lanes, all distinct, and every
    (zero lane, sign triple) appears once (4 x 2^3 = 32)."""
    seen = set()
    for p in range(32):
        lanes = O.stq1_pattern(p)
        assert sorted(map(abs, lanes)) == [0, 1, 1, 1]
        seen.add(tuple(lanes))
    assert len(seen) == 32
    all_patterns = set()
    for z in range(4):
        for signs in itertools.product((1, -1), repeat=3):
            v = list(signs)
            v.insert(z, 0)
            all_patterns.add(tuple(v))
    assert seen == all_patterns


def test_stq1_sizes_match_pages():
    g = {k: float(v[0][0]) for k, v in _kv("stq1_format.txt").items()}
    z, s, d = synth.stq1_pattern_fields(11, 0, 0, 0, 64 * 3)
    codes, scales = O.stq1_pack(z, s, d)
    n_blk = 3
    assert codes.size == n_blk * g["code_bytes"]
    assert scales.nbytes == n_blk * g["scale_bytes"]
    per_block = (codes.size + scales.nbytes) / n_blk
    assert per_block == g["block_bytes"]
    assert per_block * 8 / g["block_weights"] == g["bpw"]
    assert codes.size / n_blk * 8 / g["block_weights"] == g["bpw_codes_only"]
    assert g["groups_per_block"] * g["bits_per_group"] / 8 == g["code_bytes"]
    assert g["patterns"] == 2 ** g["bits_per_group"] == 32
    w = O.stq1_decode(codes, scales).reshape(-1, 4)
    assert ((w == 0).sum(axis=1) == g["zeros_per_group"]).all()


def test_stq1_layout_handwritten_examples():
    ex = _kv("stq1_layout_example.txt")
    for v in ex["pattern"]:
        p, lanes = int(v[0]), [int(t) for t in v[1:]]
        assert O.stq1_pattern(p) == lanes, p
    d1 = np.array([0x3C00], dtype=np.uint16)          # fp16 1.0
    # block where group g has pattern g % 32
    p = np.arange(64) % 32
    codes, _ = O.stq1_pack(p >> 3, p & 7, d1)
    assert codes.tobytes().hex() == "".join(ex["block_pg_mod32"][0])
    w = O.stq1_decode(codes, d1).reshape(64, 4)
    for g in range(64):
        assert list(w[g]) == [float(t) for t in O.stq1_pattern(g % 32)]
    p = np.full(64, 13)
    codes, _ = O.stq1_pack(p >> 3, p & 7, d1)
    assert codes.tobytes().hex() == "".join(ex["block_p13"][0])


def test_stq1_pack_decode_roundtrip_and_scale():
    z, s, d = synth.stq1_pattern_fields(3, 0, 1, 2, 64 * 40)
    codes, scales = O.stq1_pack(z, s, d)
    p = O.stq1_patterns_of(codes).reshape(-1)
    assert (p == z.astype(int) * 8 + s).all()
    w = O.stq1_decode(codes, scales).reshape(40, 256)
    dv = d.view(np.float16).astype(np.float64)
    for b in range(40):
        assert set(np.unique(np.abs(w[b]))) <= {0.0, dv[b]}
        assert (w[b] == 0).sum() == 64


def test_uniform_bytes_are_uniform_patterns():
    """The generator draws uniform code bytes; every 5-bit value is a valid pattern, so
    patterns (and zero lanes) come out uniform -- the distribution the workloads ask for."""
    codes, _ = synth.stq1_matrix(5, 0, 0, 0, 256 * 2000)
    p = O.stq1_patterns_of(codes).reshape(-1)
    hist = np.bincount(p, minlength=32)
    exp = p.size / 32
    chi2 = ((hist - exp) ** 2 / exp).sum()
    assert chi2 < 70, chi2          # 31 dof: p(chi2 > 70) ~ 1e-4
    zl = np.bincount(p >> 3, minlength=4) / p.size
    assert np.abs(zl - 0.25).max() < 0.01


def test_flashmoe_package_bytes():
    """Closed-form STQ1_0 matrix bytes reproduce the package's slot and sidecar sizes."""
    g = {k: int(float(v[0][0])) if k != "gateup_avg_bpw" else float(v[0][0])
         for k, v in _kv("flashmoe_package.txt").items()}
    H, I = g["hidden"], g["moe_intermediate"]
    n = H * I
    stq = n // 256 * 42
    assert stq == 2_064_384
    iq2 = n // 256 * g["iq2xxs_block_bytes"]
    assert g["iq2xxs_block_bytes"] * 8 / 256 == 2.0625
    iq3 = n // 256 * g["iq3xxs_block_bytes"]
    iq4 = n // 256 * g["iq4xs_block_bytes"]
    slot = (g["stq1_gateup_layers"] * 2 * stq + g["iq2xxs_gateup_layers"] * 2 * iq2
            + g["iq3xxs_down_layers"] * iq3 + g["iq4xs_down_layers"] * iq4)
    assert g["stq1_gateup_layers"] + g["iq2xxs_gateup_layers"] == g["moe_layers"]
    assert slot == g["slot_bytes"]
    assert slot * g["routed_experts"] == g["sidecar_bytes"]
    avg = (g["stq1_gateup_layers"] * 1.3125 + g["iq2xxs_gateup_layers"] * 2.0625) / g["moe_layers"]
    assert round(avg, 2) == g["gateup_avg_bpw"]


# ----------------------------------------------------------------------------- number formats
def test_e2m1_values():
    mags = [float(t) for t in _kv("e2m1_values.txt")["code_magnitudes"][0]]
    v = O.e2m1_value(np.arange(16))
    assert list(v[:8]) == mags
    assert list(v[8:]) == [-m for m in mags]


def test_e4m3_decode_vs_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    mine = O.e4m3_value(np.arange(256))
    nan = np.isnan(ref)
    assert (np.isnan(mine) == nan).all() and nan.sum() == 2
    assert (mine[~nan] == ref[~nan]).all()
    assert np.nanmax(mine) == O.E4M3_MAX


def test_ue8m0_values():
    v = O.ue8m0_value(np.arange(256))
    assert np.isnan(v[255])
    assert all(v[c] == math.ldexp(1.0, c - 127) for c in range(255))


def _e4m3_bruteforce(y):
    """Nearest finite E4M3 value by search; ties to the even code; beyond 448 saturate."""
    vals = O.e4m3_value(np.arange(128))[:127]      # non-negative finite values, codes 0..126
    out = []
    for t in np.asarray(y, dtype=np.float64).reshape(-1):
        a = abs(t)
        dist = np.abs(vals - a)
        best = np.flatnonzero(dist == dist.min())
        c = int(best[0]) if len(best) == 1 else int([b for b in best if b % 2 == 0][0])
        if a > 448:
            c = 126
        out.append(c | (128 if math.copysign(1.0, t) < 0 else 0))
    return np.array(out, dtype=np.uint8)


def test_e4m3_encode_vs_bruteforce_and_torch():
    # every bf16 magnitude from 2^-12 up to 512, both signs, plus exact ties
    bits = np.arange(0x3980, 0x4400, dtype=np.uint32)
    vals = (bits << 16).view(np.float32).astype(np.float64)
    vals = np.concatenate([vals, -vals, [0.0, -0.0, 2 ** -10, 3 * 2 ** -10, 17.0, 19.0, 464.0, 480.0]])
    mine = O.e4m3_encode(vals)
    assert (mine == _e4m3_bruteforce(vals)).all()
    small = np.abs(vals) < 464
    t = torch.tensor(vals[small], dtype=torch.float32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert (mine[small] == t).all()


def test_mx_quantize_rule():
    g = np.random.default_rng(0)
    rows = [g.standard_normal(32),
            np.zeros(32),
            np.full(32, 2.0 ** -140),          # clamps at scale byte 0
            np.full(32, 2.0 ** 140),           # clamps at scale byte 254
            np.r_[256.0, g.integers(-16, 17, 31)],
            g.standard_normal(32) * 1e-5,
            np.r_[511.0, g.standard_normal(31)]]
    v = np.stack(rows)
    q, s = O.mx_quantize_e4m3(v)
    for i, row in enumerate(v):
        amax = np.abs(row).max()
        if amax == 0:
            assert s[i, 0] == 0 and (q[i] == 0).all()
            continue
        X = int(s[i, 0]) - 127
        if -127 < X < 127:
            assert 256 <= amax / 2.0 ** X < 512          # scale rule: floor(log2 amax) - 8
        assert (q[i] == _e4m3_bruteforce(row / 2.0 ** X)).all()
    assert s[2, 0] == 0 and s[3, 0] == 254
    # exact integer group: 256 forces X = 0 and small integers stay exact
    assert (O.mx_dequantize_e4m3(q[4:5], s[4:5]) == v[4]).all()


def test_bf16_rne_vs_torch():
    g = np.random.default_rng(1)
    x = np.concatenate([g.standard_normal(20000).astype(np.float32),
                        (g.standard_normal(2000) * 1e-30).astype(np.float32),
                        np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8)], dtype=np.float32)])
    ref = torch.tensor(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert (O.f64_to_bf16_bits(x.astype(np.float64)) == ref).all()
    assert (synth.f32_to_bf16_bits(x) == ref).all()       # the generator agrees too


# ----------------------------------------------------------------------------- routing
def test_route_bruteforce_subsets():
    g = np.random.default_rng(2)
    for E, k in [(6, 2), (7, 3), (5, 5), (8, 1)]:
        logits = g.standard_normal((5, E))
        _, ids, w = O.route(k, logits_in=logits)
        for t in range(5):
            best = max(itertools.combinations(range(E), k), key=lambda c: sum(logits[t, list(c)]))
            assert set(ids[t]) == set(best)
            assert list(ids[t]) == sorted(best, key=lambda e: -logits[t, e])
            full = scipy.special.softmax(logits[t])
            ref = full[ids[t]] / full[ids[t]].sum()
            assert np.allclose(w[t], ref, rtol=1e-14, atol=0)
            assert abs(w[t].sum() - 1) < 1e-14


def test_route_ties_and_bias():
    logits = np.array([[1.0, 3.0, 3.0, 0.5, 3.0]])
    _, ids, w = O.route(3, logits_in=logits)
    assert list(ids[0]) == [1, 2, 4]
    assert np.allclose(w[0], 1 / 3)
    _, ids, _ = O.route(2, logits_in=logits, bias=np.array([5.0, 0, 0, 0, 0]))
    assert list(ids[0]) == [0, 1]


def test_route_nan_rows():
    """A NaN logit ranks above every number and NaNs tie: the selection equals that of the row
    with every NaN replaced by one common value above all the others (a finite case already
    pinned above), and a selection holding a NaN gets NaN weights.  An all-NaN row (what a NaN
    in x gives) therefore selects experts 0 .. k-1, as an all-equal row does."""
    g = np.random.default_rng(12)
    E, k = 12, 4
    for nan_at in ([3], [7, 2], [0, 5, 11], list(range(E))):
        row = g.standard_normal(E)
        row[nan_at] = np.nan
        repl = np.where(np.isnan(row), np.nanmax(np.append(row, 0.0)) + 1e3, row)
        _, ids, w = O.route(k, logits_in=row[None, :])
        _, ids_r, _ = O.route(k, logits_in=repl[None, :])
        assert list(ids[0]) == list(ids_r[0])
        assert np.isnan(w).all()
        assert ((ids >= 0) & (ids < E)).all()
    _, ids, _ = O.route(k, logits_in=np.full((1, E), np.nan))
    _, ids0, _ = O.route(k, logits_in=np.zeros((1, E)))
    assert list(ids[0]) == list(ids0[0]) == list(range(k))


def test_route_from_bf16_matches_bruteforce_dot():
    x = synth.activations(0, 0, 2, 64)
    wr = synth.router_weights(0, 0, 4, 64)
    logits, _, _ = O.route(2, x, wr)
    for t in range(2):
        for e in range(4):
            acc = 0.0
            for h in range(64):
                a = np.array([np.uint32(x[t, h]) << 16], dtype=np.uint32).view(np.float32)[0]
                b = np.array([np.uint32(wr[e, h]) << 16], dtype=np.uint32).view(np.float32)[0]
                acc += float(a) * float(b)
            assert abs(acc - logits[t, e]) <= 1e-15 * 64


# ----------------------------------------------------------------------------- permute
def test_permute_vs_stable_sort():
    g = np.random.default_rng(3)
    for T, k, E in [(1, 8, 256), (7, 2, 8), (64, 8, 256), (5, 3, 4)]:
        ids = np.stack([g.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
        sp, off, pp = O.permute(ids, E)
        flat = ids.reshape(-1)
        ref = sorted(range(flat.size), key=lambda f: flat[f])     # Python's sort is stable
        assert list(sp) == ref
        assert list(off) == [0] + list(np.cumsum(np.bincount(flat, minlength=E)))
        assert (sp[pp] == np.arange(flat.size)).all()
        assert (np.diff(flat[sp]) >= 0).all()


def test_permute_drops_unroutable_ids():
    """Ids outside [0, E) take no sorted position: the routed pairs are Python's stable sort
    of the valid ids, pair_pos is -1 for the others, offsets end at the routed count and
    sorted_pair is -1 past it."""
    g = np.random.default_rng(13)
    E, T, k = 6, 9, 3
    ids = g.integers(-2, E + 2, (T, k)).astype(np.int32)
    sp, off, pp = O.permute(ids, E)
    flat = ids.reshape(-1)
    valid = [f for f in range(flat.size) if 0 <= flat[f] < E]
    ref = sorted(valid, key=lambda f: flat[f])
    n = len(ref)
    assert list(sp[:n]) == ref and (sp[n:] == -1).all()
    assert off[E] == n and list(off) == [0] + list(np.cumsum(np.bincount(flat[valid], minlength=E)))
    assert all(pp[f] == -1 for f in range(flat.size) if f not in valid)
    assert all(sp[pp[f]] == f for f in valid)


def test_combine_skips_unrouted_pairs():
    """A pair with pair_pos -1 contributes exactly what a zero routing weight would."""
    g = np.random.default_rng(14)
    yp = g.standard_normal((5, 7))
    w = g.random((3, 2))
    pp = np.array([4, -1, 0, 2, -1, 3])
    w0 = w.copy()
    w0[0, 1] = w0[2, 0] = 0.0
    pp0 = np.where(pp < 0, 1, pp)
    assert np.array_equal(O.combine(yp, w, pp), O.combine(yp, w0, pp0))


# ----------------------------------------------------------------------------- expert math
def test_silu_vs_scipy():
    g = np.linspace(-30, 30, 10001)
    assert np.allclose(O.silu(g), g * scipy.special.expit(g), rtol=1e-15, atol=1e-300)


def test_swiglu_bruteforce_loops():
    g = np.random.default_rng(4)
    K, N, n = 8, 6, 3
    a = g.standard_normal((n, K))
    Wg, Wu, Wd = g.standard_normal((N, K)), g.standard_normal((N, K)), g.standard_normal((K, N))
    h, y = O.swiglu_expert(a, Wg, Wu, Wd)
    for r in range(n):
        hh = []
        for i in range(N):
            gi = sum(a[r, c] * Wg[i, c] for c in range(K))
            ui = sum(a[r, c] * Wu[i, c] for c in range(K))
            hh.append(gi / (1 + math.exp(-gi)) * ui)
        assert np.allclose(h[r], hh, rtol=1e-13)
        for o in range(K):
            assert math.isclose(y[r, o], sum(hh[i] * Wd[o, i] for i in range(N)), rel_tol=1e-12, abs_tol=1e-12)


def test_onehot_input_returns_ternary_column():
    codes, scales = synth.stq1_matrix(9, 0, 0, 0, 16 * 256)
    W = O.stq1_matrix(codes, scales, 16, 256)
    j = 77
    a = np.zeros((1, 256))
    a[0, j] = 1.0
    col = (a @ W.T)[0]
    dv = O.fp16_to_f64(scales)
    for r in range(16):
        blk = (r * 256 + j) // 256
        assert col[r] in (0.0, dv[blk], -dv[blk])
    assert (col == 0).mean() < 0.6


def test_mxfp4_unit_scale_integer_matmul():
    """Scale bytes 127 and integer-valued activations: the MX gate stage equals an integer
    matmul computed with Python ints."""
    g = np.random.default_rng(5)
    N, K = 5, 64
    codes = g.integers(0, 256, (N, K // 2), dtype=np.uint8)
    W = O.mxfp4_matrix(codes, np.full((N, K // 32), 127, np.uint8), N, K)
    assert np.all(W == np.round(W * 2) / 2)
    act = g.integers(-16, 17, (3, K)).astype(np.float64)
    act[:, 0] = 256.0
    act[:, 32] = -256.0
    q, s = O.mx_quantize_e4m3(act)
    assert (s == 127).all()
    a = O.mx_dequantize_e4m3(q, s)
    assert (a == act).all()
    got = a @ W.T
    Wi = (W * 2).astype(np.int64).tolist()
    for r in range(3):
        for o in range(N):
            ref = sum(int(act[r, c]) * Wi[o][c] for c in range(K))
            assert got[r, o] * 2 == ref


def test_mxfp4_nibble_order():
    codes = np.array([[0x2A, 0x00] * 16], dtype=np.uint8)     # low nibble 0xA = -1, high 0x2 = +1
    W = O.mxfp4_matrix(codes, np.array([[127, 127]], np.uint8), 1, 64)[0]
    assert W[0] == -1.0 and W[1] == 1.0 and W[2] == 0.0 and W[3] == 0.0


def test_combine_identity_single_expert():
    g = np.random.default_rng(6)
    y = g.standard_normal((4, 8))
    ids = np.zeros((4, 1), dtype=np.int32)
    sp, off, pp = O.permute(ids, 1)
    out = O.combine(y, np.ones((4, 1)), pp)
    assert (out == y[pp]).all()
    w = np.array([[0.25, 0.75]] * 2)
    yp = g.standard_normal((4, 3))
    pp2 = np.array([2, 0, 3, 1])
    out = O.combine(yp, w, pp2, y_shared=np.ones((2, 3)), residual=np.full((2, 3), 2.0))
    assert np.allclose(out[0], 3 + 0.25 * yp[2] + 0.75 * yp[0])
    assert np.allclose(out[1], 3 + 0.25 * yp[3] + 0.75 * yp[1])


def test_rmsnorm_closed_form():
    r = np.array([[3.0, 4.0] * 4, [1.0] * 8])
    a = O.bf16_to_f64(O.rmsnorm_bf16(r, eps=0.0))
    s = math.sqrt(12.5)
    assert np.allclose(a[0], [3 / s, 4 / s] * 4, rtol=2 ** -8)
    assert (a[1] == 1.0).all()
    a = O.bf16_to_f64(O.rmsnorm_bf16(np.array([[1e-4] * 8]), eps=1e-6))
    assert np.allclose(a, 1e-4 / math.sqrt(1e-8 + 1e-6), rtol=2 ** -8)


# ----------------------------------------------------------------------------- whole layer, tiny
def test_tiny_layer_bruteforce():
    """Config-0 shapes: the oracle layer equals a pure-Python loop over tokens and slots
    that decodes every weight through stq1_pattern one group at a time."""
    c = synth.cfg(0)
    x = synth.activations(c.seed, 0, c.T, c.H)
    wr = synth.router_weights(c.seed, 0, c.E, c.H)
    fam = [synth.stq1_family(c.seed, 0, m, c.E, c.I * c.H) for m in range(3)]
    shapes = [(c.I, c.H), (c.I, c.H), (c.H, c.I)]

    def get_w(e, m):
        return O.stq1_matrix(fam[m][0][e], fam[m][1][e], *shapes[m])

    res = O.moe_layer(x, c.k, get_w, "stq1", wr_bits=wr)
    xf = O.bf16_to_f64(x)

    def weight(e, m, r, col):
        N, K = shapes[m]
        flat = r * K + col
        blk, within = divmod(flat, 256)
        grp, lane = divmod(within, 4)
        pbytes = fam[m][0][e][blk * 40:(blk + 1) * 40]
        nib = (pbytes[grp // 2] >> (4 * (grp % 2))) & 15
        hb = (int.from_bytes(bytes(pbytes[32:40]), "little") >> grp) & 1
        d = float(np.array([fam[m][1][e][blk]], np.uint16).view(np.float16)[0])
        return O.stq1_pattern(int(nib) | (hb << 4))[lane] * d

    for t in range(c.T):
        out = np.zeros(c.H)
        for j in range(c.k):
            e = int(res["ids"][t, j])
            hvec = []
            for i in range(c.I):
                gi = sum(xf[t, q] * weight(e, 0, i, q) for q in range(c.H))
                ui = sum(xf[t, q] * weight(e, 1, i, q) for q in range(c.H))
                hvec.append(gi / (1 + math.exp(-gi)) * ui)
            for o in range(c.H):
                out[o] += res["w"][t, j] * sum(hvec[i] * weight(e, 2, o, i) for i in range(c.I))
        assert np.allclose(res["out"][t], out, rtol=1e-10, atol=1e-12)


def _bf16_value(bits):
    """bf16 bits -> Python float through the IEEE binary32 it is the top half of."""
    import struct
    return struct.unpack("<f", struct.pack("<I", int(bits) << 16))[0]


def test_shared_expert_bruteforce_loops():
    """The bf16 shared expert equals pure-Python loops over bf16 bits decoded one by one:
    h_i = silu(sum_c x_c Wg[i,c]) * sum_c x_c Wu[i,c], y_o = sum_i h_i Wd[o,i] (gate inside
    the SiLU, up outside it)."""
    T, H, I = 2, 16, 8
    x = synth.activations(40, 0, T, H)
    wg, wu, wd = synth.shared_weights(40, 0, I, H)
    y = O.shared_expert(x, wg, wu, wd)
    for t in range(T):
        xs = [_bf16_value(v) for v in x[t]]
        h = []
        for i in range(I):
            gi = sum(xs[c] * _bf16_value(wg[i, c]) for c in range(H))
            ui = sum(xs[c] * _bf16_value(wu[i, c]) for c in range(H))
            h.append(gi / (1 + math.exp(-gi)) * ui)
        for o in range(H):
            ref = sum(h[i] * _bf16_value(wd[o, i]) for i in range(I))
            assert math.isclose(y[t, o], ref, rel_tol=1e-12, abs_tol=1e-15)


_E2M1_MAG = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def _mx_brute(vals):
    """MX E4M3 quantise-dequantise of a list whose length is a multiple of 32, by search over
    the finite E4M3 values (torch's float8_e4m3fn decoding of all 256 codes): per group the
    shared exponent floor(log2 amax) - 8 (math.frexp), then each v / 2^X goes to the nearest
    value, a tie to the one with an even code, magnitudes past 448 to 448."""
    codes = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    fin = [(float(v), c) for c, v in enumerate(codes) if np.isfinite(v) and c < 128]
    out = []
    for g0 in range(0, len(vals), 32):
        grp = vals[g0:g0 + 32]
        amax = max(abs(v) for v in grp)
        if amax == 0:
            out += [0.0] * 32
            continue
        X = max(-127, min(127, math.frexp(amax)[1] - 1 - 8))
        for v in grp:
            y = min(abs(v) / 2.0 ** X, 448.0)
            best = min(fin, key=lambda vc: (abs(vc[0] - y), vc[1] % 2))
            out.append(math.copysign(best[0], v) * 2.0 ** X)
    return out


def test_expert_ffn_mxfp4_bruteforce():
    """The MXFP4 branch of expert_ffn: x MX-quantised along H, gathered by sorted pair, gate
    and up with E2M1 weights times their UE8M0 group scales, SiLU(gate) * up MX-quantised
    along I, then down -- equal to pure-Python loops with a brute-force MX quantiser and a
    hand-decoded E2M1 table."""
    g = np.random.default_rng(41)
    T, H, I, E, k = 3, 64, 32, 3, 2
    x = synth.f32_to_bf16_bits(g.standard_normal((T, H)).astype(np.float32))
    shp = [(I, H), (I, H), (H, I)]
    fam = [(g.integers(0, 256, (E, n, kk // 2), dtype=np.uint8),
            (127 + g.integers(-3, 2, (E, n, kk // 32))).astype(np.uint8)) for n, kk in shp]
    ids = np.array([[0, 2], [2, 1], [0, 1]], dtype=np.int32)
    sp, off, _ = O.permute(ids, E)
    get_w = lambda e, m: O.mxfp4_matrix(fam[m][0][e], fam[m][1][e], *shp[m])
    y, h = O.expert_ffn(x, ids, sp, off, get_w, "mxfp4")

    def w_at(e, m, r, c):
        code = int(fam[m][0][e][r, c // 2]) >> (4 * (c % 2)) & 15
        mag = _E2M1_MAG[code & 7] * 2.0 ** (int(fam[m][1][e][r, c // 32]) - 127)
        return -mag if code & 8 else mag

    xq = [_mx_brute([_bf16_value(v) for v in x[t]]) for t in range(T)]
    for e in range(E):
        for pos in range(off[e], off[e + 1]):
            a = xq[sp[pos] // k]
            hv = []
            for i in range(I):
                gi = sum(a[c] * w_at(e, 0, i, c) for c in range(H))
                ui = sum(a[c] * w_at(e, 1, i, c) for c in range(H))
                hv.append(gi / (1 + math.exp(-gi)) * ui)
            hq = _mx_brute(hv)
            assert np.array_equal(h[pos], hq)
            for o in range(H):
                ref = sum(hq[i] * w_at(e, 2, o, i) for i in range(I))
                assert math.isclose(y[pos, o], ref, rel_tol=1e-12, abs_tol=1e-15)


# ----------------------------------------------------------------------------- STQ1_0 encoders
# "Hy4-preview-GGUF" (AngelSlim), section 3, Our encoder: the upstream encoder (d = amax,
# zero at the smallest |x|) and the weighted least-squares one (LS scale, imatrix-weighted
# incremental-cost zero placement, 3 alternating rounds).

def _grid_block_inputs(g, n_blk):
    """Weights already on the ternary grid: random patterns and fp16 scales, x = d * lanes."""
    z = g.integers(0, 4, n_blk * 64)
    s = g.integers(0, 8, n_blk * 64)
    d = np.abs(g.standard_normal(n_blk) * 0.02).astype(np.float16)
    d[d == 0] = np.float16(0.01)
    lanes = np.array([O.stq1_pattern(int(p)) for p in (8 * z + s)], dtype=np.float64)
    x = (lanes.reshape(n_blk, 256) * d.astype(np.float64)[:, None]).reshape(-1)
    return x, z, s, d.view(np.uint16)


@pytest.mark.parametrize("method", ["upstream", "wls"])
def test_stq1_encode_recovers_grid_inputs(method):
    """Inputs already on the grid (what the upstream encoder was made for: QAT weights) come
    back exactly from both encoders, with or without an imatrix."""
    g = np.random.default_rng(31)
    x, z, s, d_bits = _grid_block_inputs(g, 12)
    want = O.stq1_pack(z, s, d_bits)
    for imat in (None, np.exp(g.standard_normal(512))):
        codes, scales = O.stq1_encode(x, 512, imatrix=imat, method=method)
        assert (codes == want[0]).all() and (scales == want[1]).all()


def test_stq1_ls_scale_matches_weighted_lstsq():
    """For a fixed selection, d minimises sum w (x - d sel)^2: numpy's least-squares solver on
    the sqrt(w)-weighted one-column system gives the same d."""
    g = np.random.default_rng(32)
    K = 256
    x = g.standard_normal(3 * 256) * 0.03
    w = np.exp(g.standard_normal(K))
    xb, wb = O._stq_blocks(x, K, w)
    z = g.integers(0, 4, (3, 64))
    d = O.stq1_ls_scale(xb, wb, z)
    for b in range(3):
        sel = np.sign(xb[b]) + (xb[b] == 0)
        sel[np.arange(64), z[b]] = 0
        a = (np.sqrt(wb[b]) * sel).reshape(-1, 1)
        ref = np.linalg.lstsq(a, (np.sqrt(wb[b]) * xb[b]).reshape(-1), rcond=None)[0][0]
        assert abs(d[b] - ref) <= 1e-12 * abs(ref)


def test_stq1_zero_placement_is_the_best_zero_for_the_group():
    """Given d, zeroing the lane of least incremental cost is the zero choice of least
    weighted group error sum_j w_j (x_j - d q_j)^2 (q = sign(x) on kept lanes): brute force
    over the four choices."""
    g = np.random.default_rng(33)
    x = g.standard_normal(2 * 256) * 0.03
    w = np.exp(g.standard_normal(256))
    xb, wb = O._stq_blocks(x, 256, w)
    d = np.array([0.02, 0.05])
    z = O.stq1_zero_placement(xb, wb, d)
    for b in range(2):
        for grp in range(64):
            errs = []
            for zz in range(4):
                q = np.sign(xb[b, grp])
                q[zz] = 0
                errs.append((wb[b, grp] * (xb[b, grp] - d[b] * q) ** 2).sum())
            assert z[b, grp] == int(np.argmin(errs))


def test_stq1_wls_alternation_never_increases_error_and_beats_upstream():
    """Each half-step of the alternation minimises the weighted error over its own variable,
    so the error never rises from round to round, and the result is never worse than the
    upstream encoder's (whose selection the first LS step starts from)."""
    g = np.random.default_rng(34)
    K = 512
    # heavy-tailed rows (Student t, 3 degrees of freedom) make amax a poor scale
    x = g.standard_t(3, 16 * 256) * 0.02
    w = np.exp(g.standard_normal(K))
    xb, wb = O._stq_blocks(x, K, w)

    def err(z, d):
        q = np.sign(xb) + (xb == 0)
        q[np.arange(4)[None, None, :] == z[:, :, None]] = 0
        return (wb * (xb - d[:, None, None] * q) ** 2).sum(axis=(1, 2))

    z = np.argmin(np.abs(xb), axis=2)
    e_up = err(z, np.abs(xb).max(axis=(1, 2)))
    prev = e_up
    for _ in range(O.STQ_ENC_ROUNDS):
        d = O.stq1_ls_scale(xb, wb, z)
        e1 = err(z, d)
        z = O.stq1_zero_placement(xb, wb, d)
        e2 = err(z, d)
        assert (e1 <= prev * (1 + 1e-12)).all() and (e2 <= e1 * (1 + 1e-12)).all()
        prev = e2
    # the oracle's encoder is this sequence plus a final LS fit
    zf, _, df = O.stq1_encode_parts(x, K, w, "wls")
    assert (err(zf.reshape(-1, 64), df) <= prev * (1 + 1e-12)).all()
    assert (err(zf.reshape(-1, 64), df) < e_up).all()
    # and after fp16 rounding of d the packed encodings keep the order on these rows
    cu, su = O.stq1_encode(x, K, w, "upstream")
    cw, sw = O.stq1_encode(x, K, w, "wls")
    assert O.stq1_weighted_ssd(x, K, cw, sw, w).sum() < 0.5 * O.stq1_weighted_ssd(x, K, cu, su, w).sum()


def test_stq1_encode_signs_ties_and_zero_blocks():
    """Kept lanes carry sign(x) (0 counts as positive), the first lane wins a tie for the
    zero, and an all-zero block encodes d = 0."""
    x = np.zeros(256)
    x[:4] = [0.5, -0.5, 0.25, -0.25]           # tie |x| between lanes 2 and 3: lane 2 zeroed
    x[4:8] = [0.0, 0.0, 1.0, -1.0]             # tie at 0 between lanes 0 and 1: lane 0 zeroed
    z, s, d = O.stq1_encode_parts(x, 256, method="upstream")
    assert z[0] == 2 and s[0] == 0b110         # kept lanes 0, 1, 3: +, -, - (bit i: i-th kept lane)
    assert z[1] == 0 and s[1] == 0b100         # kept lanes 1, 2, 3: +0 -> +, +, -
    assert d[0] == 1.0
    codes, scales = O.stq1_encode(np.zeros(512), 256)
    assert (scales == 0).all() and (O.stq1_decode(codes, scales) == 0).all()


# ----------------------------------------------------------------------------- MXFP8 shared expert
def test_mxfp8_weight_decode_vs_torch():
    """MXFP8 weights ("Hy4-preview-SF-WFP4AFP8", Quant Diff table: shared experts MXFP8 W8A8
    g32) decode as torch's float8_e4m3fn value times 2^(scale byte - 127), per 32 inputs."""
    codes, scales = synth.mxfp8_matrix(5, 0, 0, 8, 64)
    assert not ((codes == 0x7F) | (codes == 0xFF)).any()
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).double().numpy()
    ref = ref * np.exp2(scales.astype(np.float64) - 127).repeat(32, axis=1)
    assert (O.mx_dequantize_e4m3(codes, scales) == ref).all()


def test_mxfp8_shared_expert_is_the_swiglu_of_dequantised_operands():
    """The W8A8 shared expert with x already on its MX grid (so quantising x changes nothing)
    and weights decoding to small integers: gate and up are integer matmuls, checked through
    a down projection that picks one h entry (unit weight on the grid) per output."""
    g = np.random.default_rng(35)
    T, H, I = 3, 64, 32
    xv = g.integers(-7, 8, (T, H)).astype(np.float64)
    xv[:, 0] = 7                                    # each group's max 7: scale 2^(2-8), exact
    xv[:, 32] = 7
    x_bits = O.f64_to_bf16_bits(xv)
    # E4M3 codes of small integers at scale byte 127: values in {-3..3}
    ints = g.integers(-3, 4, (I, H))
    code_of = {0: 0x00, 1: 0x38, 2: 0x40, 3: 0x44}
    enc = np.vectorize(lambda v: code_of[abs(v)] | (0x80 if v < 0 else 0))
    wg = (enc(ints).astype(np.uint8), np.full((I, H // 32), 127, np.uint8))
    ints_u = g.integers(-3, 4, (I, H))
    wu = (enc(ints_u).astype(np.uint8), np.full((I, H // 32), 127, np.uint8))
    eye = np.zeros((I, I), dtype=np.int64)
    eye[np.arange(I), np.arange(I)] = 1
    wd = (enc(eye).astype(np.uint8), np.full((I, I // 32), 127, np.uint8))
    y = O.shared_expert_mxfp8(x_bits, wg, wu, wd)[:, :I]
    gate = (xv.astype(np.int64) @ ints.T).astype(np.float64)
    up = (xv.astype(np.int64) @ ints_u.T).astype(np.float64)
    h = gate / (1 + np.exp(-gate)) * up
    hq = O.mx_dequantize_e4m3(*O.mx_quantize_e4m3(h))
    assert np.array_equal(y, hq)
