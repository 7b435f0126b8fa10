"""Shared test plumbing: seeded layer inputs (from synth), device upload, oracle weight
providers and the error metric.  No arithmetic of the layer lives here."""
from __future__ import annotations

import numpy as np

import synth
from oracle import moe_oracle as O

TOL = 2e-3   # max |out - ref| / RMS(ref row), fp32 accumulation vs the float64 oracle


def shapes(c):
    return [(c.I, c.H), (c.I, c.H), (c.H, c.I)]


def layer_inputs(c, layer=0, with_routed=True):
    """numpy inputs of one layer of config c."""
    inp = dict(x=synth.activations(c.seed, layer, c.T, c.H))
    if c.logits_given:
        inp["logits_in"] = synth.prefill_logits(c.seed, layer, c.T, c.E)
        inp["wr"] = None
    else:
        inp["wr"] = synth.router_weights(c.seed, layer, c.E, c.H)
        inp["logits_in"] = None
    inp["bias"] = synth.zipf_bias(c.seed, layer, c.E) if c.zipf else None
    if with_routed:
        if c.fmt == "stq1":
            inp["routed"] = [synth.stq1_family(c.seed, layer, m, c.E, c.I * c.H) for m in range(3)]
        else:
            sh = shapes(c)
            inp["routed"] = [synth.mxfp4_family(c.seed, layer, m, c.E, *sh[m]) for m in range(3)]
    inp["shared"] = synth.shared_weights(c.seed, layer, c.I, c.H) if c.shared else None
    return inp


def oracle_weights(c, routed, cache=None):
    """get_w(e, m) for the oracle from the numpy families (decoded lazily, cached)."""
    sh = shapes(c)
    cache = {} if cache is None else cache

    def get_w(e, m):
        key = (e, m)
        if key not in cache:
            codes, scales = routed[m]
            if c.fmt == "stq1":
                cache[key] = O.stq1_matrix(codes[e], scales[e], *sh[m])
            else:
                cache[key] = O.mxfp4_matrix(codes[e], scales[e], *sh[m])
        return cache[key]

    return get_w


def oracle_weights_regen(c, layer):
    """get_w(e, m) that regenerates one expert matrix from its seeded stream."""
    sh = shapes(c)

    def get_w(e, m):
        n = sh[m][0] * sh[m][1]
        codes, scales = synth.stq1_matrix(c.seed, layer, e, m, n)
        return O.stq1_matrix(codes, scales, *sh[m])

    return get_w


def row_err(out, ref):
    """max_i |out - ref| / RMS(ref row), per row."""
    out = np.asarray(out, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rms = np.sqrt(np.mean(ref * ref, axis=-1))
    return np.abs(out - ref).max(axis=-1) / np.maximum(rms, 1e-300)


def near_tie_tokens(logits, k, eps=1e-5):
    """Tokens whose k-th and (k+1)-th largest logits are within eps (several top-k sets are
    then correct given fp32-vs-fp64 accumulation)."""
    s = -np.sort(-np.asarray(logits), axis=1)
    if s.shape[1] <= k:
        return np.zeros(s.shape[0], dtype=bool)
    return (s[:, k - 1] - s[:, k]) <= eps


def valid_selection(logits_row, ids_row, k, eps=1e-5):
    """A top-k choice is valid when every chosen logit is >= the k-th largest - eps, ids
    are distinct and ordered by non-increasing logit (within eps)."""
    lr = np.asarray(logits_row)
    kth = -np.sort(-lr)[k - 1]
    chosen = lr[np.asarray(ids_row)]
    return (len(set(ids_row)) == k and (chosen >= kth - eps).all()
            and (np.diff(chosen) <= eps).all())
