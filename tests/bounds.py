"""Per-element error bounds derived from each HIP path's arithmetic (test helpers).

The stated tolerance (fp32 inputs: max-abs 1e-5; bf16 inputs:
2e-2 + 1e-2 |ref|) is loose enough to pass a dropped 32-key step or a
mis-scaled softmax at long lengths.  Beside it, parity tests assert a bound
that follows from how each kernel computes, using error-model terms the
oracle reports for every output element (``reference.decode_ex(...,
terms=True)``):

    sigma_c = sum_j w_j |v_jc - ref_c|    spread of V about the output
    mu_c    = sum_j w_j |v_jc|            weighted mean magnitude of V
    kappa   = |scale| max_j sum_c |q_c k_jc|   largest absolute score sum
    n       = visible keys of the row

with w_j the exact softmax weights.  U = 2^-24 is the fp32 unit roundoff.

Scores (every path).  Products of bf16 (or FP8 converted to bf16) values are
exact in fp32; the sum over d products, the multiply by scale*log2(e) (and by
k_scale for FP8 caches) and the subtraction of the reference round at most
d + 8 times relative to sum_c |q_c k_jc| scaled, so a score's exponent is off
by at most (d + 8) U kappa / ln 2 in base 2; the exponent's own rounding
(at most 2 kappa / ln 2 + 9 units of U) and v_exp_f32 add at most 16 U: each
weight carries a relative error of at most  e_w = (d + 8) U kappa + 16 U.
A relative error e_j in weights shared by numerator and denominator moves
the output by at most max_j e_j * sigma_c (first order).

Accumulation.  The weighted sum and the weight sum are sums of n terms in
fp32 (matrix-core accumulation, online rescaling, the combine of the waves'
or pieces' parts, the final division): each contributes at most
(n + 64) U relative to sum_j w_j |v_j|, i.e. 2 (n + 64) U mu_c together.

bf16 carries 8 significant bits: rounding to nearest is off by at most half
an ulp, 2^-8 of the value; truncation by less than an ulp, 2^-7.

Decode (bf16 or FP8 cache, bf16 output).  Weights enter P*V as hi + lo bf16
terms (hi the truncation, off by less than 2^-7; lo that remainder rounded to
nearest, off by at most 2^-8 of it): relative error below 2^-15, in the
numerator only, so 2^-15 mu_c.  The bf16 output rounds to nearest even: at
most 2^-8 of the fp32 value (plus 4 U for the final scale multiply).

Prefill (bf16 output).  Weights are rounded to bf16 (relative 2^-8) and the
same rounded weights form numerator and denominator (the weight sum is a
matrix product against ones), so the rounding moves the output by at most
2^-8 / (1 - 2^-8) * sigma_c (to first order; 1.01 * 2^-8 taken).

fp32 decode (fp32 output).  Scores and weights as above (the query is
rounded once when it is multiplied by the scale); no bf16 terms.
"""
from __future__ import annotations

import numpy as np

from oracle import reference as orc

U = 2.0 ** -24
BF16_OUT = 2.0 ** -8 + 4 * U   # bf16 rounding of the result, plus the last multiply
SLACK = 1.0 + 2.0 ** -8        # the output rounding also scales the fp32 error


def weight_rel_err(kappa, d):
    return (d + 8) * U * np.asarray(kappa, np.float64) + 16 * U


def decode_bound(ref, sigma, mu, kappa, n, d):
    """bf16 output, hi + lo weights (gqa_decode bf16, gqa_decode_ex)."""
    ew = weight_rel_err(kappa, d)[..., None]
    nn = np.asarray(n, np.float64)[..., None]
    fp32 = ew * sigma + 2.0 ** -15 * mu + 2.0 * (nn + 64.0) * U * mu
    return BF16_OUT * np.abs(ref) + SLACK * fp32


def decode_bound_f32(ref, sigma, mu, kappa, n, d):
    """fp32 inputs and output (the vector-ALU decode kernel)."""
    ew = weight_rel_err(kappa, d + 1)[..., None]
    nn = np.asarray(n, np.float64)[..., None]
    return 4 * U * np.abs(ref) + ew * sigma + 2.0 * (nn + 64.0) * U * mu


def prefill_bound(ref, sigma, mu, kappa, n, d):
    """bf16 output, bf16 weights shared by numerator and denominator."""
    ew = weight_rel_err(kappa, d)[..., None]
    nn = np.asarray(n, np.float64)[..., None]
    fp32 = (1.01 * 2.0 ** -8 + ew) * sigma + 2.0 * (nn + 64.0) * U * mu
    return BF16_OUT * np.abs(ref) + SLACK * fp32


def assert_within(got, ref, bound, what):
    """Every element inside its derived bound; returns the largest err/bound."""
    got = np.asarray(got, np.float64)
    err = np.abs(got - ref)
    bad = ~(err <= bound)
    if bad.any():
        i = np.unravel_index(int(np.argmax(np.where(bad, err / np.maximum(bound, 1e-300), 0))), err.shape)
        raise AssertionError("%s: %d element(s) above the derived bound; worst at %s: err %.3g, "
                             "bound %.3g, ref %.4g" % (what, int(bad.sum()), i, err[i], bound[i], ref[i]))
    ratio = np.divide(err, bound, out=np.zeros_like(err), where=bound > 0)
    return float(ratio.max(initial=0.0))


# --- oracle outputs with their terms, per kind of case ----------------------

def decode_terms(c, rows=None):
    """Oracle of a plain-decode case (q [B,Hq,d]) with its terms.

    Runs through the extended oracle with one new token per sequence, whose
    output equals oracle_decode bit for bit.  rows: flat b*Hq + h indices,
    as for reference.decode (None = all).  Rows of zero-length sequences
    are 0 with zero terms.  Returns (ref, sigma, mu, kappa, n), ref shaped
    [B,Hq,d] or [len(rows),d].
    """
    B, Hq, d = c.q.shape
    sl = np.asarray(c.seqlens, np.int32)
    flat = np.arange(B * Hq) if rows is None else np.asarray(rows, np.int64)
    n = sl[flat // Hq].astype(np.int64)
    keep = n > 0
    ref = np.zeros((flat.size, d))
    sig, mu, kap = np.zeros_like(ref), np.zeros_like(ref), np.zeros(flat.size)
    if keep.any():
        q1 = np.ascontiguousarray(c.q[:, None])
        o, s, m, k = orc.decode_ex(q1, c.k, c.v, np.maximum(sl, 1), c.scale, rows=flat[keep],
                                   terms=True)
        ref[keep], sig[keep], mu[keep], kap[keep] = o, s, m, k
    if rows is None:
        shp = (B, Hq, d)
        return ref.reshape(shp), sig.reshape(shp), mu.reshape(shp), kap.reshape(B, Hq), n.reshape(B, Hq)
    return ref, sig, mu, kap, n


def prefill_terms(p, rows=None):
    """Oracle of a causal prefill case with its terms: the prompt's P
    positions are P new tokens over the prompt's own K/V (equal to
    oracle_prefill bit for bit).  rows: flat (b*P + i)*Hq + h indices."""
    B, P, Hq, d = p.q.shape
    res = orc.decode_ex(p.q, p.k, p.v, np.full(B, P, np.int32), p.scale, rows=rows, terms=True)
    flat = np.arange(B * P * Hq) if rows is None else np.asarray(rows, np.int64)
    n = (flat // Hq) % P + 1
    if rows is None:
        n = n.reshape(B, P, Hq)
    return res + (n,)


def ex_terms(c, rows=None):
    """Oracle of an extended-decode case with its terms.  rows: flat
    ((b*T + t)*Hq + h) indices."""
    B, T, Hq, d = c.q.shape
    res = orc.decode_ex(c.q, c.k, c.v, c.seqlens, c.scale, k_scale=c.k_scale, v_scale=c.v_scale,
                        block_table=c.block_table, block_size=c.block_size, window=c.window,
                        rows=rows, kv_format=c.kv_format or "e4m3", terms=True)
    flat = np.arange(B * T * Hq) if rows is None else np.asarray(rows, np.int64)
    t = (flat // Hq) % T
    pos = np.asarray(c.seqlens, np.int64)[flat // (Hq * T)] - T + t
    lo = np.maximum(0, pos - c.window + 1) if c.window > 0 else np.zeros_like(pos)
    n = pos - lo + 1
    if rows is None:
        n = n.reshape(B, T, Hq)
    return res + (n,)
