"""Pins of the oracle's error-model terms and of its prefill byte count.

The terms (``reference.decode_ex(..., terms=True)``) feed the derived
tolerances of the parity tests: sigma_c = sum_j w_j |v_jc - out_c|,
mu_c = sum_j w_j |v_jc| and kappa = |scale| max_j sum_c |q_c k_jc|.  They are
checked here against a pure-Python computation from brute-force weights and
against closed forms, and the output returned with them must equal the
oracle's plain outputs bit for bit.
"""
import math

import numpy as np
import pytest

import gqa_inputs as gi
from oracle import counts, reference as orc
from tests.helpers import widen


def _py_terms(qrow, krows, vrows, scale):
    """Pure Python: plain softmax weights (no maximum subtracted), then the terms."""
    e = [math.exp(scale * math.fsum(a * b for a, b in zip(qrow, kr))) for kr in krows]
    z = math.fsum(e)
    w = [x / z for x in e]
    d = len(qrow)
    out = [math.fsum(w[j] * vrows[j][c] for j in range(len(w))) for c in range(d)]
    sig = [math.fsum(w[j] * abs(vrows[j][c] - out[c]) for j in range(len(w))) for c in range(d)]
    mu = [math.fsum(w[j] * abs(vrows[j][c]) for j in range(len(w))) for c in range(d)]
    kap = abs(scale) * max(math.fsum(abs(a) * abs(b) for a, b in zip(qrow, kr)) for kr in krows)
    return out, sig, mu, kap


def _fp8_widen(codes, sc, fmt):
    torch = pytest.importorskip("torch")
    tdt = torch.float8_e4m3fn if fmt == "e4m3" else torch.float8_e5m2
    t = torch.from_numpy(np.ascontiguousarray(codes)).view(tdt).to(torch.float64).numpy()
    return t * np.asarray(sc, np.float64)[:, None]


@pytest.mark.parametrize("kv,paged,window", [("same", False, 0), ("same", True, 3), ("fp8", True, 0),
                                             ("e5m2", False, 4)])
def test_terms_match_pure_python(kv, paged, window):
    c = gi.decode_ex_case(2, 3, 4, 2, 8, 12, [12, 5], "bf16", seed=81, kv=kv, paged=paged,
                          block_size=4, window=window)
    out, sig, mu, kap = orc.decode_ex(c.q, c.k, c.v, c.seqlens, c.scale, k_scale=c.k_scale,
                                      v_scale=c.v_scale, block_table=c.block_table,
                                      block_size=c.block_size, window=window,
                                      kv_format=c.kv_format or "e4m3", terms=True)
    if kv != "same":
        kw, vw = _fp8_widen(c.k, c.k_scale, c.kv_format), _fp8_widen(c.v, c.v_scale, c.kv_format)
    else:
        kw, vw = widen(c.k), widen(c.v)
    q = widen(c.q)
    B, T, Hq, d = c.q.shape
    Hkv = c.k.shape[2]
    for b in range(B):
        for t in range(T):
            pos = int(c.seqlens[b]) - T + t
            lo = max(0, pos - window + 1) if window else 0
            for h in range(Hq):
                g = h // (Hq // Hkv)
                rows = []
                for j in range(lo, pos + 1):
                    if c.block_table is None:
                        rows.append((b, j))
                    else:
                        rows.append((int(c.block_table[b, j // c.block_size]), j % c.block_size))
                kr = [kw[x, y, g].tolist() for x, y in rows]
                vr = [vw[x, y, g].tolist() for x, y in rows]
                po, ps, pm, pk = _py_terms(q[b, t, h].tolist(), kr, vr, c.scale)
                assert np.allclose(out[b, t, h], po, rtol=1e-12, atol=1e-13)
                assert np.allclose(sig[b, t, h], ps, rtol=1e-11, atol=1e-13)
                assert np.allclose(mu[b, t, h], pm, rtol=1e-12, atol=1e-13)
                assert math.isclose(kap[b, t, h], pk, rel_tol=1e-12)


def test_single_key_terms():
    """One visible key: weight 1, so sigma = 0, mu = |v|, kappa = |scale| sum |q||k|."""
    c = gi.decode_case(2, 8, 2, 64, 4, [1, 1], "f32", q_seed=82, kv_seed=83, scale=-0.3)
    out, sig, mu, kap = orc.decode_ex(np.ascontiguousarray(c.q[:, None]), c.k, c.v, c.seqlens,
                                      c.scale, terms=True)
    for b in range(2):
        for h in range(8):
            v0 = widen(c.v[b, 0, h // 4])
            assert np.array_equal(out[b, 0, h], v0)
            assert np.all(sig[b, 0, h] == 0.0)
            assert np.array_equal(mu[b, 0, h], np.abs(v0))
            want = 0.3 * math.fsum(np.abs(widen(c.q[b, h])) * np.abs(widen(c.k[b, 0, h // 4])))
            assert math.isclose(kap[b, 0, h], want, rel_tol=1e-14)


def test_uniform_weight_terms():
    """Scale 0: every visible key weighs 1/n, so the terms are plain means."""
    n = 7
    c = gi.decode_case(1, 4, 1, 16, 9, [n], "bf16", q_seed=84, kv_seed=85, scale=0.0)
    out, sig, mu, kap = orc.decode_ex(np.ascontiguousarray(c.q[:, None]), c.k, c.v, c.seqlens,
                                      0.0, terms=True)
    v = widen(c.v[0, :n, 0])
    mean = np.array([math.fsum(v[:, col]) / n for col in range(16)])
    spread = np.array([math.fsum(np.abs(v[:, col] - mean[col])) / n for col in range(16)])
    mag = np.array([math.fsum(np.abs(v[:, col])) / n for col in range(16)])
    for h in range(4):
        assert np.allclose(out[0, 0, h], mean, rtol=1e-14, atol=1e-15)
        assert np.allclose(sig[0, 0, h], spread, rtol=1e-13, atol=1e-15)
        assert np.allclose(mu[0, 0, h], mag, rtol=1e-14, atol=1e-15)
        assert kap[0, 0, h] == 0.0


def test_terms_leave_outputs_unchanged():
    """With terms requested the outputs stay those of the plain oracles, bit for bit."""
    c = gi.decode_case(3, 16, 4, 128, 300, [300, 77, 1], "bf16", q_seed=86, kv_seed=87)
    plain = orc.decode(c.q, c.k, c.v, c.seqlens, c.scale)
    got = orc.decode_ex(np.ascontiguousarray(c.q[:, None]), c.k, c.v, c.seqlens, c.scale,
                        terms=True)[0]
    assert np.array_equal(got[:, 0], plain)
    p = gi.prefill_case(2, 70, 8, 2, 64, "bf16", seed=88)
    got = orc.decode_ex(p.q, p.k, p.v, np.full(2, 70, np.int32), p.scale, terms=True)[0]
    assert np.array_equal(got, orc.prefill(p.q, p.k, p.v, True, p.scale))
    e = gi.decode_ex_case(2, 3, 8, 2, 128, 64, [64, 9], "bf16", seed=89, kv="fp8", paged=True,
                          block_size=16, window=20)
    kw = dict(k_scale=e.k_scale, v_scale=e.v_scale, block_table=e.block_table, block_size=16,
              window=20)
    assert np.array_equal(orc.decode_ex(e.q, e.k, e.v, e.seqlens, e.scale, terms=True, **kw)[0],
                          orc.decode_ex(e.q, e.k, e.v, e.seqlens, e.scale, **kw))


# --- prefill byte count -------------------------------------------------------

def test_prefill_bytes_by_hand():
    """B=1, P=2, Hq=2, Hkv=1, d=2, bf16: Q and O 1*2*2*2 = 8 elements each,
    K and V 1*2*1*2 = 4 each; 24 elements of 2 bytes = 48 bytes."""
    assert counts.prefill_bytes(1, 2, 2, 1, 2, 2) == 48


def test_prefill_bytes_causal_workload():
    """B=2, P=4096, Hq=32, Hkv=8, d=128, bf16: Q and O 2*4096*32*128*2 B =
    67,108,864 B each, K and V 2*4096*8*128*2 B = 16,777,216 B each."""
    assert counts.prefill_bytes(2, 4096, 32, 8, 128, 2) == 167772160 == 2 * 67108864 + 2 * 16777216


@pytest.mark.parametrize("B,P,Hq,Hkv,d,dtype", [(2, 37, 8, 2, 64, "bf16"), (1, 5, 4, 4, 128, "f32"),
                                                (3, 16, 6, 1, 64, "bf16")])
def test_prefill_bytes_equal_the_buffers(B, P, Hq, Hkv, d, dtype):
    """The count equals the bytes of the buffers one call reads and writes:
    q, k and v as generated, and an output shaped like q; its K/V part is the
    pages' cache formula 2 * L * Hkv * d per sequence times the element size."""
    p = gi.prefill_case(B, P, Hq, Hkv, d, dtype, seed=90)
    elt = p.q.itemsize
    out_bytes = np.empty_like(p.q).nbytes
    assert counts.prefill_bytes(B, P, Hq, Hkv, d, elt) == p.q.nbytes + p.k.nbytes + p.v.nbytes + out_bytes
    assert p.k.nbytes + p.v.nbytes == counts.kv_cache_bytes(P, Hkv, d, elt, batch=B)
