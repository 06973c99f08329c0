"""Pure-Python fp64 brute force for tiny inputs -- TEST INFRASTRUCTURE.

Written independently of the C oracle, as a second reading of the same
definition:

* group of 1-indexed query head h is ceil(h / (H/G)), the form printed in the
  "GQA reading notes" (zhongzhuzhou.org), section "方法详解 > GQA 架构";
* head_h = softmax(q_h K_g^T / sqrt(d)) V_g, the plain softmax with no
  maximum subtracted (valid only for the small scores of tiny tests);
* prefill under a causal mask attends prompt position i to keys 0..i
  ("从MHA到GQA", gzher.com, the prefill/decode discussion).

Inputs are nested Python lists of floats (already widened); nothing here
calls numpy or C.
"""
from __future__ import annotations

import math


def _group_1indexed(h1: int, H: int, G: int) -> int:
    """ceil(h1 / (H/G)) for 1-indexed head h1, with H/G an integer."""
    per = H // G
    return -(-h1 // per)


def _attend(qrow, krows, vrows, scale):
    e = [math.exp(scale * sum(a * b for a, b in zip(qrow, kr))) for kr in krows]
    z = sum(e)
    d = len(vrows[0])
    return [sum(e[j] * vrows[j][c] for j in range(len(krows))) / z for c in range(d)]


def decode(q, k, v, seqlens, scale):
    """q[B][Hq][d], k/v[B][Lmax][Hkv][d] -> out[B][Hq][d]."""
    B, H = len(q), len(q[0])
    G = len(k[0][0])
    out = []
    for b in range(B):
        n = seqlens[b]
        rows = []
        for h1 in range(1, H + 1):
            g = _group_1indexed(h1, H, G) - 1
            if n == 0:
                rows.append([0.0] * len(q[b][h1 - 1]))
                continue
            krows = [k[b][j][g] for j in range(n)]
            vrows = [v[b][j][g] for j in range(n)]
            rows.append(_attend(q[b][h1 - 1], krows, vrows, scale))
        out.append(rows)
    return out


def prefill(q, k, v, causal, scale):
    """q[B][P][Hq][d], k/v[B][P][Hkv][d] -> out[B][P][Hq][d]."""
    B, P, H = len(q), len(q[0]), len(q[0][0])
    G = len(k[0][0])
    out = []
    for b in range(B):
        pos_rows = []
        for i in range(P):
            n = i + 1 if causal else P
            head_rows = []
            for h1 in range(1, H + 1):
                g = _group_1indexed(h1, H, G) - 1
                krows = [k[b][j][g] for j in range(n)]
                vrows = [v[b][j][g] for j in range(n)]
                head_rows.append(_attend(q[b][i][h1 - 1], krows, vrows, scale))
            pos_rows.append(head_rows)
        out.append(pos_rows)
    return out


def decode_ex(q, k, v, seqlens, scale, window=0, block_table=None, block_size=0):
    """Several new tokens per sequence, optional window and paged addressing.

    q[B][T][Hq][d].  k/v hold already-widened (and, for FP8 rows, already
    scaled) values: [B][Lmax][Hkv][d], or a pool [nblocks][block_size][Hkv][d]
    addressed through block_table[b][j // block_size].  Token t of sequence b
    is at position seqlens[b] - T + t and sees the keys up to it, the last
    ``window`` of them when window > 0.
    """
    B, T, H = len(q), len(q[0]), len(q[0][0])
    G = len(k[0][0])
    out = []
    for b in range(B):
        tok_rows = []
        for t in range(T):
            pos = seqlens[b] - T + t
            first = max(0, pos - window + 1) if window > 0 else 0
            keys = list(range(first, pos + 1))
            head_rows = []
            for h1 in range(1, H + 1):
                g = _group_1indexed(h1, H, G) - 1
                if block_table is None:
                    krows = [k[b][j][g] for j in keys]
                    vrows = [v[b][j][g] for j in keys]
                else:
                    krows = [k[block_table[b][j // block_size]][j % block_size][g] for j in keys]
                    vrows = [v[block_table[b][j // block_size]][j % block_size][g] for j in keys]
                head_rows.append(_attend(q[b][t][h1 - 1], krows, vrows, scale))
            tok_rows.append(head_rows)
        out.append(tok_rows)
    return out
