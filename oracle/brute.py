"""Scalar brute-force causal GQA: pure-Python loops, ``math.fsum`` and ``math.exp``.

TEST INFRASTRUCTURE ONLY (like ``oracle.oracle``): a second, independent
writing of the same definition, used on tiny shapes to cross-check the NumPy
oracle. It touches no NumPy arithmetic: every score, weight and output is a
Python float built from exactly rounded sums.

For query head ``h`` the KV head is ``h // (n_heads // n_kv_heads)``; query
row ``i`` at absolute position ``position_offset + i`` sees keys
``j <= position_offset + i`` (kopitiam-runtime 0.2.4 ``src/attention.rs``,
module doc and ``causal_mask``). Weights are ``exp(s_j - max s) / sum``.
"""
from __future__ import annotations

import math

__all__ = ["gqa_attention", "gqa_attention_arms"]


def gqa_attention(q, k, v, n_heads, n_kv_heads, position_offset, scale):
    """``q[i][h][c]``, ``k[j][g][c]``, ``v[j][g][c]`` nested sequences -> ``out[i][h][c]``."""
    assert n_kv_heads > 0 and n_heads % n_kv_heads == 0
    group = n_heads // n_kv_heads
    seq_q, seq_kv = len(q), len(k)
    dv = len(v[0][0]) if seq_kv else 0
    out = []
    for i in range(seq_q):
        row = []
        last = position_offset + i
        visible = [j for j in range(seq_kv) if j <= last]
        for h in range(n_heads):
            g = h // group
            s = [scale * math.fsum(float(q[i][h][c]) * float(k[j][g][c]) for c in range(len(q[i][h])))
                 for j in visible]
            m = max(s)
            w = [math.exp(x - m) for x in s]
            z = math.fsum(w)
            row.append([math.fsum(w[n] * float(v[j][g][c]) for n, j in enumerate(visible)) / z
                        for c in range(dv)])
        out.append(row)
    return out


def gqa_attention_arms(q, k, v, n_heads, n_kv_heads, position_offset, scale, window=0,
                       softcap=0.0, alibi=None, sinks=None):
    """The same with a layer's optional arms: key ``j`` is visible to the row at
    position ``p`` iff ``j <= p`` and (``window <= 0`` or ``p - j < window``); the
    logit is ``scale * q.k``, then ``softcap * tanh(logit / softcap)`` if
    ``softcap > 0``, plus ``alibi[h] * (j - p)``; the softmax denominator also
    counts ``exp(sinks[h])``, a logit with no value."""
    assert n_kv_heads > 0 and n_heads % n_kv_heads == 0
    group = n_heads // n_kv_heads
    dv = len(v[0][0]) if len(k) else 0
    out = []
    for i in range(len(q)):
        p = position_offset + i
        visible = [j for j in range(len(k)) if j <= p and (window <= 0 or p - j < window)]
        row = []
        for h in range(n_heads):
            g = h // group
            logits = []
            for j in visible:
                x = scale * math.fsum(float(q[i][h][c]) * float(k[j][g][c])
                                      for c in range(len(q[i][h])))
                if softcap > 0:
                    x = softcap * math.tanh(x / softcap)
                if alibi is not None:
                    x += float(alibi[h]) * (j - p)
                logits.append(x)
            extra = [float(sinks[h])] if sinks is not None else []
            m = max(logits + extra)
            w = [math.exp(x - m) for x in logits]
            z = math.fsum(w + [math.exp(x - m) for x in extra])
            row.append([math.fsum(w[n] * float(v[j][g][c]) for n, j in enumerate(visible)) / z
                        for c in range(dv)])
        out.append(row)
    return out
