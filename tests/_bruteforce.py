"""Arbitrary-precision brute force for tiny attention problems (a pin, not an oracle).

Pure-Python loops over mpmath numbers at 50 significant digits.  It is written
from the softmax's own definition -- P_ij = exp(s_ij) / sum_j exp(s_ij), with no
max subtraction -- so it shares neither code nor formulation with the fp64
oracle, whose max-shifted logsumexp it therefore checks.  Only for S <= ~10,
d <= ~8.
"""

import mpmath


def attention_bruteforce(q, k, v, causal, scale, dps=50):
    """q, k: [S][d] and v: [S][dv] nested sequences of floats (one head).

    Returns (o [S][dv], lse [S]) as Python floats.
    """
    S = len(q)
    d = len(q[0])
    dv = len(v[0])
    o_out, lse_out = [], []
    with mpmath.workdps(dps):
        sc = mpmath.mpf(float(scale))
        for i in range(S):
            keys = list(range(i + 1)) if causal else list(range(S))
            s = []
            for j in keys:
                dot = mpmath.mpf(0)
                for c in range(d):
                    dot += mpmath.mpf(float(q[i][c])) * mpmath.mpf(float(k[j][c]))
                s.append(sc * dot)
            w = [mpmath.exp(x) for x in s]
            z = mpmath.mpf(0)
            for x in w:
                z += x
            row = []
            for c in range(dv):
                acc = mpmath.mpf(0)
                for t, j in enumerate(keys):
                    acc += (w[t] / z) * mpmath.mpf(float(v[j][c]))
                row.append(float(acc))
            o_out.append(row)
            lse_out.append(float(mpmath.log(z)))
    return o_out, lse_out
