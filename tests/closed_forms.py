"""Closed forms of attention on inputs with two kinds of keys (scale 1).

Every query row is e0.  Keys of the first kind have k = 0 and v = e1; keys
of the second kind have k = c e0 and v = e2.  A row that sees n0 keys of the
first kind and m of the second scores them 0 and c, so by the definition of
the softmax ([TL] section 2.1) written out for two values, with
z = n0 + m e^c, p0 = 1/z and p1 = e^c/z,

    O = n0 p0 e1 + m p1 e2,   LSE = ln z,

and every other column of O is zero.  With dO = e2 for every row, the
gradients of [TL] section 5 (dP = dO V^T, Delta = rowsum(dO o O),
dS = P o (dP - Delta), dQ = s dS K, dK = s dS^T Q, dV = P^T dO) have
dP = 0 on the first kind and 1 on the second, Delta = m p1, and

    dQ_i = c m p1 (1 - Delta) e0,
    dK_j = -sum_i p0 Delta e0 (first kind),  sum_{i sees j} p1 (1 - Delta) e0,
    dV_j =  sum_i p0 e2 (first kind),        sum_{i sees j} p1 e2,

the sums running over the rows of every query head that shares the key.
"""

import math


def forward(n0: int, m: int, c: float):
    """(weight of e1, weight of e2, LSE) of a row seeing n0 and m keys"""
    w = m * math.exp(c)
    z = n0 + w
    return n0 / z, w / z, math.log(z)


def backward(n0: int, m_rows, heads: int, c: float):
    """Gradients for dO = e2.  m_rows[i] is the number of second-kind keys
    row i sees (the first m_rows[i] of them); every row sees all n0 keys of
    the first kind; heads query heads share the keys.  Returns
    (dq0 per row, dk0 of a first-kind key, dk0 per second-kind key,
    dv2 of a first-kind key, dv2 per second-kind key)."""
    ec = math.exp(c)
    p0 = [1.0 / (n0 + m * ec) for m in m_rows]
    p1 = [ec / (n0 + m * ec) for m in m_rows]
    delta = [m * b for m, b in zip(m_rows, p1)]
    dq0 = [c * m * b * (1.0 - dl) for m, b, dl in zip(m_rows, p1, delta)]
    dk0_first = -heads * sum(a * dl for a, dl in zip(p0, delta))
    dv2_first = heads * sum(p0)
    n_second = max(m_rows) if m_rows else 0
    dk0_second, dv2_second = [], []
    for t in range(n_second):
        rows = [i for i, m in enumerate(m_rows) if m > t]
        dk0_second.append(heads * sum(p1[i] * (1.0 - delta[i]) for i in rows))
        dv2_second.append(heads * sum(p1[i] for i in rows))
    return dq0, dk0_first, dk0_second, dv2_first, dv2_second
