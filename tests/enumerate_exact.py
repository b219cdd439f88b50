"""Exact (rational) enumeration of the SANTA / S²ANTA index distributions for tiny inputs.

Test-side brute force, independent of the oracle's sampler: probabilities are Fractions, the CDF is a
Fraction running sum, and the distribution of the sampled indices follows from interval overlaps
alone ("Stochastic Sparse Attention for Memory-Bound Inference", Section 2 and Section 2.1;
Appendix A.4 fixes the half-open intervals [F(j-1), F(j))).
"""

from fractions import Fraction
from itertools import product


def cdf(p):
    F, acc = [], Fraction(0)
    for x in p:
        acc += x
        F.append(acc)
    return F


def overlap(a0, a1, b0, b1):
    lo, hi = max(a0, b0), min(a1, b1)
    return hi - lo if hi > lo else Fraction(0)


def stratum_dist(p, m, S):
    """P(J = j | T ~ U[m/S, (m+1)/S)) for each key j."""
    F = cdf(p)
    lo, hi = Fraction(m, S), Fraction(m + 1, S)
    out = []
    prev = Fraction(0)
    for f in F:
        out.append(overlap(prev, f, lo, hi) * S)
        prev = f
    return out


def iid_joint(p, S):
    """All index tuples with their probabilities under i.i.d. categorical sampling."""
    nk = len(p)
    for J in product(range(nk), repeat=S):
        pr = Fraction(1)
        for j in J:
            pr *= p[j]
        if pr:
            yield J, pr


def strat_joint(p, S):
    dists = [stratum_dist(p, m, S) for m in range(S)]
    nk = len(p)
    for J in product(range(nk), repeat=S):
        pr = Fraction(1)
        for m, j in enumerate(J):
            pr *= dists[m][j]
            if not pr:
                break
        if pr:
            yield J, pr


def sys_pieces(p, S):
    """Systematic sampling: U ~ U[0, 1/S); the index tuple is constant between breakpoints F_j - m/S.

    Yields (J, probability, midpoint U) per piece.
    """
    F = cdf(p)
    width = Fraction(1, S)
    cuts = {Fraction(0), width}
    for m in range(S):
        for f in F:
            c = f - Fraction(m, S)
            if 0 < c < width:
                cuts.add(c)
    cuts = sorted(cuts)
    for a, b in zip(cuts[:-1], cuts[1:]):
        mid = (a + b) / 2
        J = []
        for m in range(S):
            t = mid + Fraction(m, S)
            j = next(i for i, f in enumerate(F) if t < f)
            J.append(j)
        yield tuple(J), (b - a) * S, mid


def moments(joint, V):
    """Exact mean vector and variance trace of the estimator (1/S) sum_m V[J_m]."""
    d = len(V[0])
    mean = [Fraction(0)] * d
    second = Fraction(0)
    total = Fraction(0)
    for item in joint:
        J, pr = item[0], item[1]
        S = len(J)
        est = [sum((V[j][i] for j in J), Fraction(0)) / S for i in range(d)]
        for i in range(d):
            mean[i] += pr * est[i]
        second += pr * sum(e * e for e in est)
        total += pr
    assert total == 1
    var = second - sum(m * m for m in mean)
    return mean, var
