"""Safe softmax of rows and the online-normaliser state, in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring): imported by tests, smoke and
the bench's cpu_baseline leg, never by the GPU library.

Two kinds of function live here:

* ``softmax_rows`` / ``logsumexp_rows`` — vectorised over rows with NumPy, the plain
  three-scan definition: scan 1 takes the row maximum m, scan 2 sums exp(x - m)
  into l, scan 3 divides exp(x - m) by l ([SNS] section 3, with the max subtraction
  of section 2.1).
* ``online_state`` / ``merge_state`` / ``online_weighted`` / ``weighted_full`` — pure
  Python float scalar instruments, one element at a time, that spell out the
  recurrences the pages state ([SNS] sections 4 and 4.1; [FAM] "why per-block
  softmaxes cannot be averaged").  They exist to be checked against the three-scan
  definition and to fix the semantics of the empty state.

Reading taken where the pages are silent: the state of an empty sequence is
(m, l) = (-inf, 0) and acts as the identity of ``merge_state``.  Written literally,
the merge rule would evaluate exp(-inf - (-inf)) = NaN when both sides are empty; a
side whose m is -inf contributes nothing instead.
"""

import math

import numpy as np

NEG_INF = -math.inf


# ----------------------------------------------------------------------------
# Vectorised three-scan definition.
# ----------------------------------------------------------------------------

def softmax_rows(x):
    """Three-scan safe softmax along the last axis, in float64.

    [SNS] section 3: scan 1 computes m = max_i x_i, scan 2 computes
    l = sum_i exp(x_i - m), scan 3 writes exp(x_i - m) / l.  Subtracting m is the
    exact identity of section 2.1 (numerator and denominator both times e^-m).

    ``x`` may be any real float dtype; it is upcast to float64 exactly.
    Returns ``(y, m, l)`` with ``y`` shaped like ``x`` and ``m``, ``l`` holding one
    value per row.
    """
    x = np.asarray(x, dtype=np.float64)
    if x.shape[-1] == 0:
        raise ValueError("softmax of an empty row is undefined")
    m = np.max(x, axis=-1, keepdims=True)              # scan 1
    l = np.sum(np.exp(x - m), axis=-1, keepdims=True)  # scan 2
    y = np.exp(x - m) / l                              # scan 3
    return y, m[..., 0], l[..., 0]


def logsumexp_rows(x):
    """ln sum_i exp(x_i) of each row, as m + ln l from the scans above."""
    _, m, l = softmax_rows(x)
    return m + np.log(l)


# ----------------------------------------------------------------------------
# Scalar online-normaliser instruments (pure Python floats = IEEE binary64).
# ----------------------------------------------------------------------------

def _decay(m_old, m_new):
    """Factor that moves a sum taken relative to m_old onto the base m_new.

    The empty state (m_old = -inf) has nothing to move: its factor is 0.
    """
    if m_old == NEG_INF:
        return 0.0
    return math.exp(m_old - m_new)


def online_state(xs):
    """(m, l) of a sequence, one element at a time ([SNS] section 4).

    For each new element x the running maximum becomes max(m, x); the old sum is
    multiplied by exp(m_old - m_new) so it is taken relative to the new maximum,
    and exp(x - m_new) is added.  The empty sequence gives (-inf, 0).
    """
    m, l = NEG_INF, 0.0
    for x in xs:
        x = float(x)
        m_next = max(m, x)
        l = l * _decay(m, m_next) + math.exp(x - m_next)
        m = m_next
    return m, l


def merge_state(a, b):
    """Combine the (m, l) states of two disjoint pieces of one row ([SNS] 4.1).

    m = max(m_a, m_b) and l = l_a exp(m_a - m) + l_b exp(m_b - m).  In exact
    arithmetic this operator is associative and commutative, which is what lets a
    row be reduced as a tree ([SNS] section 4.2; [INT] follow-up 1 states the same
    rescaling of the two partial sums).  (-inf, 0) is its identity.
    """
    m_a, l_a = float(a[0]), float(a[1])
    m_b, l_b = float(b[0]), float(b[1])
    m = max(m_a, m_b)
    if m == NEG_INF:
        return NEG_INF, 0.0
    return m, l_a * _decay(m_a, m) + l_b * _decay(m_b, m)


def online_weighted(scores, values):
    """One-pass softmax-weighted sum of scalars by the (m, l, u) recurrence.

    [FAM] "why per-block softmaxes cannot be averaged": keep the running maximum m,
    the unnormalised total l and the weighted total u.  A new score a with value v
    sets m' = max(m, a); both l and u are multiplied by exp(m - m') and the new term
    enters with weight exp(a - m').  The result is u / l.  For vector values the
    same factor multiplies every component; the attention oracle covers that case.

    Returns ``(u / l, m, l)``.
    """
    m, l, u = NEG_INF, 0.0, 0.0
    for a, v in zip(scores, values):
        a = float(a)
        m_next = max(m, a)
        c = _decay(m, m_next)
        w = math.exp(a - m_next)
        l = c * l + w
        u = c * u + w * float(v)
        m = m_next
    if l == 0.0:
        raise ValueError("weighted softmax of an empty row is undefined")
    return u / l, m, l


def weighted_full(scores, values):
    """Softmax-weighted sum with all weights formed first (the comparison path).

    Take m = max of the scores, every weight exp(s - m), then
    sum(w v) / sum(w).  Sums use ``math.fsum`` so the order of addition does not
    matter to the last bit.
    """
    s = [float(a) for a in scores]
    if not s:
        raise ValueError("weighted softmax of an empty row is undefined")
    m = max(s)
    w = [math.exp(a - m) for a in s]
    return math.fsum(wi * float(v) for wi, v in zip(w, values)) / math.fsum(w)
