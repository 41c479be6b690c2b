"""Reference VRSP (variance-reduced sequence placement), in plain Python.

TEST INFRASTRUCTURE ONLY.  Used by the tests to check the library's VRSP bit
for bit, and timed as the CPU baseline of that utility; it shares no code with
the library.

Workload proxy (Libra technical review, section 3.1, eq. 1, and section 4.1,
eq. 5): a packed sequence S_i whose raw samples have lengths l_ij costs
F_i = sum_j l_ij^2.

Algorithm 1 (Libra technical review, section 4.2; Libra paper, section 4.2):
the D = GBS packed sequences of one optimizer-step window go into K = D / P
pools of exactly P sequences each.  Sequences are taken in order of
decreasing F_i, equal workloads by increasing index i; each goes to the
least-loaded pool that still holds fewer than P sequences, equal loads by
increasing pool index.  The reordered list S' concatenates the pools in pool
order (the pools are numbered GA-major), each pool's sequences in the order
they were assigned (a reading: the pages leave the order inside a pool open).

The pages keep the non-full pools in a min-heap; this reference instead scans
every pool for the least-loaded non-full one, which selects the same pool.
R = max_k load_k / mean_k load_k is the inter-pool imbalance of eq. 4;
R - 1 is the residual the pages report.
"""
from __future__ import annotations


def workload(lengths) -> int:
    """F = sum of squared raw-sample lengths of one packed sequence (eq. 1)."""
    return sum(int(l) * int(l) for l in lengths)


def vrsp(F, P: int):
    """Algorithm 1.  Returns (pool_of[i], S' as a list of indices, pool loads)."""
    D = len(F)
    if P <= 0 or D == 0 or D % P != 0:
        raise ValueError("the window must hold a whole number of pools")
    K = D // P
    order = sorted(range(D), key=lambda i: (-int(F[i]), i))
    load = [0] * K
    members = [[] for _ in range(K)]
    pool_of = [-1] * D
    for i in order:
        best = -1
        for k in range(K):
            if len(members[k]) < P and (best < 0 or (load[k], k) < (load[best], best)):
                best = k
        members[best].append(i)
        load[best] += int(F[i])
        pool_of[i] = best
    s_prime = [i for k in range(K) for i in members[k]]
    return pool_of, s_prime, load


def imbalance(loads) -> float:
    """R - 1 = max / mean - 1 over the pools' workloads."""
    mean = sum(loads) / len(loads)
    return max(loads) / mean - 1.0 if mean > 0 else 0.0
