"""Greedy-id comparison shared by the GPU tests of the Q6_K head.

The GPU's id for a projected row must equal the oracle's.  The one accepted
difference is a near tie: the oracle's logit of its own id o exceeds its
logit of the GPU's id g by no more than the float bound of one logit,
1e-5 * sum_b |t_b| + 1e-6 (the larger of the two rows' block-term sums), and
g and o are different weight rows.  Every accepted near tie is printed, so a
run shows how many it took.
"""
import sys

REL, ABS = 1e-5, 1e-6


def check_ids(gpu_ids, ref_ids, logits, bound, what="ids", equal_rows=None):
    """Assert the rule above for every row; return the accepted near ties as
    (row, gpu id, oracle id, gap, bound) tuples."""
    accepted = []
    for r, (g, o) in enumerate(zip(gpu_ids, ref_ids)):
        g, o = int(g), int(o)
        if g == o:
            continue
        assert 0 <= g < logits.shape[1], f"{what} row {r}: id {g} out of range"
        gap = float(logits[r, o] - logits[r, g])
        tol = REL * max(float(bound[r, o]), float(bound[r, g])) + ABS
        assert gap <= tol, f"{what} row {r}: gpu {g} oracle {o} gap {gap} > {tol}"
        if equal_rows is not None:
            assert not equal_rows(g, o), f"{what} row {r}: equal weight rows must give the lower id"
        accepted.append((r, g, o, gap, tol))
    print(f"{what}: {len(accepted)} near-tie id differences accepted {accepted}",
          file=sys.stderr, flush=True)
    return accepted
