"""Checking a greedy decode token against the oracle's logits.

Where rounding can reorder near-equal logits, several tokens are correct
greedy choices.  A token is held to the oracle's argmax only where the
oracle's top-2 gap exceeds twice the logit tolerance (the tolerance being
relative to the largest |logit|); elsewhere it must be one of the near-ties:
its own oracle logit within that margin of the top."""
import numpy as np


def greedy_ok(token: int, oracle_logits, tol: float) -> bool:
    lg = np.asarray(oracle_logits, dtype=np.float64)
    margin = 2.0 * tol * float(np.abs(lg).max())
    top2 = np.sort(lg)[-2:]
    if top2[1] - top2[0] > margin:
        return int(token) == int(np.argmax(lg))
    return bool(lg[int(token)] >= top2[1] - margin)
