"""Parity rule between a GPU selection row and the fp64 oracle.

Scores: |gpu - ref| <= rtol*|ref| + mtol*A, where A = sum_j |w_j| sum_e |q_je k_e|
bounds every partial sum (the mtol term only matters where ReLU cancellation
leaves ref near 0; 1e-5 ~ (d + H) * 2^-24, the fp32 accumulation bound).
Sets: with b the oracle's last selected key and t(s) a key's tolerance, a key is
"sure-in" when ref(s) - t(s) > ref(b) + t(b) and "sure-out" when
ref(s) + t(s) < ref(b) - t(b). A GPU row must hold min(sel, n) distinct eligible
indices in ascending order (then -1 padding), every sure-in key and no sure-out
key. When the k-th and (k+1)-th oracle scores are separated by more than the
tolerance this is set equality; "exact" reports whether the sets are equal.
"""
from __future__ import annotations

import numpy as np

RTOL = 1e-3
MTOL = 1e-5


class Result:
    def __init__(self):
        self.rows = 0
        self.exact = 0
        self.band = 0
        self.max_rel = 0.0
        self.failures = []

    def add(self, ok, exact, rel, msg=None):
        self.rows += 1
        self.exact += int(exact)
        self.band += int(ok and not exact)
        self.max_rel = max(self.max_rel, rel)
        if not ok:
            self.failures.append(msg)

    def summary(self):
        return (f"rows={self.rows} exact={self.exact} band={self.band} "
                f"fail={len(self.failures)} max_rel_err={self.max_rel:.3g}")


def check_row(gpu_idx, gpu_score, universe, ref, mass, sel, res, tag="",
              rtol=RTOL, mtol=MTOL):
    """Check one output row.

    universe: eligible key indices (int); ref, mass: oracle score and mass per
    universe key; gpu_idx/gpu_score: the GPU row (length sel; score may be None).
    """
    universe = np.asarray(universe, np.int64)
    ref = np.asarray(ref, np.float64)
    mass = np.asarray(mass, np.float64)
    gpu_idx = np.asarray(gpu_idx, np.int64)
    n = universe.size
    m = min(sel, n)
    head, tail = gpu_idx[:m], gpu_idx[m:]
    if np.any(tail != -1):
        return res.add(False, False, 0.0, f"{tag}: padding is not -1")
    if np.any(head < 0):
        return res.add(False, False, 0.0, f"{tag}: fewer than {m} indices")
    if np.any(np.diff(head) <= 0):
        return res.add(False, False, 0.0, f"{tag}: indices not strictly ascending")
    pos = np.searchsorted(universe, head)
    pos = np.minimum(pos, n - 1)
    if np.any(universe[pos] != head):
        return res.add(False, False, 0.0, f"{tag}: index outside the eligible keys")
    tol = rtol * np.abs(ref) + mtol * mass
    rel = 0.0
    if gpu_score is not None:
        gs = np.asarray(gpu_score, np.float64)
        if np.any(np.isfinite(gs[m:])):
            return res.add(False, False, 0.0, f"{tag}: padding score is not -inf")
        err = np.abs(gs[:m] - ref[pos])
        if np.any(err > tol[pos]):
            i = int(np.argmax(err - tol[pos]))
            return res.add(False, False, 0.0,
                           f"{tag}: score of key {head[i]} is {gs[i]!r}, oracle {ref[pos][i]!r}")
        nz = np.abs(ref[pos]) > 0
        if np.any(nz):
            rel = float(np.max(err[nz] / np.abs(ref[pos][nz])))
    order = np.lexsort((universe, -ref))
    want = np.sort(universe[order[:m]])
    if np.array_equal(want, head):
        return res.add(True, True, rel)
    if m == n:
        return res.add(False, False, rel, f"{tag}: selection must be every eligible key")
    b = order[m - 1]
    lo, hi = ref[b] - tol[b], ref[b] + tol[b]
    sure_in = universe[(ref - tol) > hi]
    sure_out = universe[(ref + tol) < lo]
    got = set(head.tolist())
    if not set(sure_in.tolist()) <= got:
        return res.add(False, False, rel, f"{tag}: a sure-in key is missing")
    if got & set(sure_out.tolist()):
        return res.add(False, False, rel, f"{tag}: a sure-out key is selected")
    return res.add(True, False, rel)
