"""The float64 oracle run sequence by sequence on the host cores, for parity at full size.

Test infrastructure: the inputs are written once to memory-mapped .npy files,
and spawned worker processes (fresh interpreters that import numpy and the
oracle only, never the GPU) each run the oracle on whole sequences, which are
independent (one learner and one chain per sequence).  The result arrays are
assembled in sequence order, so they are those of the oracle's own batched
functions.
"""

from __future__ import annotations

import multiprocessing as mp
import os
import sys
import tempfile

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def workers() -> int:
    """Host cores to use: the process's CPU share, at most 16."""
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    return max(1, min(16, n))


def _init(root):
    if root not in sys.path:
        sys.path.insert(0, root)


def _load(d, name):
    return np.load(os.path.join(d, name + ".npy"), mmap_mode="r")


def _verify_one(job):
    import oracle
    d, b, draft_name, drafter, delta, exact_kl, T = job
    target = _load(d, "target")[b:b + 1]
    draft = _load(d, draft_name)
    draft = draft[drafter, b:b + 1] if drafter is not None else draft[b:b + 1]
    tok, r, u = _load(d, "draft_tokens")[b:b + 1], _load(d, "r")[b:b + 1], _load(d, "u")[b:b + 1]
    if delta is None:
        return oracle.spec_verify(target, draft, tok, r, u, T)
    return oracle.spec_cactus_verify(target, draft, tok, r, u, delta, T, exact_kl=exact_kl)


def _gamma_one(job):
    import oracle
    d, b, K, T = job
    target = _load(d, "target")[b:b + 1, :K]
    drafts = _load(d, "drafts")[:, b:b + 1]
    traj = _load(d, "traj")[b:b + 1]
    return oracle.spec_counterfactual_gamma(target, drafts, traj, T)


def _stack(parts):
    return {k: np.concatenate([p[k] for p in parts]) for k in parts[0]}


class OraclePool:
    """with OraclePool(x) as pool: pool.verify(...), pool.gamma(...)"""

    def __init__(self, x: dict, procs: int | None = None):
        self.dir = tempfile.mkdtemp(prefix="oracle_pool_")
        for k, v in x.items():
            if isinstance(v, np.ndarray):
                np.save(os.path.join(self.dir, k + ".npy"), v)
        self.procs = procs or workers()
        self.pool = mp.get_context("spawn").Pool(self.procs, initializer=_init, initargs=(ROOT,))

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.pool.close()
        self.pool.join()
        for f in os.listdir(self.dir):
            os.remove(os.path.join(self.dir, f))
        os.rmdir(self.dir)

    def verify(self, seqs, *, delta=None, exact_kl=False, T=1.0, draft="draft", drafters=None):
        """oracle.spec_verify (delta None) or spec_cactus_verify over the sequences `seqs`.
        drafters [B]: take sequence b's draft rows from drafts[drafters[b], b]."""
        jobs = [(self.dir, int(b), draft, None if drafters is None else int(drafters[b]), delta, exact_kl, T)
                for b in seqs]
        return _stack(self.pool.map(_verify_one, jobs, chunksize=1))

    def gamma(self, seqs, K, T=1.0):
        """oracle.spec_counterfactual_gamma over the sequences `seqs` (gamma [B, K, N], est_len, loss)."""
        return _stack(self.pool.map(_gamma_one, [(self.dir, int(b), K, T) for b in seqs], chunksize=1))
