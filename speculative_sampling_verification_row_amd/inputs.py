"""Seeded synthetic inputs shaped like the workloads the pages evaluate.

This module holds no verification arithmetic: it only draws numbers.  Both
the CPU oracle (through the tests) and the HIP path consume what it returns.

Every draw comes from a numpy Philox stream keyed by
``SeedSequence(seed, spawn_key=(config_id, stream, round, row))`` so that each
row is reproducible on its own and rows can be drawn in parallel threads.

Recipes (see also the design notes):
* logits: float32 N(0, sigma^2) draws rounded to bf16 (round-to-nearest-even);
* peaked rows: each target row independently, with probability ``peak_frac``,
  gets ``peak_boost`` added to one uniformly chosen logit before rounding;
* draft (drafter i) = bf16(float32(target_bf16) + sigma_i * N(0, 1));
* drafted tokens are drawn from the drafting drafter's softmax at temperature
  T, and trajectory tokens from the target's, both by the Gumbel-max trick
  (argmax of z / T + Gumbel noise, in float64): exact sampling that never
  forms a probability;
* uniforms are float32 in [0, 1) (multiples of 2**-24).

The pages measure on GSM8K, IFEval, GPQA, HumanEval, MedQA, CNN-DM and SQL with
Llama-3.1 / Qwen3 models; none of that is available, and these synthetic
logits with the models' vocabulary sizes stand in for it.
"""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Optional, Sequence

import numpy as np

# Stream ids of the spawn key.
S_TARGET, S_NOISE, S_PEAK, S_SIGMA, S_DTOK, S_R, S_U, S_TRAJ, S_SEL, S_V, S_DELAY, S_LOSS = range(12)

_THREADS = max(1, min(16, len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else 4))


def _rng(seed: int, config_id: int, stream: int, rnd: int, row: int) -> np.random.Generator:
    return np.random.Generator(np.random.Philox(np.random.SeedSequence(seed, spawn_key=(config_id, stream, rnd, row))))


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
    return (rounded >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _parallel(fn, n: int):
    if n <= 1 or _THREADS == 1:
        for i in range(n):
            fn(i)
        return
    with ThreadPoolExecutor(max_workers=_THREADS) as ex:
        list(ex.map(fn, range(n)))


def gumbel_max_token(bits_row: np.ndarray, temperature: float, gen: np.random.Generator) -> int:
    """One draw from softmax(z / T) of a bf16 row by the Gumbel-max trick."""
    z = bf16_to_f32(bits_row).astype(np.float64) / temperature
    g = -np.log(-np.log(gen.random(z.shape[0])))
    return int(np.argmax(z + g))


def target_logits(B: int, rows: int, V: int, sigma: float, *, peak_frac: float = 0.0,
                  peak_boost: float = 12.0, seed: int = 0, config_id: int = 0, rnd: int = 0) -> np.ndarray:
    """[B, rows, V] bf16 bits, N(0, sigma^2) with optional peaked rows."""
    out = np.empty((B * rows, V), dtype=np.uint16)

    def one(r: int) -> None:
        g = _rng(seed, config_id, S_TARGET, rnd, r)
        x = g.standard_normal(V, dtype=np.float32)
        x *= np.float32(sigma)
        if peak_frac > 0.0:
            gp = _rng(seed, config_id, S_PEAK, rnd, r)
            if gp.random() < peak_frac:
                x[int(gp.integers(V))] += np.float32(peak_boost)
        out[r] = bf16_bits(x)

    _parallel(one, B * rows)
    return out.reshape(B, rows, V)


def draft_logits(target_bits: np.ndarray, sigma: float, *, seed: int = 0, config_id: int = 0,
                 rnd: int = 0, drafter: int = 0, rows: Optional[int] = None) -> np.ndarray:
    """bf16(float32(target) + sigma * N(0, 1)) for the first ``rows`` rows of every sequence."""
    B, R, V = target_bits.shape
    rows = R if rows is None else rows
    out = np.empty((B, rows, V), dtype=np.uint16)

    def one(idx: int) -> None:
        b, k = divmod(idx, rows)
        g = _rng(seed, config_id, S_NOISE, rnd, (drafter * B + b) * rows + k)
        n = g.standard_normal(V, dtype=np.float32)
        n *= np.float32(sigma)
        n += bf16_to_f32(target_bits[b, k])
        out[b, k] = bf16_bits(n)

    _parallel(one, B * rows)
    return out


def uniforms(shape, *, seed: int = 0, config_id: int = 0, stream: int = S_R, rnd: int = 0) -> np.ndarray:
    """float32 uniforms in [0, 1)."""
    return _rng(seed, config_id, stream, rnd, 0).random(shape, dtype=np.float32)


def sample_tokens(bits: np.ndarray, temperature: float, *, seed: int = 0, config_id: int = 0,
                  stream: int = S_DTOK, rnd: int = 0) -> np.ndarray:
    """[B, K] int32 tokens, one Gumbel-max draw per row of bits [B, K, V]."""
    B, K, _ = bits.shape
    out = np.empty((B, K), dtype=np.int32)

    def one(idx: int) -> None:
        b, k = divmod(idx, K)
        out[b, k] = gumbel_max_token(bits[b, k], temperature, _rng(seed, config_id, stream, rnd, idx))

    _parallel(one, B * K)
    return out


# ---------------------------------------------------------------------------
# Workload configurations
# ---------------------------------------------------------------------------

@dataclass(frozen=True)
class SpsWorkload:
    """Lossless (or Cactus) verification: B sequences, K drafts, vocab V."""
    name: str
    B: int
    K: int
    V: int
    target_sigma: float
    draft_sigma: float
    peak_frac: float = 0.0
    peak_boost: float = 12.0
    temperature: float = 1.0
    config_id: int = 2
    deltas: Sequence[float] = field(default_factory=tuple)


@dataclass(frozen=True)
class GammaWorkload:
    """HedgeSpec evaluation of N drafters (optionally fused with verification)."""
    name: str
    B: int
    K: int
    N: int
    V: int
    target_sigma: float
    sigmas: Optional[Sequence[float]] = None   # explicit per-drafter noise
    sigma_range: Optional[tuple] = None        # (lo, hi): drawn uniformly per drafter
    peak_frac: float = 0.0
    temperature: float = 1.0
    fused: bool = False                        # verify sel[b]'s drafts in the same launch
    draft_from: str = "sel"                    # "sel" or "drafter0"
    rounds: int = 1
    config_id: int = 3


# The five workloads of the evaluation plan.
SMALL_MIXED = GammaWorkload("sps+gamma small: B=4 K=5 N=7 V=32000", B=4, K=5, N=7, V=32000,
                            target_sigma=2.0, sigma_range=(0.3, 2.0), fused=True,
                            draft_from="drafter0", config_id=1)
LLAMA_SPS = SpsWorkload("lossless SpS verify: B=64 K=5 V=128256", B=64, K=5, V=128256,
                        target_sigma=2.5, draft_sigma=0.8, peak_frac=0.01, config_id=2)
HEDGE_EVAL = GammaWorkload("HedgeSpec evaluation: B=32 K=5 N=7 V=128256", B=32, K=5, N=7, V=128256,
                           target_sigma=2.0, sigmas=(0.3, 0.5, 0.8, 1.2, 1.6, 2.0, 2.5),
                           rounds=256, config_id=3)
QWEN_CACTUS = SpsWorkload("Cactus verify: B=64 m=20 V=151936", B=64, K=20, V=151936,
                          target_sigma=3.0, draft_sigma=1.0, deltas=(0.0, 0.5, 1.0), config_id=4)
POOL21 = GammaWorkload("21-drafter pool, fused: B=64 K=8 N=21 V=151936", B=64, K=8, N=21, V=151936,
                       target_sigma=3.0, sigmas=tuple(0.2 + 0.14 * i for i in range(21)),
                       fused=True, config_id=5)

WORKLOADS = {1: SMALL_MIXED, 2: LLAMA_SPS, 3: HEDGE_EVAL, 4: QWEN_CACTUS, 5: POOL21}


def make_sps_inputs(w: SpsWorkload, *, seed: int = 0, rnd: int = 0, B: Optional[int] = None,
                    V: Optional[int] = None) -> dict:
    """Inputs of one verification call.  ``B`` / ``V`` override the sizes (smaller tests)."""
    B = w.B if B is None else B
    V = w.V if V is None else V
    K = w.K
    cid = w.config_id
    target = target_logits(B, K + 1, V, w.target_sigma, peak_frac=w.peak_frac, peak_boost=w.peak_boost,
                           seed=seed, config_id=cid, rnd=rnd)
    draft = draft_logits(target, w.draft_sigma, seed=seed, config_id=cid, rnd=rnd, rows=K)
    return {
        "target": target,
        "draft": draft,
        "draft_tokens": sample_tokens(draft, w.temperature, seed=seed, config_id=cid, rnd=rnd),
        "r": uniforms((B, K), seed=seed, config_id=cid, stream=S_R, rnd=rnd),
        "u": uniforms((B, K + 1), seed=seed, config_id=cid, stream=S_U, rnd=rnd),
        "temperature": w.temperature,
    }


def drafter_sigmas(w: GammaWorkload, *, seed: int = 0) -> np.ndarray:
    if w.sigmas is not None:
        return np.asarray(w.sigmas, dtype=np.float64)
    lo, hi = w.sigma_range
    return lo + (hi - lo) * _rng(seed, w.config_id, S_SIGMA, 0, 0).random(w.N)


def make_gamma_inputs(w: GammaWorkload, *, seed: int = 0, rnd: int = 0, B: Optional[int] = None,
                      V: Optional[int] = None, N: Optional[int] = None) -> dict:
    """Inputs of one evaluation call: target [B, K+1, V], drafts [N, B, K, V], trajectory,
    and (for the fused form) the selected drafter, its drafted tokens and uniforms."""
    B = w.B if B is None else B
    V = w.V if V is None else V
    N = w.N if N is None else N
    K = w.K
    cid = w.config_id
    sig = drafter_sigmas(w, seed=seed)[:N]
    target = target_logits(B, K + 1, V, w.target_sigma, peak_frac=w.peak_frac, seed=seed,
                           config_id=cid, rnd=rnd)
    drafts = np.stack([draft_logits(target, float(sig[i]), seed=seed, config_id=cid, rnd=rnd,
                                    drafter=i, rows=K) for i in range(N)])
    if w.draft_from == "drafter0":
        sel = np.zeros(B, dtype=np.int32)
    else:
        sel = _rng(seed, cid, S_SEL, rnd, 0).integers(0, N, size=B).astype(np.int32)
    sel_rows = np.stack([drafts[sel[b], b] for b in range(B)])
    return {
        "target": target,
        "drafts": drafts,
        "sigmas": sig,
        "traj": sample_tokens(target[:, :K], w.temperature, seed=seed, config_id=cid, stream=S_TRAJ, rnd=rnd),
        "sel": sel,
        "draft_tokens": sample_tokens(sel_rows, w.temperature, seed=seed, config_id=cid, stream=S_DTOK, rnd=rnd),
        "r": uniforms((B, K), seed=seed, config_id=cid, stream=S_R, rnd=rnd),
        "u": uniforms((B, K + 1), seed=seed, config_id=cid, stream=S_U, rnd=rnd),
        "temperature": w.temperature,
    }


def hedge_schedule(T: int, B: int, K: int, *, seed: int = 0, config_id: int = 3) -> dict:
    """Selection uniforms v [T, B] and delays [T, B] in {0, ..., 2K} for T rounds."""
    return {
        "v": _rng(seed, config_id, S_V, 0, 0).random((T, B), dtype=np.float32),
        "delays": _rng(seed, config_id, S_DELAY, 0, 0).integers(0, 2 * K + 1, size=(T, B)).astype(np.int32),
    }


def synthetic_losses(T: int, B: int, N: int, K: int, *, seed: int = 0, config_id: int = 3) -> np.ndarray:
    """[T, B, N] float32 losses in [0, K]: drafter i has mean quality ranked by i with noise.
    Stand-in loss streams for learner tests that do not need full-vocabulary rows."""
    g = _rng(seed, config_id, S_LOSS, 0, 0)
    base = np.linspace(0.2, 0.8, N, dtype=np.float64)
    x = base[None, None, :] + 0.25 * g.standard_normal((T, B, N))
    return (np.clip(x, 0.0, 1.0) * K).astype(np.float32)
