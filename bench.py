"""Benchmark of the verification hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload llama_sps]

One step is one launch of the hot path over one batch of synthetic input
already resident in HBM.  The default workload is lossless verification of
B=64 sequences x K=5 drafts over the Llama-3.1 vocabulary (V=128256, 1% of
target rows peaked); the other workloads (--workload) are available for
measurement and profiling.

Timing: untimed warm-up steps (at least W, and whole steps until 100 ms have
passed, so that the GPU's clocks have settled; the JSON reports how many), then
K timed steps back to back, bracketed by device synchronisation and by one pair
of HIP events on the launch stream, whose span / K is the mean launch duration
used for the roofline.  200 more launches, in batches of 10, give its spread
(median, p10, p90).  To keep the 256 MB Infinity Cache from serving the inputs,
steps rotate over enough identical copies of the inputs (>= 1 GiB in total)
that each launch reads lines no earlier launch left in the cache.

Output: one JSON line on stdout (progress goes to stderr) with the metric,
the roofline of the dominant kernel (algorithmic bytes per launch / mean
launch time vs the 8 TB/s HBM peak; `traffic` from the committed rocprofv3
FETCH_SIZE/WRITE_SIZE summary when it was taken on the current kernel
sources), and the float64 CPU oracle timed on the host cores on a bounded
sample of the same workload.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
GAMMA_WORKLOADS = ("hedge_eval", "pool21", "small_mixed", "hedge_loop")


def kernel_of(key: str) -> str:
    """The library's kernel that a workload's step launches."""
    if key == "stream_read":
        return "stream_read_kernel"
    if key.endswith("_tree"):
        return "tree_kernel"
    return "gamma_kernel" if key in GAMMA_WORKLOADS else "verify_kernel"


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def source_hash() -> str:
    """Hash of the verification library's sources' code: comments and whitespace are
    left out, so that only a change of the code itself makes recorded counters stale.
    The streaming-read probe is a library of its own and is left out too."""
    csrc = os.path.join(ROOT, "speculative_sampling_verification_row_amd", "csrc")
    h = hashlib.sha256()
    for name in sorted(os.listdir(csrc)):
        if name.startswith("stream_probe"):
            continue
        if name.endswith((".hip", ".hpp", ".h", ".cpp")):
            with open(os.path.join(csrc, name), "r") as f:
                text = f.read()
            text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
            text = re.sub(r"//[^\n]*", " ", text)
            text = " ".join(text.split())
            h.update(name.encode() + b"\0" + text.encode())
    return h.hexdigest()[:16]


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def host_cores() -> int:
    """The process's CPU share, at most 16 (the GPU machine's share for one GPU)."""
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    return max(1, min(16, n))


def _oracle_sequence(job):
    """One sequence of a workload through the oracle (all-core leg; a spawned worker)."""
    kind, d, b, extra = job
    if ROOT not in sys.path:
        sys.path.insert(0, ROOT)
    import oracle
    ld = lambda k: np.load(os.path.join(d, k + ".npy"), mmap_mode="r")
    sl = slice(b, b + 1)
    if kind == "sps":
        oracle.spec_verify(ld("target")[sl], ld("draft")[sl], ld("draft_tokens")[sl], ld("r")[sl], ld("u")[sl])
    elif kind == "cactus":
        oracle.spec_cactus_verify(ld("target")[sl], ld("draft")[sl], ld("draft_tokens")[sl], ld("r")[sl],
                                  ld("u")[sl], extra["delta"], exact_kl=extra["exact_kl"])
    elif kind == "gamma":
        K = extra["K"]
        oracle.spec_counterfactual_gamma(ld("target")[sl, :K], ld("drafts")[:, sl], ld("traj")[sl])
        if extra["fused"]:
            s_ = int(ld("sel")[b])
            oracle.spec_verify(ld("target")[sl], ld("drafts")[s_, sl], ld("draft_tokens")[sl], ld("r")[sl],
                               ld("u")[sl])
    elif kind == "tree":
        K = extra["K"]
        oracle.spec_tree_gamma(ld("target")[sl, :K], ld("drafts")[:, sl], extra["topk"])
    return b


def cpu_all_cores(kind: str, x: dict, extra: dict, B: int, n_seq: int, cores: int):
    """The oracle over n_seq sequences of the batch (cycling), row-parallel on `cores` spawned
    processes reading memory-mapped inputs.  Returns the wall seconds."""
    import multiprocessing as mp
    import shutil
    import tempfile
    d = tempfile.mkdtemp(prefix="bench_oracle_")
    try:
        for k, v in x.items():
            if isinstance(v, np.ndarray):
                np.save(os.path.join(d, k + ".npy"), v)
        with mp.get_context("spawn").Pool(cores) as pool:
            pool.map(_oracle_sequence, [(kind, d, b % B, extra) for b in range(cores)])  # warm the workers
            t0 = time.perf_counter()
            pool.map(_oracle_sequence, [(kind, d, b % B, extra) for b in range(n_seq)], chunksize=1)
            return time.perf_counter() - t0
    finally:
        shutil.rmtree(d, ignore_errors=True)


# ---------------------------------------------------------------------------
# Workloads
# ---------------------------------------------------------------------------

class Workload:
    key = ""
    desc = ""
    positions = 0          # verified draft positions per launch
    algo_bytes = 0         # bytes the method must move per launch (every logit it needs once + small arrays)
    bonus_rows = None      # bonus target rows among them: sequences that accepted every draft

    def count_bonus(self, accepted_len, K: int, B: int, V: int) -> None:
        """The bonus row K of a sequence is needed (and read) only when it accepted all K
        drafts: count those in the launch's own outputs and add their rows."""
        self.bonus_rows = int((accepted_len == K).sum().item())
        self.algo_bytes = self.base_bytes + 2 * V * self.bonus_rows
        log(f"bonus rows read: {self.bonus_rows} of {B} sequences accepted every draft")

    def setup(self, copies_min_bytes: int):
        raise NotImplementedError

    def launch(self, i: int):
        raise NotImplementedError

    def cpu_sample(self, budget_s: float):
        """Run the oracle on a bounded sample; returns (positions, seconds, cpu_seconds, sample text)."""
        raise NotImplementedError


def _dev(torch, bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


class SpsLike(Workload):
    """spec_verify (delta None) or spec_cactus_verify (spec_cactus_kl_verify with
    exact_kl) over one SpsWorkload."""

    def __init__(self, key, w, delta=None, exact_kl=False):
        self.key, self.w, self.delta, self.exact_kl = key, w, delta, exact_kl
        B, K, V = w.B, w.K, w.V
        self.desc = w.name + ("" if delta is None else f" delta={delta}") + (" exact-KL gamma*" if exact_kl else "")
        self.positions = B * K
        # target and draft rows of positions 0..K-1; bonus rows are added once counted
        rows = 2 * B * K
        small = B * K * 4 * 2 + B * (K + 1) * 4 + B * 4 * 2 + B * K + (B * K * 4 if delta is not None else 0)
        self.base_bytes = self.algo_bytes = 2 * V * rows + small

    def setup(self, copies_min_bytes):
        import torch
        from speculative_sampling_verification_row_amd import binding
        from speculative_sampling_verification_row_amd import inputs as gen
        self.torch, self.binding = torch, binding
        log(f"generating inputs: {self.desc}")
        self.x = gen.make_sps_inputs(self.w)
        t = _dev(torch, self.x["target"])
        d = _dev(torch, self.x["draft"])
        n = max(1, -(-copies_min_bytes // (2 * (t.numel() + d.numel()))))
        self.copies = [(t, d)] + [(t.clone(), d.clone()) for _ in range(n - 1)]
        self.tok = torch.from_numpy(self.x["draft_tokens"]).cuda()
        self.r = torch.from_numpy(self.x["r"]).cuda()
        self.u = torch.from_numpy(self.x["u"]).cuda()
        self.ws = binding.make_workspace(self.w.B, self.w.K, 1)
        # one prepared call per copy: a launch only enqueues the kernel
        if self.delta is None:
            self.calls = [binding.prepare_verify(t, d, self.tok, self.r, self.u, self.w.temperature, workspace=self.ws)
                          for t, d in self.copies]
        else:
            self.calls = [binding.prepare_cactus_verify(t, d, self.tok, self.r, self.u, self.delta,
                                                        self.w.temperature, workspace=self.ws,
                                                        exact_kl=self.exact_kl)
                          for t, d in self.copies]
        log(f"{len(self.copies)} input copies of {2 * (t.numel() + d.numel()) / 1e6:.1f} MB")
        self.count_bonus(self.calls[0].run()[0], self.w.K, self.w.B, self.w.V)

    def launch(self, i):
        self.calls[i % len(self.calls)].launch()

    def cpu_kind(self):
        if self.delta is None:
            return "sps", {}
        return "cactus", {"delta": self.delta, "exact_kl": self.exact_kl}

    def cpu_sample(self, budget_s):
        import oracle
        x, B = self.x, self.w.B
        done, pos, t0, c0 = 0, 0, time.perf_counter(), time.process_time()
        while True:
            b = done % B
            sl = slice(b, b + 1)
            if self.delta is None:
                oracle.spec_verify(x["target"][sl], x["draft"][sl], x["draft_tokens"][sl], x["r"][sl], x["u"][sl])
            else:
                oracle.spec_cactus_verify(x["target"][sl], x["draft"][sl], x["draft_tokens"][sl], x["r"][sl],
                                          x["u"][sl], self.delta, exact_kl=self.exact_kl)
            done += 1
            pos += self.w.K
            if time.perf_counter() - t0 >= budget_s:
                break
        return pos, time.perf_counter() - t0, time.process_time() - c0, f"{done} sequences of this batch, one at a time"


class GammaLike(Workload):
    def __init__(self, key, w):
        self.key, self.w = key, w
        B, K, N, V = w.B, w.K, w.N, w.V
        self.desc = w.name
        self.positions = B * K
        # target rows 0..K-1 and every drafter's rows; a fused call's bonus rows are added once counted
        rows = B * K + N * B * K
        small = B * K * 4 + B * K * N * 4 + 2 * B * N * 4
        if w.fused:
            small += B * 4 + B * K * 4 * 2 + B * (K + 1) * 4 + B * 4 * 2 + B * K
        self.base_bytes = self.algo_bytes = 2 * V * rows + small

    def setup(self, copies_min_bytes):
        import torch
        from speculative_sampling_verification_row_amd import binding
        from speculative_sampling_verification_row_amd import inputs as gen
        self.torch, self.binding = torch, binding
        log(f"generating inputs: {self.desc}")
        self.x = gen.make_gamma_inputs(self.w)
        t = _dev(torch, self.x["target"])
        d = _dev(torch, self.x["drafts"])
        per = 2 * (t.numel() + d.numel())
        n = max(1, -(-copies_min_bytes // per))
        self.copies = [(t, d)] + [(t.clone(), d.clone()) for _ in range(n - 1)]
        i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()
        f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()
        self.traj = i32(self.x["traj"])
        self.kw = {}
        if self.w.fused:
            self.kw = dict(sel=i32(self.x["sel"]), draft_tokens=i32(self.x["draft_tokens"]), r_accept=f32(self.x["r"]),
                           u_resample=f32(self.x["u"]))
        self.ws = binding.make_workspace(self.w.B, self.w.K, self.w.N)
        self.calls = [binding.prepare_counterfactual_gamma(t, d, self.traj, self.w.temperature, workspace=self.ws,
                                                           **self.kw) for t, d in self.copies]
        log(f"{len(self.copies)} input copies of {per / 1e6:.1f} MB")
        if self.w.fused:
            self.count_bonus(self.calls[0].run()["accepted_len"], self.w.K, self.w.B, self.w.V)

    def launch(self, i):
        self.calls[i % len(self.calls)].launch()

    def cpu_kind(self):
        return "gamma", {"K": self.w.K, "fused": bool(self.w.fused)}

    def cpu_sample(self, budget_s):
        import oracle
        x, B, K = self.x, self.w.B, self.w.K
        done, t0, c0 = 0, time.perf_counter(), time.process_time()
        while True:
            b = done % B
            oracle.spec_counterfactual_gamma(x["target"][b:b + 1, :K], x["drafts"][:, b:b + 1], x["traj"][b:b + 1])
            if self.w.fused:
                s = int(x["sel"][b])
                oracle.spec_verify(x["target"][b:b + 1], x["drafts"][s, b:b + 1], x["draft_tokens"][b:b + 1],
                                   x["r"][b:b + 1], x["u"][b:b + 1])
            done += 1
            if time.perf_counter() - t0 >= budget_s:
                break
        return done * K, time.perf_counter() - t0, time.process_time() - c0, f"{done} sequences of this batch, one at a time"


class TreeLike(GammaLike):
    """spec_tree_gamma over one GammaWorkload's target and drafter rows (topk children)."""

    def __init__(self, key, w, topk):
        super().__init__(key, w)
        B, K, N, V = w.B, w.K, w.N, w.V
        self.topk = topk
        self.desc = f"{w.name}, draft-tree gamma with {topk} children per node"
        self.algo_bytes = 2 * V * (B * K + N * B * K) + B * K * N * 4

    def setup(self, copies_min_bytes):
        import torch
        from speculative_sampling_verification_row_amd import binding
        from speculative_sampling_verification_row_amd import inputs as gen
        self.torch, self.binding = torch, binding
        log(f"generating inputs: {self.desc}")
        self.x = gen.make_gamma_inputs(self.w)
        K = self.w.K
        t = _dev(torch, self.x["target"][:, :K])
        d = _dev(torch, self.x["drafts"])
        per = 2 * (t.numel() + d.numel())
        n = max(1, -(-copies_min_bytes // per))
        self.copies = [(t, d)] + [(t.clone(), d.clone()) for _ in range(n - 1)]
        self.ws = binding.make_tree_workspace(self.w.B, K, self.w.N, self.w.V, self.topk)
        self.calls = [binding.prepare_tree_gamma(t, d, self.topk, self.w.temperature, workspace=self.ws)
                      for t, d in self.copies]
        log(f"{len(self.copies)} input copies of {per / 1e6:.1f} MB")

    def cpu_kind(self):
        return "tree", {"K": self.w.K, "topk": self.topk}

    def cpu_sample(self, budget_s):
        import oracle
        x, B, K = self.x, self.w.B, self.w.K
        done, t0, c0 = 0, time.perf_counter(), time.process_time()
        while True:
            b = done % B
            oracle.spec_tree_gamma(x["target"][b:b + 1, :K], x["drafts"][:, b:b + 1], self.topk)
            done += 1
            if time.perf_counter() - t0 >= budget_s:
                break
        return done * K, time.perf_counter() - t0, time.process_time() - c0, f"{done} sequences of this batch, one at a time"


class LoopLike(GammaLike):
    """One HedgeSpec round resident on the device, replayed from a captured graph: the
    learner (NormalHedge, delay from censoring counted on the device) selects each
    sequence's drafter, then the fused spec_counterfactual_gamma evaluates all N drafters
    and verifies the selected one.  One step = one round.  Consecutive rounds read
    different copies of the rows (a graph per copy, >= 1 GiB in all), as fresh rows would
    arrive, so the Infinity Cache does not serve a round from the last one's reads."""

    ROUNDS = 4096

    def __init__(self, key, w):
        import dataclasses
        super().__init__(key, dataclasses.replace(w, fused=True, draft_from="drafter0"))
        self.desc = (f"{self.w.name}, fused HedgeSpec round (censoring queue + NormalHedge + gamma + verify) "
                     "from a graph")

    def setup(self, copies_min_bytes):
        import torch
        from speculative_sampling_verification_row_amd import inputs as gen
        from speculative_sampling_verification_row_amd.loop import HedgeSpecLoop
        self.torch = torch
        log(f"generating inputs: {self.desc}")
        self.x = x = gen.make_gamma_inputs(self.w)
        i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()
        f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()
        t, d = _dev(torch, x["target"]), _dev(torch, x["drafts"])
        per = 2 * (t.numel() + d.numel())
        n = max(1, -(-copies_min_bytes // per))
        small = {"traj": i32(x["traj"]), "draft_tokens": i32(x["draft_tokens"]), "r_accept": f32(x["r"]),
                 "u_resample": f32(x["u"])}
        rows = [dict(small, target=t, drafts=d)] + [dict(small, target=t.clone(), drafts=d.clone())
                                                    for _ in range(n - 1)]
        sch = gen.hedge_schedule(self.ROUNDS, self.w.B, self.w.K)
        self.loop = HedgeSpecLoop(rows, f32(sch["v"]), 1.0 / self.w.K, self.w.temperature)
        self.loop.step()          # eager round: library set-up outside the capture
        torch.cuda.synchronize()
        self.loop.reset()
        self.loop.capture()
        # bonus rows: the mean over the first rounds (each round selects its own drafters)
        self.loop.reset()
        full, nr = 0, 64
        for _ in range(nr):
            self.loop.replay()
            full += int((self.loop.out["accepted_len"] == self.w.K).sum().item())
        self.bonus_rows = full / nr
        self.algo_bytes = int(round(self.base_bytes + 2 * self.w.V * self.bonus_rows))
        log(f"bonus rows read: {self.bonus_rows:.2f} of {self.w.B} sequences per round (mean of {nr} rounds)")
        self.loop.reset()
        log(f"captured a round per row copy ({n} copies of {per / 1e6:.1f} MB) as graphs")

    def launch(self, i):
        self.loop.replay()


class StreamRead(Workload):
    """The streaming-read probe over the same bytes as llama_sps's logits: a plain read with
    the statistics phase's access pattern, the read ceiling of the verification kernels."""

    def __init__(self, key, nbytes):
        self.key, self.positions, self.algo_bytes = key, 0, nbytes
        self.desc = f"streaming read of {nbytes / 1e6:.1f} MB (the statistics phase's access pattern)"

    def setup(self, copies_min_bytes):
        import torch
        from speculative_sampling_verification_row_amd import binding
        self.probe = binding.StreamProbe()
        n = max(1, -(-copies_min_bytes // self.algo_bytes))
        self.bufs = [torch.ones(self.algo_bytes // 2, dtype=torch.int16, device="cuda") for _ in range(n)]
        self.grid = 2 * torch.cuda.get_device_properties(0).multi_processor_count
        self.out = torch.empty(self.grid * 256, dtype=torch.int32, device="cuda")
        log(f"{n} buffers of {self.algo_bytes / 1e6:.1f} MB, grid {self.grid}")

    def launch(self, i):
        self.probe.read(self.bufs[i % len(self.bufs)], self.out, self.grid)


def workloads():
    from speculative_sampling_verification_row_amd import inputs as gen
    return {
        "stream_read": lambda: StreamRead("stream_read", 180589376),
        "llama_sps": lambda: SpsLike("llama_sps", gen.LLAMA_SPS),
        "qwen_cactus": lambda: SpsLike("qwen_cactus", gen.QWEN_CACTUS, delta=1.0),
        "qwen_cactus_d0": lambda: SpsLike("qwen_cactus_d0", gen.QWEN_CACTUS, delta=0.0),
        "qwen_cactus_d05": lambda: SpsLike("qwen_cactus_d05", gen.QWEN_CACTUS, delta=0.5),
        "qwen_cactus_kl": lambda: SpsLike("qwen_cactus_kl", gen.QWEN_CACTUS, delta=1.0, exact_kl=True),
        "hedge_eval": lambda: GammaLike("hedge_eval", gen.HEDGE_EVAL),
        "pool21": lambda: GammaLike("pool21", gen.POOL21),
        "small_mixed": lambda: GammaLike("small_mixed", gen.SMALL_MIXED),
        "hedge_eval_tree": lambda: TreeLike("hedge_eval_tree", gen.HEDGE_EVAL, topk=8),
        "pool21_tree": lambda: TreeLike("pool21_tree", gen.POOL21, topk=8),
        "hedge_loop": lambda: LoopLike("hedge_loop", gen.HEDGE_EVAL),
    }


def load_traffic(key: str, per_launch_algo: int):
    """HBM traffic per launch from the committed PMC summary, if taken on these sources."""
    path = os.path.join(ROOT, "profiles", f"{kernel_of(key)}_{key}_pmc.json")
    if not os.path.exists(path):
        return None
    try:
        d = json.load(open(path))
    except (OSError, ValueError):
        return None
    if d.get("source_hash") != source_hash():
        return None
    return d.get("traffic_bytes_per_launch")


def summarize_pmc(key: str, fetch_csv: str, write_csv: str, calib_mib: int, command: str) -> dict:
    """Per-launch HBM traffic of the workload's kernel from two rocprofv3 --pmc counter_collection CSVs
    (FETCH_SIZE, WRITE_SIZE, both KiB per dispatch).  Each counter is scaled by what it reads
    for the plain device copy of `calib_mib` MiB that the same run made (--copy-calib-mib)."""
    import csv
    kernel = kernel_of(key)

    def per_kernel(path, counter):
        mine, calib = [], []
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            v = float(r["Counter_Value"])
            # plain or template instance, with or without the demangled return type
            if re.match(rf"(void )?specv::{kernel}(<[^>]*>)?\(", r["Kernel_Name"]):
                mine.append(v)
            elif "copyBuffer" in r["Kernel_Name"] and v > 0.4 * calib_mib * 1024:
                calib.append(v)
        if not mine or not calib:
            raise SystemExit(f"{path}: no {kernel} dispatches or no calibration copy for {counter}")
        return float(np.mean(mine)), float(np.mean(calib[-3:])), len(mine)

    f_k, f_c, nf = per_kernel(fetch_csv, "FETCH_SIZE")
    w_k, w_c, nw = per_kernel(write_csv, "WRITE_SIZE")
    expect = calib_mib * 1024.0
    f_scale, w_scale = expect / f_c, expect / w_c
    traffic = (f_k * f_scale + w_k * w_scale) * 1024.0
    return {"kernel": kernel, "workload": key, "source_hash": source_hash(),
            "fetch_kib_raw": f_k, "write_kib_raw": w_k, "dispatches": [nf, nw],
            "calib_copy_mib": calib_mib, "calib_fetch_kib_raw": f_c, "calib_write_kib_raw": w_c,
            "fetch_scale": f_scale, "write_scale": w_scale,
            "traffic_bytes_per_launch": traffic, "command": command}


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=60)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--warmup-ms", type=float, default=100.0,
                    help="keep warming up (whole steps) until this much GPU time has passed, so that the "
                         "clocks have settled before the timed steps")
    ap.add_argument("--workload", default="llama_sps")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of the oracle CPU baseline (0: skip)")
    ap.add_argument("--copies-gib", type=float, default=1.0)
    ap.add_argument("--reps", type=int, default=200,
                    help="launches after the timed steps for the spread of the launch duration (0: skip)")
    ap.add_argument("--copy-calib-mib", type=int, default=0,
                    help="also run a plain device copy of this many MiB (PMC calibration)")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/<kernel>_<workload>_pmc.json from two rocprofv3 --pmc "
                         "counter_collection CSVs of this script run with --copy-calib-mib, then exit")
    ap.add_argument("--pmc-command", default="", help="the rocprofv3 command recorded in the summary")
    args = ap.parse_args(argv)

    if args.pmc_summary:
        d = summarize_pmc(args.workload, *args.pmc_summary, args.copy_calib_mib or 256, args.pmc_command)
        path = os.path.join(ROOT, "profiles", f"{kernel_of(args.workload)}_{args.workload}_pmc.json")
        with open(path, "w") as f:
            json.dump(d, f, indent=1)
            f.write("\n")
        print(json.dumps(d, indent=1))
        return 0

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(sequences shard across GPUs with no exchange; see the design notes).", file=sys.stderr)
        return 2

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    torch.cuda.set_device(0)
    from speculative_sampling_verification_row_amd import binding
    binding.load()

    wl = workloads()[args.workload]()
    wl.setup(int(args.copies_gib * (1 << 30)))
    torch.cuda.synchronize()

    if args.copy_calib_mib > 0:
        n = args.copy_calib_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"calibration copy: {args.copy_calib_mib} MiB x 3")

    # Warm-up: at least W steps, and whole steps until --warmup-ms have passed: with
    # 10 steps (0.5 ms on llama_sps) the timed steps ran while the GPU's clocks were
    # still rising and measured 4-12% slower than the steady state.
    warm = 0
    t_w = time.perf_counter()
    while warm < args.warmup or (time.perf_counter() - t_w) * 1e3 < args.warmup_ms:
        for _ in range(max(1, args.warmup) if warm < args.warmup else 10):
            wl.launch(warm)
            warm += 1
        torch.cuda.synchronize()

    # The K launches run back to back between one pair of HIP events recorded on the
    # launching stream (torch's current stream, which the binding launches on): the
    # mean launch duration is their span / K.  An event pair around every launch would
    # add its own fence and timestamp work to each launch.
    K = args.steps
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record()
    for i in range(K):
        wl.launch(warm + i)
    ev1.record()
    t_enq = time.perf_counter() - t0
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / K
    mean_launch_s = ev0.elapsed_time(ev1) * 1e-3 / K
    achieved = wl.algo_bytes / mean_launch_s / 1e9
    log(f"launch ms: mean {mean_launch_s * 1e3:.4f} (HIP events around {K} back-to-back launches); "
        f"wall/step {ms_step:.4f} ms; {achieved:.0f} GB/s algorithmic; host enqueue {t_enq * 1e6 / K:.1f} us/step")
    # The spread, after the timed steps: args.reps more launches in back-to-back
    # batches of 10, each batch between its own pair of events (a sample is a batch's
    # mean launch duration).
    dist = None
    if args.reps >= 10:
        nb = args.reps // 10
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(nb)]
        torch.cuda.synchronize()
        for j in range(nb):
            evs[j][0].record()
            for i in range(10):
                wl.launch(warm + K + 10 * j + i)
            evs[j][1].record()
        torch.cuda.synchronize()
        per = np.array([a.elapsed_time(b) / 10.0 for a, b in evs])
        dist = {"reps": nb * 10, "batch": 10, "median_ms": float(np.median(per)),
                "p10_ms": float(np.percentile(per, 10)), "p90_ms": float(np.percentile(per, 90))}
        log(f"launch ms over {nb * 10} more launches (batches of 10): median {dist['median_ms']:.4f} "
            f"p10 {dist['p10_ms']:.4f} p90 {dist['p90_ms']:.4f}")

    traffic = load_traffic(wl.key, wl.algo_bytes)

    cpu = None
    if args.cpu_seconds > 0 and wl.positions > 0:
        log(f"oracle CPU baseline, one core, ~{args.cpu_seconds:.0f} s")
        pos, secs, cpu_secs, sample = wl.cpu_sample(args.cpu_seconds)
        cores1 = max(1, int(round(cpu_secs / secs)))
        single = {"value": pos / secs, "unit": "positions/s", "cores": cores1,
                  "sample": f"{sample} ({pos} positions in {secs:.1f} s, float64 numpy)"}
        cpu = dict(single, kind="oracle", cpu_model=cpu_model())
        ncores = host_cores()
        if ncores > 1 and hasattr(wl, "cpu_kind"):
            kind, extra = wl.cpu_kind()
            per_seq = pos / wl.w.K          # sequences the one-core leg did
            n_seq = max(ncores, int(per_seq / secs * args.cpu_seconds * ncores))
            log(f"oracle CPU baseline, {ncores} processes, {n_seq} sequences")
            wall = cpu_all_cores(kind, wl.x, extra, wl.w.B, n_seq, ncores)
            cpu = {"value": n_seq * wl.w.K / wall, "unit": "positions/s", "cores": ncores, "kind": "oracle",
                   "sample": f"{n_seq} sequences of this batch (cycling), one per task, on {ncores} spawned "
                             f"processes in {wall:.1f} s, float64 numpy",
                   "cpu_model": cpu_model(), "single_core": single}

    if wl.key == "stream_read":
        print(json.dumps({"metric": "streaming read bandwidth", "value": achieved, "unit": "GB/s",
                          "n_gpus": 1, "steps": K, "ms_per_step": ms_step, "higher_is_better": True,
                          "config": {"workload": wl.desc, "bytes_per_step": wl.algo_bytes},
                          "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                       "frac": achieved / HBM_PEAK_GBS, "kernel": kernel_of(wl.key),
                                       "mean_launch_ms": mean_launch_s * 1e3, "launch_spread": dist}}), flush=True)
        return 0

    out = {
        "metric": "verified draft positions/sec at V=128k-152k",
        "value": wl.positions / (ms_step * 1e-3),
        "unit": "positions/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": warm,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wl.desc, "positions_per_step": wl.positions,
                   "algorithmic_bytes_per_step": wl.algo_bytes, "bonus_rows_per_step": wl.bonus_rows},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": kernel_of(args.workload), "mean_launch_ms": mean_launch_s * 1e3,
                     "launch_spread": dist},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
