"""Host-side pieces of bench.py (no GPU): the one-GPU guard, the kernel each workload
times, and the source hash that decides whether recorded counters still apply."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, cwd=ROOT, timeout=120)
    assert res.returncode != 0
    assert "one GPU" in (res.stdout + res.stderr) or "1 GPU" in (res.stdout + res.stderr)


def test_workloads_map_to_their_kernels():
    assert bench.kernel_of("llama_sps") == "verify_kernel"
    assert bench.kernel_of("qwen_cactus_kl") == "verify_kernel"
    assert bench.kernel_of("hedge_eval") == "gamma_kernel" and bench.kernel_of("hedge_loop") == "gamma_kernel"
    assert bench.kernel_of("pool21_tree") == "tree_kernel"
    assert set(bench.workloads()) >= {"llama_sps", "qwen_cactus", "qwen_cactus_kl", "hedge_eval", "pool21",
                                      "hedge_eval_tree", "pool21_tree", "hedge_loop"}


def test_source_hash_ignores_comments_only(tmp_path, monkeypatch):
    src = tmp_path / "speculative_sampling_verification_row_amd" / "csrc"
    src.mkdir(parents=True)
    f = src / "k.hip"
    f.write_text("int a = 1; // note\n/* block */ int b = 2;\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h0 = bench.source_hash()
    f.write_text("int a = 1;   // another note\n\n/* other\n block */ int b = 2;\n")
    assert bench.source_hash() == h0
    f.write_text("int a = 1; int b = 3;\n")
    assert bench.source_hash() != h0
