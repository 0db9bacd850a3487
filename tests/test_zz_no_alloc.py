"""spec_verify_noalloc (the verification entry point that allocates nothing: its workspace
is a device array inside the library) against spec_verify on the same inputs, through the
C ABI: two calls in a row, the second with a smaller input, each bit-identical to
spec_verify's results and matching the oracle under the parity rules; a call whose layout
exceeds the array is refused before anything is launched."""

import ctypes

import numpy as np
import pytest

import oracle
from speculative_sampling_verification_row_amd import inputs as gen

from gpu_util import banner, dev_bf16, dev_f32, dev_i32
from parity import compare_verify, to_np

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def lib():
    from speculative_sampling_verification_row_amd import binding
    L = binding.load()
    f = L.spec_verify_noalloc
    P, I, I64, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float
    f.restype = I
    f.argtypes = [P, I64, P, I64, P, P, P, I, I, I, F, P, P, P, P]
    return binding, L


def case(B, K, V, seed):
    w = gen.SpsWorkload("noalloc", B=B, K=K, V=V, target_sigma=2.5, draft_sigma=0.8, peak_frac=0.01,
                        config_id=93)
    return gen.make_sps_inputs(w, seed=seed)


def call_noalloc(binding, L, x):
    B, K1, V = x["target"].shape
    K = K1 - 1
    # rows on a pitch that is a multiple of 8 elements (a ragged V is padded)
    t, ts = binding.as_rows(dev_bf16(x["target"]))
    d, ds = binding.as_rows(dev_bf16(x["draft"]))
    tok, r, u = dev_i32(x["draft_tokens"]), dev_f32(x["r"]), dev_f32(x["u"])
    A = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    o = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    m = torch.full((B, K), 7, dtype=torch.uint8, device="cuda")
    P = binding._ptr
    st = L.spec_verify_noalloc(P(t), ts, P(d), ds, P(tok), P(r), P(u), B, K, V, 1.0, P(A), P(o), P(m),
                               binding._stream())
    assert st == 0, st
    torch.cuda.synchronize()
    return to_np(A), to_np(o), to_np(m)


def test_noalloc_matches_spec_verify_twice(lib):
    binding, L = lib
    for B, K, V, seed in [(64, 5, 128256, 1), (7, 3, 20001, 2)]:
        banner(f"noalloc B={B} K={K} V={V}")
        x = case(B, K, V, seed)
        got = call_noalloc(binding, L, x)
        ws = binding.make_workspace(B, K, 1)
        ref = binding.spec_verify(dev_bf16(x["target"]), dev_bf16(x["draft"]), dev_i32(x["draft_tokens"]),
                                  dev_f32(x["r"]), dev_f32(x["u"]), workspace=ws)
        for a, b in zip(got, ref):
            np.testing.assert_array_equal(a, to_np(b))
        compare_verify(oracle.spec_verify(x["target"], x["draft"], x["draft_tokens"], x["r"], x["u"]), *got,
                       f"noalloc B={B}")


def test_noalloc_refuses_a_layout_beyond_its_array(lib):
    binding, L = lib
    P = ctypes.c_void_p(16)   # never dereferenced: the call returns before any launch
    B, K, V = 4096, 20, 1000
    assert L.spec_workspace_bytes(B, K, 1) > (16 << 20)
    st = L.spec_verify_noalloc(P, V, P, V, P, P, P, B, K, V, 1.0, P, P, P, binding._stream())
    assert st == -7
    assert L.spec_status_str(-7)
