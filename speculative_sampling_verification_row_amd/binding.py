"""ctypes binding of libspecverify.so: torch tensors in, raw pointers to the C ABI.

Argument marshalling only -- every step of the computation runs in the HIP
kernels of the library.  The library is loaded on first use; if it has not
been built, calls raise instead of falling back to anything else.

Logits are passed as torch.bfloat16 (or int16/uint16 bit patterns) on the GPU,
laid out [B, rows, V] with unit stride along V.  When the row stride is not a
multiple of 8 elements (for example V not a multiple of 8 in a contiguous
tensor) the rows are copied into a padded buffer first, because the kernels
stream rows with 16-byte loads.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libspecverify.so")

SPEC_OK = 0
STATUS = {0: "SPEC_OK", -1: "SPEC_ERR_NULL", -2: "SPEC_ERR_SHAPE", -3: "SPEC_ERR_PARAM",
          -4: "SPEC_ERR_ALIGN", -5: "SPEC_ERR_WORKSPACE", -6: "SPEC_ERR_HIP", -7: "SPEC_ERR_TOO_LARGE"}
LEARNER_NORMALHEDGE = 0
LEARNER_HEDGE = 1
FAULT_WORD_OFFSET = 12  # byte offset of the workspace's fault word

_lib = None

_P = ctypes.c_void_p
_I = ctypes.c_int
_I64 = ctypes.c_int64
_F = ctypes.c_float
_SZ = ctypes.c_size_t

_SIGNATURES = {
    "spec_status_str": (ctypes.c_char_p, [_I]),
    "spec_workspace_bytes": (_SZ, [_I, _I, _I]),
    "spec_workspace_init": (_I, [_P, _SZ, _P]),
    "spec_verify": (_I, [_P, _I64, _P, _I64, _P, _P, _P, _I, _I, _I, _F, _P, _P, _P, _P, _SZ, _P]),
    "spec_cactus_verify": (_I, [_P, _I64, _P, _I64, _P, _P, _P, _I, _I, _I, _F, _F, _P, _P, _P, _P, _P, _SZ, _P]),
    "spec_cactus_kl_verify": (_I, [_P, _I64, _P, _I64, _P, _P, _P, _I, _I, _I, _F, _F, _P, _P, _P, _P, _P, _SZ, _P]),
    "hedge_exp_update": (_I, [_P, _P, _P, _P, _F, _F, _P, _P, _I, _I, _P]),
    "spec_acceptance_loss": (_I, [_P, _P, _I, _I, _I, _P]),
    "hedge_queue_update": (_I, [_P, _P, _P, _P, _P, _P, _P, _F, _P, _P, _P, _I, _I, _I, _I, _P]),
    "spec_tree_gamma": (_I, [_P, _I64, _I, _P, _I64, _I64, _I, _I, _I, _I, _I, _F, _P, _P, _SZ, _P]),
    "spec_tree_workspace_bytes": (_SZ, [_I, _I, _I, _I, _I]),
    "spec_counterfactual_gamma": (_I, [_P, _I64, _I, _P, _I64, _I64, _P, _I, _I, _I, _I, _F, _P, _P, _P,
                                       _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "hedge_update": (_I, [_P, _P, _P, _P, _F, _P, _P, _I, _I, _P]),
    "hedge_censored_update": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _F, _F, _P, _P, _P, _I, _I, _I, _I, _P]),
    "spec_hedgespec_round": (_I, [_P, _I64, _I, _P, _I64, _I64, _P, _I, _I, _I, _I, _F, _P, _P, _P, _P, _P, _P,
                                  _P, _P, _P, _P, _P, _P, _P, _P, _I, _F, _F, _P, _P, _P, _I, _I, _P, _SZ, _P]),
}


class SpecError(RuntimeError):
    """A non-zero status from the C ABI."""

    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {STATUS.get(status, status)}")
        self.status = status


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the HIP library (once) and declare its signatures."""
    global _lib
    if _lib is None:
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built; run __graft_entry__.build() "
                               "or python -m speculative_sampling_verification_row_amd.build")
        lib = ctypes.CDLL(path)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def _check(fn: str, status: int) -> None:
    if status != SPEC_OK:
        raise SpecError(fn, status)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _need_cuda(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("all tensors must be on the GPU")


def as_rows(x: torch.Tensor) -> tuple:
    """Logits [..., rows, V] -> (tensor, row_stride) with a uniform row pitch that
    is a multiple of 8 elements and 16-byte-aligned rows (copying if needed)."""
    if x.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise ValueError("logits must be bf16 (or raw 16-bit patterns)")
    V = x.shape[-1]
    lead = x.shape[:-1]
    rows = 1
    for d in lead:
        rows *= d
    ok = x.stride(-1) == 1
    if ok and len(lead) > 0:
        pitch = x.stride(-2)
        expect = pitch
        for i in range(len(lead) - 1, -1, -1):
            if x.stride(i) != expect:
                ok = False
                break
            expect *= x.shape[i]
    pitch = x.stride(-2) if len(lead) > 0 else V
    if ok and pitch % 8 == 0 and pitch >= V and x.data_ptr() % 16 == 0:
        return x, pitch
    pitch = (V + 7) // 8 * 8
    buf = torch.zeros(lead + (pitch,), dtype=x.dtype, device=x.device)
    buf[..., :V] = x
    return buf, pitch


def _as(x: Optional[torch.Tensor], dtype, strict: bool, what: str) -> Optional[torch.Tensor]:
    """x as a contiguous tensor of `dtype`; with `strict`, raise instead of copying (a
    prepared launch must read the caller's own buffer if the caller rewrites it)."""
    if x is None:
        return None
    if x.dtype == dtype and x.is_contiguous():
        return x
    if strict:
        raise ValueError(f"{what} would be copied ({x.dtype}, contiguous={x.is_contiguous()}); pass a "
                         f"contiguous {dtype} tensor so that writes into it reach the launches")
    return x.to(dtype).contiguous()


def _rows(x: torch.Tensor, strict: bool, what: str) -> tuple:
    t, pitch = as_rows(x)
    if strict and t is not x:
        raise ValueError(f"{what} would be copied into padded rows; pass rows whose pitch is a multiple "
                         "of 8 elements on a 16-byte-aligned base")
    return t, pitch


def workspace_bytes(B: int, K: int, N: int = 1) -> int:
    return int(load().spec_workspace_bytes(B, K, N))


def make_workspace(B: int, K: int, N: int = 1, device="cuda") -> torch.Tensor:
    """A zeroed workspace; every completed call leaves it zero again."""
    return torch.zeros(workspace_bytes(B, K, N), dtype=torch.uint8, device=device)


class WorkspaceFault(RuntimeError):
    """A wait between a kernel's workgroups timed out: that call's outputs are unspecified."""


def workspace_fault(ws: torch.Tensor) -> int:
    """The workspace's fault word (0 = no wait between workgroups timed out); synchronises."""
    return int(ws[FAULT_WORD_OFFSET:FAULT_WORD_OFFSET + 4].view(torch.int32).item())


def check_workspace(ws: torch.Tensor, name: str = "call", stream=None) -> None:
    """Synchronise `stream` and raise WorkspaceFault if a call on `ws` timed out in a wait
    between its workgroups (the device was shared with work that kept part of the grid
    from running).  The workspace is zeroed again before raising, so it can be reused."""
    s = torch.cuda.current_stream() if stream is None else stream
    s.synchronize()
    if workspace_fault(ws) != 0:
        workspace_init(ws, stream)
        s.synchronize()
        raise WorkspaceFault(f"{name}: a wait between workgroups timed out; outputs are unspecified "
                             "(the kernel needs every workgroup of its grid resident: no concurrent kernels)")


def workspace_init(ws: torch.Tensor, stream=None) -> None:
    _check("spec_workspace_init", load().spec_workspace_init(_ptr(ws), ws.numel(), _stream(stream)))


class Launcher:
    """One call with its tensors fixed: launch() only enqueues the kernel -- no
    allocation, no synchronisation and no checks beyond the C ABI's own -- and
    returns the outputs (overwritten by every launch).  check() is the
    synchronisation point: it waits for the stream and raises WorkspaceFault if a
    launch since the last check timed out.  `inputs` are the device tensors the
    kernel reads (a caller streaming new rows writes into these).  It keeps every
    tensor it points to alive."""

    def __init__(self, name: str, args: tuple, outputs, keep: tuple, workspace=None, inputs=None):
        self.name = name
        self._fn = getattr(load(), name)
        self._args = args
        self.outputs = outputs
        self._keep = keep
        self.workspace = workspace
        self.inputs = inputs or {}

    def launch(self, stream=None):
        st = self._fn(*self._args, _stream(stream))
        if st != SPEC_OK:
            raise SpecError(self.name, st)
        return self.outputs

    def check(self, stream=None) -> None:
        if self.workspace is not None:
            check_workspace(self.workspace, self.name, stream)

    def run(self, stream=None):
        """launch(), then check(): one synchronous call."""
        out = self.launch(stream)
        self.check(stream)
        return out


def spec_verify(target, draft, draft_tokens, r_accept, u_resample, temperature: float = 1.0, *,
                workspace: Optional[torch.Tensor] = None, with_mask: bool = True, stream=None):
    """Lossless verification.  target [B, K+1, V], draft [B, K, V] bf16; draft_tokens [B, K]
    int32; r_accept [B, K], u_resample [B, K+1] float32.  Returns (accepted_len [B],
    out_token [B], accept_mask [B, K] or None)."""
    return prepare_verify(target, draft, draft_tokens, r_accept, u_resample, temperature, workspace=workspace,
                          with_mask=with_mask).run(stream)


def spec_cactus_verify(verifier, draft, draft_tokens, r_accept, u_resample, delta: float,
                       temperature: float = 1.0, *, workspace=None, with_mask: bool = True,
                       with_gamma_star: bool = True, stream=None):
    """Cactus verification; returns (accepted_len, out_token, accept_mask, gamma_star)."""
    return prepare_cactus_verify(verifier, draft, draft_tokens, r_accept, u_resample, delta, temperature,
                                 workspace=workspace, with_mask=with_mask,
                                 with_gamma_star=with_gamma_star).run(stream)


def spec_cactus_kl_verify(verifier, draft, draft_tokens, r_accept, u_resample, delta: float,
                          temperature: float = 1.0, *, workspace=None, with_mask: bool = True,
                          with_gamma_star: bool = True, stream=None):
    """Cactus verification with gamma* the exact root of the KL budget; returns
    (accepted_len, out_token, accept_mask, gamma_star)."""
    return prepare_cactus_verify(verifier, draft, draft_tokens, r_accept, u_resample, delta, temperature,
                                 workspace=workspace, with_mask=with_mask, with_gamma_star=with_gamma_star,
                                 exact_kl=True).run(stream)


def prepare_verify(target, draft, draft_tokens, r_accept, u_resample, temperature: float = 1.0, *,
                   workspace: Optional[torch.Tensor] = None, with_mask: bool = True) -> Launcher:
    """spec_verify with its tensors fixed (see Launcher)."""
    return _prepare_verify("spec_verify", target, draft, draft_tokens, r_accept, u_resample, None, temperature,
                           workspace, with_mask, False)


def prepare_cactus_verify(verifier, draft, draft_tokens, r_accept, u_resample, delta: float,
                          temperature: float = 1.0, *, workspace=None, with_mask: bool = True,
                          with_gamma_star: bool = True, exact_kl: bool = False) -> Launcher:
    """spec_cactus_verify (spec_cactus_kl_verify with exact_kl) with its tensors fixed (see Launcher)."""
    name = "spec_cactus_kl_verify" if exact_kl else "spec_cactus_verify"
    return _prepare_verify(name, verifier, draft, draft_tokens, r_accept, u_resample, delta,
                           temperature, workspace, with_mask, with_gamma_star)


def _prepare_verify(name, target, draft, tokens, r, u, delta, temperature, workspace, with_mask, with_gstar):
    _need_cuda(target, draft, tokens, r, u)
    B, K1, V = target.shape
    K = K1 - 1
    if tuple(draft.shape) != (B, K, V):
        raise ValueError("draft must be [B, K, V] with target [B, K+1, V]")
    t, ts = as_rows(target)
    d, ds = as_rows(draft)
    tokens = tokens.to(torch.int32).contiguous()
    r = r.to(torch.float32).contiguous()
    u = u.to(torch.float32).contiguous()
    dev = target.device
    A = torch.empty(B, dtype=torch.int32, device=dev)
    tok = torch.empty(B, dtype=torch.int32, device=dev)
    mask = torch.empty((B, K), dtype=torch.uint8, device=dev) if with_mask else None
    ws = make_workspace(B, K, 1, dev) if workspace is None else workspace
    keep = (t, d, tokens, r, u, A, tok, mask, ws)
    inputs = {"target": t, "draft": d, "draft_tokens": tokens, "r_accept": r, "u_resample": u}
    if name == "spec_verify":
        args = (_ptr(t), ts, _ptr(d), ds, _ptr(tokens), _ptr(r), _ptr(u), B, K, V, float(temperature),
                _ptr(A), _ptr(tok), _ptr(mask), _ptr(ws), ws.numel())
        return Launcher(name, args, (A, tok, mask), keep, ws, inputs)
    gstar = torch.empty((B, K), dtype=torch.float32, device=dev) if with_gstar else None
    args = (_ptr(t), ts, _ptr(d), ds, _ptr(tokens), _ptr(r), _ptr(u), B, K, V, float(delta), float(temperature),
            _ptr(A), _ptr(tok), _ptr(mask), _ptr(gstar), _ptr(ws), ws.numel())
    return Launcher(name, args, (A, tok, mask, gstar), keep + (gstar,), ws, inputs)


def tree_workspace_bytes(B: int, K: int, N: int, V: int, topk: int) -> int:
    return int(load().spec_tree_workspace_bytes(B, K, N, V, topk))


def make_tree_workspace(B: int, K: int, N: int, V: int, topk: int, device="cuda") -> torch.Tensor:
    """A zeroed spec_tree_gamma workspace for vocabularies up to V; every completed call
    leaves it zero again."""
    return torch.zeros(tree_workspace_bytes(B, K, N, V, topk), dtype=torch.uint8, device=device)


def spec_tree_gamma(target, drafts, topk: int, temperature: float = 1.0, *, workspace=None, stream=None):
    """Draft-tree acceptance probabilities.  target [B, R >= K, V], drafts [N, B, K, V] bf16.
    Returns gamma [B, K, N] float32."""
    return prepare_tree_gamma(target, drafts, topk, temperature, workspace=workspace).run(stream)[0]


def prepare_tree_gamma(target, drafts, topk: int, temperature: float = 1.0, *, workspace=None) -> Launcher:
    """spec_tree_gamma with its tensors fixed (see Launcher)."""
    _need_cuda(target, drafts)
    N, B, K, V = drafts.shape
    if target.shape[0] != B or target.shape[2] != V or target.shape[1] < K:
        raise ValueError("target must be [B, R >= K, V]")
    R = target.shape[1]
    t, ts = as_rows(target)
    d, ds = as_rows(drafts)
    dstr = ds * B * K
    gamma = torch.empty((B, K, N), dtype=torch.float32, device=target.device)
    ws = make_tree_workspace(B, K, N, V, topk, target.device) if workspace is None else workspace
    args = (_ptr(t), ts, R, _ptr(d), ds, dstr, B, K, N, V, int(topk), float(temperature), _ptr(gamma), _ptr(ws),
            ws.numel())
    return Launcher("spec_tree_gamma", args, (gamma,), (t, d, gamma, ws), ws, {"target": t, "drafts": d})


def spec_counterfactual_gamma(target, drafts, traj_tokens, temperature: float = 1.0, *, sel=None,
                              draft_tokens=None, r_accept=None, u_resample=None, workspace=None,
                              with_mask: bool = True, stream=None):
    """HedgeSpec evaluation.  target [B, R, V] (R >= K; R = K+1 for the fused verify),
    drafts [N, B, K, V], traj_tokens [B, K].  Returns a dict with gamma [B, K, N],
    est_len [B, N], loss [B, N] and, when sel is given, accepted_len, out_token, accept_mask."""
    return prepare_counterfactual_gamma(target, drafts, traj_tokens, temperature, sel=sel,
                                        draft_tokens=draft_tokens, r_accept=r_accept, u_resample=u_resample,
                                        workspace=workspace, with_mask=with_mask).run(stream)


def prepare_counterfactual_gamma(target, drafts, traj_tokens, temperature: float = 1.0, *, sel=None,
                                 draft_tokens=None, r_accept=None, u_resample=None, workspace=None,
                                 with_mask: bool = True, outputs: Optional[dict] = None,
                                 strict: bool = False) -> Launcher:
    """spec_counterfactual_gamma with its tensors fixed (see Launcher).  `outputs` reuses
    the output tensors of another launcher of the same shape (so that several prepared
    calls write into the same buffers); `strict` raises instead of copying an input."""
    _need_cuda(target, drafts, traj_tokens, sel, draft_tokens, r_accept, u_resample)
    N, B, K, V = drafts.shape
    if target.shape[0] != B or target.shape[2] != V:
        raise ValueError("target must be [B, R, V]")
    R = target.shape[1]
    t, ts = _rows(target, strict, "target")
    d, ds = _rows(drafts, strict, "drafts")
    drafter_stride = ds * B * K
    traj = _as(traj_tokens, torch.int32, strict, "traj_tokens")
    dev = target.device
    fused = sel is not None
    if outputs is None:
        out = {
            "gamma": torch.empty((B, K, N), dtype=torch.float32, device=dev),
            "est_len": torch.empty((B, N), dtype=torch.float32, device=dev),
            "loss": torch.empty((B, N), dtype=torch.float32, device=dev),
        }
        if fused:
            out.update(accepted_len=torch.empty(B, dtype=torch.int32, device=dev),
                       out_token=torch.empty(B, dtype=torch.int32, device=dev),
                       accept_mask=torch.empty((B, K), dtype=torch.uint8, device=dev) if with_mask else None)
    else:
        out = outputs
    A = out.get("accepted_len") if fused else None
    tok = out.get("out_token") if fused else None
    mask = out.get("accept_mask") if fused else None
    if fused:
        sel = _as(sel, torch.int32, strict, "sel")
        draft_tokens = _as(draft_tokens, torch.int32, strict, "draft_tokens")
        r_accept = _as(r_accept, torch.float32, strict, "r_accept")
        u_resample = _as(u_resample, torch.float32, strict, "u_resample")
    ws = make_workspace(B, K, N, dev) if workspace is None else workspace
    args = (_ptr(t), ts, R, _ptr(d), ds, drafter_stride, _ptr(traj), B, K, N, V, float(temperature),
            _ptr(out["gamma"]), _ptr(out["est_len"]), _ptr(out["loss"]), _ptr(sel), _ptr(draft_tokens),
            _ptr(r_accept), _ptr(u_resample), _ptr(A), _ptr(tok), _ptr(mask), _ptr(ws), ws.numel())
    keep = (t, d, traj, sel, draft_tokens, r_accept, u_resample, ws, out)
    inputs = {"target": t, "drafts": d, "traj_tokens": traj, "sel": sel, "draft_tokens": draft_tokens,
              "r_accept": r_accept, "u_resample": u_resample}
    return Launcher("spec_counterfactual_gamma", args, out, keep, ws, inputs)


def prepare_hedgespec_round(target, drafts, traj_tokens, temperature: float, learner, *, draft_tokens,
                            r_accept, u_resample, workspace=None, with_mask: bool = True,
                            outputs: Optional[dict] = None, strict: bool = False) -> Launcher:
    """spec_hedgespec_round with its tensors fixed: one HedgeSpec round in one launch.
    `learner` holds the censoring learner's device state (state, weights, queue_loss,
    queue_tokens, round, sel, sel_hist, v, K, learner, eta, loss_scale: a
    hedge.CensoredLearner); outputs["loss"] and outputs["accepted_len"] are the
    previous round's for the learner and this round's after the launch."""
    _need_cuda(target, drafts, traj_tokens, draft_tokens, r_accept, u_resample)
    N, B, K, V = drafts.shape
    if target.shape[0] != B or target.shape[2] != V:
        raise ValueError("target must be [B, R, V]")
    R = target.shape[1]
    t, ts = _rows(target, strict, "target")
    d, ds = _rows(drafts, strict, "drafts")
    drafter_stride = ds * B * K
    traj = _as(traj_tokens, torch.int32, strict, "traj_tokens")
    dev = target.device
    if outputs is None:
        out = {
            "gamma": torch.empty((B, K, N), dtype=torch.float32, device=dev),
            "est_len": torch.empty((B, N), dtype=torch.float32, device=dev),
            "loss": torch.zeros((B, N), dtype=torch.float32, device=dev),
            "accepted_len": torch.zeros(B, dtype=torch.int32, device=dev),
            "out_token": torch.empty(B, dtype=torch.int32, device=dev),
            "accept_mask": torch.empty((B, K), dtype=torch.uint8, device=dev) if with_mask else None,
        }
    else:
        out = outputs
    draft_tokens = _as(draft_tokens, torch.int32, strict, "draft_tokens")
    r_accept = _as(r_accept, torch.float32, strict, "r_accept")
    u_resample = _as(u_resample, torch.float32, strict, "u_resample")
    L = learner
    for x, dt in ((L.state, torch.float64), (L.weights, torch.float64), (L.queue_loss, torch.float64),
                  (L.queue_tokens, torch.int32), (L.round, torch.int32), (L.v, torch.float32),
                  (L.sel, torch.int32), (L.sel_hist, torch.int32)):
        if x.dtype != dt or not x.is_contiguous() or not x.is_cuda:
            raise ValueError(f"learner state: expected a contiguous {dt} device tensor")
    if int(L.K) != K or tuple(L.state.shape) != (B, N):
        raise ValueError("the learner's shape does not match the round's")
    Q = L.queue_tokens.shape[1]
    T = L.v.shape[0]
    ws = make_workspace(B, K, N, dev) if workspace is None else workspace
    args = (_ptr(t), ts, R, _ptr(d), ds, drafter_stride, _ptr(traj), B, K, N, V, float(temperature),
            _ptr(out["gamma"]), _ptr(out["est_len"]), _ptr(out["loss"]), _ptr(draft_tokens), _ptr(r_accept),
            _ptr(u_resample), _ptr(out["accepted_len"]), _ptr(out["out_token"]), _ptr(out.get("accept_mask")),
            _ptr(L.state), _ptr(L.weights), _ptr(L.queue_loss), _ptr(L.queue_tokens), _ptr(L.round),
            int(L.learner), float(L.eta), float(L.loss_scale), _ptr(L.v), _ptr(L.sel), _ptr(L.sel_hist), Q, T,
            _ptr(ws), ws.numel())
    keep = (t, d, traj, draft_tokens, r_accept, u_resample, ws, out, L)
    inputs = {"target": t, "drafts": d, "traj_tokens": traj, "draft_tokens": draft_tokens,
              "r_accept": r_accept, "u_resample": u_resample}
    return Launcher("spec_hedgespec_round", args, out, keep, ws, inputs)


def hedge_update(cum_regret, weights, loss, loss_scale: float, *, has_loss=None, v_select=None,
                 sel_out=None, stream=None):
    """One NormalHedge round per sequence, in place on cum_regret / weights ([B, N] float64).
    Returns sel_out [B] int32 when v_select is given."""
    lib = load()
    _need_cuda(cum_regret, weights, loss, has_loss, v_select)
    if cum_regret.dtype != torch.float64 or weights.dtype != torch.float64:
        raise ValueError("learner state must be float64")
    if not (cum_regret.is_contiguous() and weights.is_contiguous()):
        raise ValueError("learner state must be contiguous")
    B, N = cum_regret.shape
    loss = loss.to(torch.float32).contiguous()
    if has_loss is not None:
        has_loss = has_loss.to(torch.uint8).contiguous()
    if v_select is not None:
        v_select = v_select.to(torch.float32).contiguous()
        if sel_out is None:
            sel_out = torch.empty(B, dtype=torch.int32, device=cum_regret.device)
    st = lib.hedge_update(_ptr(cum_regret), _ptr(weights), _ptr(loss), _ptr(has_loss), float(loss_scale),
                          _ptr(v_select), _ptr(sel_out), B, N, _stream(stream))
    _check("hedge_update", st)
    return sel_out


def hedge_exp_update(cum_loss, weights, loss, loss_scale: float, eta: float, *, has_loss=None, v_select=None,
                     sel_out=None, stream=None):
    """One exponential-weights Hedge round per sequence, in place on cum_loss / weights ([B, N]
    float64).  Returns sel_out [B] int32 when v_select is given."""
    lib = load()
    _need_cuda(cum_loss, weights, loss, has_loss, v_select)
    if cum_loss.dtype != torch.float64 or weights.dtype != torch.float64:
        raise ValueError("learner state must be float64")
    if not (cum_loss.is_contiguous() and weights.is_contiguous()):
        raise ValueError("learner state must be contiguous")
    B, N = cum_loss.shape
    loss = loss.to(torch.float32).contiguous()
    if has_loss is not None:
        has_loss = has_loss.to(torch.uint8).contiguous()
    if v_select is not None:
        v_select = v_select.to(torch.float32).contiguous()
        if sel_out is None:
            sel_out = torch.empty(B, dtype=torch.int32, device=cum_loss.device)
    st = lib.hedge_exp_update(_ptr(cum_loss), _ptr(weights), _ptr(loss), _ptr(has_loss), float(loss_scale),
                              float(eta), _ptr(v_select), _ptr(sel_out), B, N, _stream(stream))
    _check("hedge_exp_update", st)
    return sel_out


def spec_acceptance_loss(gamma, *, out=None, stream=None):
    """Acceptance-probability loss of a chunk: sum over positions of 1 - gamma.
    gamma [B, K, N] float32 -> loss [B, N] float32."""
    lib = load()
    _need_cuda(gamma)
    gamma = gamma.to(torch.float32).contiguous()
    B, K, N = gamma.shape
    if out is None:
        out = torch.empty((B, N), dtype=torch.float32, device=gamma.device)
    _check("spec_acceptance_loss", lib.spec_acceptance_loss(_ptr(gamma), _ptr(out), B, K, N, _stream(stream)))
    return out


def hedge_censored_update(state, weights, queue_loss, queue_tokens, round_, loss, accepted_len, K: int,
                          learner: int, eta: float, loss_scale: float, v_select, sel_out, sel_hist, stream=None):
    """One round of the censoring-delay queue (see the C header); every tensor is the
    caller's device state, updated in place."""
    lib = load()
    _need_cuda(state, weights, queue_loss, queue_tokens, round_, loss, accepted_len, v_select, sel_out, sel_hist)
    for x, dt in ((state, torch.float64), (weights, torch.float64), (queue_loss, torch.float64),
                  (queue_tokens, torch.int32), (round_, torch.int32), (loss, torch.float32),
                  (accepted_len, torch.int32), (v_select, torch.float32), (sel_out, torch.int32),
                  (sel_hist, torch.int32)):
        if x.dtype != dt or not x.is_contiguous():
            raise ValueError(f"expected a contiguous {dt} tensor")
    B, N = state.shape
    Q = queue_tokens.shape[1]
    T = v_select.shape[0]
    st = lib.hedge_censored_update(_ptr(state), _ptr(weights), _ptr(queue_loss), _ptr(queue_tokens), _ptr(round_),
                                   _ptr(loss), _ptr(accepted_len), int(K), int(learner), float(eta),
                                   float(loss_scale), _ptr(v_select), _ptr(sel_out), _ptr(sel_hist), B, N, Q, T,
                                   _stream(stream))
    _check("hedge_censored_update", st)


def hedge_queue_update(cum_regret, weights, queue_loss, queue_due, round_, loss, delays, loss_scale: float,
                       v_select, sel_out, sel_hist, stream=None):
    """One round of the scheduled-delay NormalHedge queue (see the C header); in place."""
    lib = load()
    _need_cuda(cum_regret, weights, queue_loss, queue_due, round_, loss, delays, v_select, sel_out, sel_hist)
    B, N = cum_regret.shape
    Q = queue_due.shape[1]
    T = v_select.shape[0]
    st = lib.hedge_queue_update(_ptr(cum_regret), _ptr(weights), _ptr(queue_loss), _ptr(queue_due), _ptr(round_),
                                _ptr(loss), _ptr(delays), float(loss_scale), _ptr(v_select), _ptr(sel_out),
                                _ptr(sel_hist), B, N, Q, T, _stream(stream))
    _check("hedge_queue_update", st)


class StreamProbe:
    """The streaming-read probe (libstreamprobe.so): read a device buffer with the
    statistics phase's access pattern; a measurement aid, not part of the path."""

    def __init__(self, path: str = os.path.join(_HERE, "libstreamprobe.so")):
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built; run __graft_entry__.build()")
        self._lib = ctypes.CDLL(path)
        self._lib.stream_read_probe.restype = _I
        self._lib.stream_read_probe.argtypes = [_P, ctypes.c_uint64, _P, _I, _P]

    def read(self, buf: torch.Tensor, out: torch.Tensor, grid: int, stream=None) -> None:
        st = self._lib.stream_read_probe(_ptr(buf), buf.numel() * buf.element_size(), _ptr(out), int(grid),
                                         _stream(stream))
        if st != 0:
            raise RuntimeError(f"stream_read_probe failed ({st})")
