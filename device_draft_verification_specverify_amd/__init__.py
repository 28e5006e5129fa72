"""Python binding of libspecverify: batched speculative-sampling verification on MI355X.

Argument marshalling only. Every step of the computation runs in the HIP
kernels of ``libspecverify.so``; torch supplies device memory and the stream.
The functions carry the C ABI's names (see include/specverify.h) and raise if
the library has not been built -- there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
# SPECVERIFY_LIBRARY selects another build of the library (e.g. the one with
# device-side index checks, libspecverify_checked.so).
LIBRARY = os.environ.get("SPECVERIFY_LIBRARY") or os.path.join(HERE, "libspecverify.so")

SV_F32 = 0
SV_BF16 = 1
SV_OK = 0
SV_ESCRATCH = -6
SV_ENOCHECKS = -7
NOALLOC_SCRATCH_BYTES = 32 << 20
SV_ERR_TOKEN = 1
SV_ERR_TEMP = 2
SV_ERR_ROW = 4
MAX_GAMMA = 32
MAX_CHAIN_DECISIONS = 64
MAX_FANOUT = 64

_lib = None

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_U64 = ctypes.c_uint64
_INT = ctypes.c_int
_SZ = ctypes.c_size_t

_SIGNATURES = {
    "specverify_workspace_size": (_SZ, [_I64, _I64, _I64, _I64, _INT]),
    "specverify_normalize": (_INT, [_P, _INT, _I64, _I64, _I64, _I64, _I64, _P, _P, _P, _P, _SZ, _P]),
    "specverify_accept": (_INT, [_P, _P, _I64, _I64, _I64, _U64, _P, _P, _P, _P]),
    "specverify_residual_sample": (_INT, [_P, _P, _INT, _I64, _I64, _I64, _I64, _I64, _I64, _I64,
                                          _I64, _I64, _P, _P, _P, _P, _P, _U64, _P, _P, _P, _SZ,
                                          _P]),
    "specverify_step": (_INT, [_P, _P, _INT, _P, _I64, _I64, _I64, _I64, _I64, _I64, _I64, _I64,
                               _I64, _P, _U64, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "specverify_step_noalloc": (_INT, [_P, _P, _INT, _P, _I64, _I64, _I64, _I64, _I64, _I64, _I64,
                                       _I64, _I64, _P, _U64, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "specverify_accept_prob_workspace_size": (_SZ, [_I64, _I64, _I64, _I64, _INT]),
    "specverify_accept_prob": (_INT, [_P, _P, _INT, _I64, _I64, _I64, _I64, _I64, _I64, _I64, _I64,
                                      _I64, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "specverify_geometric_fanout": (_INT, [_I64, _I64, ctypes.c_double, _P]),
    "specverify_residual_topf": (_INT, [_P, _P, _INT, _I64, _I64, _I64, _I64, _I64, _I64, _I64,
                                        _I64, _I64, _P, _P, _P, _P, _P, _P, _P]),
    "specverify_cache_lookup": (_INT, [_P, _P, _I64, _I64, _I64, _P, _P, _P, _P]),
    "specverify_bandit_state_size": (_SZ, [ctypes.c_int32]),
    "specverify_bandit_init": (_INT, [_P, _SZ, ctypes.c_int32, ctypes.c_int32, _U64, ctypes.c_double]),
    "specverify_bandit_select": (_INT, [_P, _P]),
    "specverify_bandit_update": (_INT, [_P, ctypes.c_int32, ctypes.c_double]),
    "specverify_bandit_stats": (_INT, [_P, ctypes.c_int32, _P, _P]),
    "specverify_step_reward": (_INT, [_P, _I64, _I64, _P]),
    "specverify_branch_prune": (_INT, [_P, _I64, _I64, _I64, ctypes.c_double, _I64, _P, _P, _P,
                                       _P]),
    "specverify_status_string": (ctypes.c_char_p, [_INT]),
    "specverify_version": (_INT, []),
    "specverify_time_next_stream_kernel": (_INT, [_P, _P]),
    "specverify_check_count": (_INT, [_P, _INT]),
}


class SpecVerifyError(RuntimeError):
    pass


def load_library(path: str = LIBRARY) -> ctypes.CDLL:
    """Load libspecverify.so (built by __graft_entry__.build()); raises if missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(path):
            raise SpecVerifyError(f"{path} is not built; run __graft_entry__.build() first")
        lib = ctypes.CDLL(path)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def _check(status: int, what: str) -> None:
    if status != SV_OK:
        msg = load_library().specverify_status_string(status).decode()
        raise SpecVerifyError(f"{what}: status {status} ({msg})")


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return SV_F32
    if t.dtype == torch.bfloat16:
        return SV_BF16
    raise SpecVerifyError(f"logits must be float32 or bfloat16, got {t.dtype}")


def _ptr(t: torch.Tensor | None) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _need(t: torch.Tensor, dtype: torch.dtype, shape: tuple, name: str) -> None:
    if not t.is_cuda:
        raise SpecVerifyError(f"{name} must be a device tensor")
    if t.dtype != dtype or tuple(t.shape) != tuple(shape) or not t.is_contiguous():
        raise SpecVerifyError(f"{name}: want contiguous {dtype} {tuple(shape)}, got {t.dtype} "
                              f"{tuple(t.shape)} contiguous={t.is_contiguous()}")


def _logits(t: torch.Tensor, ndim: int, name: str) -> None:
    if not t.is_cuda or t.dim() != ndim or t.stride(-1) != 1:
        raise SpecVerifyError(f"{name}: want a {ndim}-d device tensor with a contiguous last axis")


def workspace_size(B: int, K: int, gamma: int, V: int, dtype: int) -> int:
    return int(load_library().specverify_workspace_size(B, K, gamma, V, dtype))


def workspace(B: int, K: int, gamma: int, V: int, dtype: int, device) -> torch.Tensor:
    n = workspace_size(B, K, gamma, V, dtype)
    if n == 0:
        raise SpecVerifyError("sizes rejected by specverify_workspace_size")
    return torch.empty(n, dtype=torch.uint8, device=device)  # any contents will do


def specverify_normalize(logits: torch.Tensor, temperature: torch.Tensor, want_argmax: bool = False,
                         ws: torch.Tensor | None = None):
    """lnZ [B, P] float64 (and argmax [B, P] int32) of logits [B, P, V]."""
    lib = load_library()
    _logits(logits, 3, "logits")
    B, P, V = logits.shape
    _need(temperature, torch.float32, (B,), "temperature")
    dt = _dtype_code(logits)
    lnz = torch.empty((B, P), dtype=torch.float64, device=logits.device)
    am = torch.empty((B, P), dtype=torch.int32, device=logits.device) if want_argmax else None
    if ws is None:
        ws = workspace(B, 0, P - 1, V, dt, logits.device)
    st = lib.specverify_normalize(logits.data_ptr(), dt, B, P, V, logits.stride(0), logits.stride(1),
                                  temperature.data_ptr(), lnz.data_ptr(), _ptr(am), ws.data_ptr(),
                                  ws.numel(), _stream(logits.device))
    _check(st, "specverify_normalize")
    return lnz, am


def specverify_accept(logp: torch.Tensor, logq: torch.Tensor, seed: int, pos0: torch.Tensor | None = None,
                      want_bits: bool = False):
    """accept_len [B, K] int32 (and accept_bits [B, K] int32 view of uint32) from ln p/ln q [B, K, gamma]."""
    lib = load_library()
    B, K, g = logp.shape
    _need(logp, torch.float32, (B, K, g), "logp")
    _need(logq, torch.float32, (B, K, g), "logq")
    if pos0 is not None:
        _need(pos0, torch.int64, (B,), "pos0")
    n = torch.empty((B, K), dtype=torch.int32, device=logp.device)
    bits = torch.empty((B, K), dtype=torch.int32, device=logp.device) if want_bits else None
    st = lib.specverify_accept(logp.data_ptr(), logq.data_ptr(), B, K, g, seed & (2 ** 64 - 1),
                               _ptr(pos0), n.data_ptr(), _ptr(bits), _stream(logp.device))
    _check(st, "specverify_accept")
    return n, bits


def specverify_residual_sample(target: torch.Tensor, draft: torch.Tensor, temperature: torch.Tensor,
                               lnZ_target: torch.Tensor, lnZ_draft: torch.Tensor,
                               argmax_target: torch.Tensor, accept_len: torch.Tensor, seed: int,
                               pos0: torch.Tensor | None = None, ws: torch.Tensor | None = None):
    """out_token [B, K] int32 given the accept lengths (see the C header)."""
    lib = load_library()
    _logits(target, 3, "target")
    _logits(draft, 4, "draft")
    B, G1, V = target.shape
    K, g = draft.shape[1], draft.shape[2]
    if G1 != g + 1 or draft.shape[0] != B or draft.shape[3] != V or draft.dtype != target.dtype:
        raise SpecVerifyError("target [B, gamma+1, V] and draft [B, K, gamma, V] disagree")
    _need(temperature, torch.float32, (B,), "temperature")
    _need(lnZ_target, torch.float64, (B, g + 1), "lnZ_target")
    _need(lnZ_draft, torch.float64, (B, K, g), "lnZ_draft")
    _need(argmax_target, torch.int32, (B, g + 1), "argmax_target")
    _need(accept_len, torch.int32, (B, K), "accept_len")
    if pos0 is not None:
        _need(pos0, torch.int64, (B,), "pos0")
    dt = _dtype_code(target)
    out = torch.empty((B, K), dtype=torch.int32, device=target.device)
    if ws is None:
        ws = workspace(B, K, g, V, dt, target.device)
    st = lib.specverify_residual_sample(
        target.data_ptr(), draft.data_ptr(), dt, B, K, g, V, target.stride(0), target.stride(1),
        draft.stride(0), draft.stride(1), draft.stride(2), temperature.data_ptr(),
        lnZ_target.data_ptr(), lnZ_draft.data_ptr(), argmax_target.data_ptr(), accept_len.data_ptr(),
        seed & (2 ** 64 - 1), _ptr(pos0), out.data_ptr(), ws.data_ptr(), ws.numel(),
        _stream(target.device))
    _check(st, "specverify_residual_sample")
    return out


@dataclass
class StepOutputs:
    accept_len: torch.Tensor       # [B, K] int32
    out_token: torch.Tensor        # [B, K] int32
    logp: torch.Tensor | None      # [B, K, gamma] float32
    logq: torch.Tensor | None      # [B, K, gamma] float32
    lnZ_target: torch.Tensor | None  # [B, gamma+1] float64
    lnZ_draft: torch.Tensor | None   # [B, K, gamma] float64
    device_error: torch.Tensor | None  # [1] int32


class StepPlan:
    """Binds the tensors of one verification step once; each call enqueues the step.

    target [B, gamma+1, V] and draft [B, K, gamma, V] (float32 or bfloat16, last
    axis contiguous, any non-negative strides), tokens [B, K, gamma] int32,
    temperature [B] float32, pos0 [B] int64 or None. Outputs are allocated here.
    """

    def __init__(self, target, draft, tokens, temperature, seed: int, pos0=None, *,
                 want_logprobs: bool = True, want_normalizers: bool = True,
                 want_error: bool = True, ws: torch.Tensor | None = None,
                 noalloc: bool = False):
        self.lib = load_library()
        _logits(target, 3, "target")
        _logits(draft, 4, "draft")
        B, G1, V = target.shape
        K, g = draft.shape[1], draft.shape[2]
        if G1 != g + 1 or draft.shape[0] != B or draft.shape[3] != V or draft.dtype != target.dtype:
            raise SpecVerifyError("target [B, gamma+1, V] and draft [B, K, gamma, V] disagree")
        _need(tokens, torch.int32, (B, K, g), "tokens")
        _need(temperature, torch.float32, (B,), "temperature")
        if pos0 is not None:
            _need(pos0, torch.int64, (B,), "pos0")
        dev = target.device
        self.B, self.K, self.gamma, self.V = B, K, g, V
        self.dtype = _dtype_code(target)
        self.target, self.draft, self.tokens, self.temperature, self.pos0 = (
            target, draft, tokens, temperature, pos0)
        self.seed = seed & (2 ** 64 - 1)
        self.out = StepOutputs(
            accept_len=torch.empty((B, K), dtype=torch.int32, device=dev),
            out_token=torch.empty((B, K), dtype=torch.int32, device=dev),
            logp=torch.empty((B, K, g), dtype=torch.float32, device=dev) if want_logprobs else None,
            logq=torch.empty((B, K, g), dtype=torch.float32, device=dev) if want_logprobs else None,
            lnZ_target=(torch.empty((B, g + 1), dtype=torch.float64, device=dev)
                        if want_normalizers else None),
            lnZ_draft=(torch.full((B, K, g), float("nan"), dtype=torch.float64, device=dev)
                       if want_normalizers else None),
            device_error=torch.zeros(1, dtype=torch.int32, device=dev) if want_error else None,
        )
        o = self.out
        self._args = (
            target.data_ptr(), draft.data_ptr(), self.dtype, tokens.data_ptr(), B, K, g, V,
            target.stride(0), target.stride(1), draft.stride(0), draft.stride(1), draft.stride(2),
            temperature.data_ptr(), self.seed, _ptr(pos0), o.accept_len.data_ptr(),
            o.out_token.data_ptr(), _ptr(o.logp), _ptr(o.logq), _ptr(o.lnZ_target),
            _ptr(o.lnZ_draft), _ptr(o.device_error))
        if noalloc:
            # the library's own scratch (specverify_step_noalloc): no workspace here
            self.ws = None
            self._fn, self._name = self.lib.specverify_step_noalloc, "specverify_step_noalloc"
        else:
            self.ws = ws if ws is not None else workspace(B, K, g, V, self.dtype, dev)
            self._args += (self.ws.data_ptr(), self.ws.numel())
            self._fn, self._name = self.lib.specverify_step, "specverify_step"
        self.device = dev

    def __call__(self, stream: int | None = None) -> StepOutputs:
        st = self._fn(*self._args, _stream(self.device) if stream is None else stream)
        _check(st, self._name)
        return self.out


def specverify_step(target, draft, tokens, temperature, seed: int, pos0=None, **kw) -> StepOutputs:
    """One fused verification step (allocates its outputs and workspace)."""
    return StepPlan(target, draft, tokens, temperature, seed, pos0, **kw)()


def accept_prob_workspace(B: int, K: int, gamma: int, V: int, dtype: int, device) -> torch.Tensor:
    n = int(load_library().specverify_accept_prob_workspace_size(B, K, gamma, V, dtype))
    if n == 0:
        raise SpecVerifyError("sizes rejected by specverify_accept_prob_workspace_size")
    return torch.zeros(n, dtype=torch.uint8, device=device)


def specverify_accept_prob(target: torch.Tensor, draft: torch.Tensor, temperature: torch.Tensor,
                           lnZ_target: torch.Tensor, lnZ_draft: torch.Tensor,
                           want_law: bool = True, ws: torch.Tensor | None = None):
    """alpha [B, K, gamma] float64 (and the accept-length law [B, K, gamma+1]) from the
    logits of a step and its normalisers (lnZ_target [B, gamma+1], lnZ_draft [B, K, gamma])."""
    lib = load_library()
    _logits(target, 3, "target")
    _logits(draft, 4, "draft")
    B, G1, V = target.shape
    K, g = draft.shape[1], draft.shape[2]
    if G1 != g + 1 or draft.shape[0] != B or draft.shape[3] != V or draft.dtype != target.dtype:
        raise SpecVerifyError("target [B, gamma+1, V] and draft [B, K, gamma, V] disagree")
    _need(temperature, torch.float32, (B,), "temperature")
    _need(lnZ_target, torch.float64, (B, g + 1), "lnZ_target")
    _need(lnZ_draft, torch.float64, (B, K, g), "lnZ_draft")
    dt = _dtype_code(target)
    dev = target.device
    if ws is None:
        ws = accept_prob_workspace(B, K, g, V, dt, dev)
    alpha = torch.empty((B, K, g), dtype=torch.float64, device=dev)
    law = torch.empty((B, K, g + 1), dtype=torch.float64, device=dev) if want_law else None
    st = lib.specverify_accept_prob(
        target.data_ptr(), draft.data_ptr(), dt, B, K, g, V, target.stride(0), target.stride(1),
        draft.stride(0), draft.stride(1), draft.stride(2), temperature.data_ptr(),
        lnZ_target.data_ptr(), lnZ_draft.data_ptr(), alpha.data_ptr(), _ptr(law), ws.data_ptr(),
        ws.numel(), _stream(dev))
    _check(st, "specverify_accept_prob")
    return alpha, law


def _fanout_array(fanout):
    arr = (ctypes.c_int32 * len(fanout))(*[int(f) for f in fanout])
    return arr


def geometric_fanout(gamma: int, total: int, ratio: float) -> list:
    """Candidates per outcome n = 0..gamma, proportional to ratio**n, summing to total."""
    out = (ctypes.c_int32 * (gamma + 1))()
    _check(load_library().specverify_geometric_fanout(gamma, total, float(ratio), out),
           "specverify_geometric_fanout")
    return list(out)


def specverify_residual_topf(target: torch.Tensor, draft: torch.Tensor, temperature: torch.Tensor,
                             lnZ_target: torch.Tensor, lnZ_draft: torch.Tensor, fanout,
                             want_weights: bool = False):
    """cand [B, K, sum F] int32 (outcome-major, best first, -1 padding) and optionally their
    float32 weights, for the fan-out F_0..F_gamma (a host sequence)."""
    lib = load_library()
    _logits(target, 3, "target")
    _logits(draft, 4, "draft")
    B, G1, V = target.shape
    K, g = draft.shape[1], draft.shape[2]
    if G1 != g + 1 or draft.shape[0] != B or draft.shape[3] != V or draft.dtype != target.dtype:
        raise SpecVerifyError("target [B, gamma+1, V] and draft [B, K, gamma, V] disagree")
    if len(fanout) != g + 1:
        raise SpecVerifyError(f"fanout needs gamma + 1 = {g + 1} entries")
    _need(temperature, torch.float32, (B,), "temperature")
    _need(lnZ_target, torch.float64, (B, g + 1), "lnZ_target")
    _need(lnZ_draft, torch.float64, (B, K, g), "lnZ_draft")
    dev = target.device
    ftot = int(sum(int(f) for f in fanout))
    cand = torch.empty((B, K, ftot), dtype=torch.int32, device=dev)
    w = torch.empty((B, K, ftot), dtype=torch.float32, device=dev) if want_weights else None
    st = lib.specverify_residual_topf(
        target.data_ptr(), draft.data_ptr(), _dtype_code(target), B, K, g, V, target.stride(0),
        target.stride(1), draft.stride(0), draft.stride(1), draft.stride(2), temperature.data_ptr(),
        lnZ_target.data_ptr(), lnZ_draft.data_ptr(), _fanout_array(fanout), cand.data_ptr(),
        _ptr(w), _stream(dev))
    _check(st, "specverify_residual_topf")
    return cand, w


def specverify_cache_lookup(cand: torch.Tensor, fanout, accept_len: torch.Tensor,
                            out_token: torch.Tensor) -> torch.Tensor:
    """slot [B, K] int32: index of out_token among the candidates of outcome accept_len, or -1."""
    lib = load_library()
    B, K, ftot = cand.shape
    g = len(fanout) - 1
    if ftot != sum(int(f) for f in fanout):
        raise SpecVerifyError("cand's last axis must equal sum(fanout)")
    _need(cand, torch.int32, (B, K, ftot), "cand")
    _need(accept_len, torch.int32, (B, K), "accept_len")
    _need(out_token, torch.int32, (B, K), "out_token")
    slot = torch.empty((B, K), dtype=torch.int32, device=cand.device)
    st = lib.specverify_cache_lookup(cand.data_ptr(), _fanout_array(fanout), B, K, g,
                                     accept_len.data_ptr(), out_token.data_ptr(), slot.data_ptr(),
                                     _stream(cand.device))
    _check(st, "specverify_cache_lookup")
    return slot


def specverify_branch_prune(logq: torch.Tensor, log_tau: float, keep: int):
    """(keep_mask [B, K] int32, prefix_len [B, K] int32, conf [B, K, gamma] float64) from the
    draft log-probabilities at the drafted tokens, logq [B, K, gamma] float32."""
    B, K, g = logq.shape
    _need(logq, torch.float32, (B, K, g), "logq")
    dev = logq.device
    mask = torch.empty((B, K), dtype=torch.int32, device=dev)
    plen = torch.empty((B, K), dtype=torch.int32, device=dev)
    conf = torch.empty((B, K, g), dtype=torch.float64, device=dev)
    st = load_library().specverify_branch_prune(logq.data_ptr(), B, K, g, float(log_tau), keep,
                                                mask.data_ptr(), plen.data_ptr(), conf.data_ptr(),
                                                _stream(dev))
    _check(st, "specverify_branch_prune")
    return mask, plen, conf


BANDIT_UCB1 = 0
BANDIT_THOMPSON = 1


class Bandit:
    """Draft selector between steps (host only): UCB1 or Thompson sampling over `arms`
    draft models, rewarded with the accepted fraction of each step's draft tokens."""

    def __init__(self, arms: int, policy: int = BANDIT_UCB1, seed: int = 0, c: float = 2.0):
        lib = load_library()
        n = int(lib.specverify_bandit_state_size(arms))
        if n == 0:
            raise SpecVerifyError(f"arms must be in [1, 256], got {arms}")
        self._lib = lib
        self._state = ctypes.create_string_buffer(n)
        _check(lib.specverify_bandit_init(self._state, n, arms, policy, seed & (2 ** 64 - 1),
                                          float(c)), "specverify_bandit_init")
        self.arms = arms

    def select(self) -> int:
        arm = ctypes.c_int32()
        _check(self._lib.specverify_bandit_select(self._state, ctypes.byref(arm)),
               "specverify_bandit_select")
        return arm.value

    def update(self, arm: int, reward: float) -> None:
        _check(self._lib.specverify_bandit_update(self._state, arm, float(reward)),
               "specverify_bandit_update")

    def stats(self, arm: int) -> tuple:
        pulls, total = ctypes.c_int64(), ctypes.c_double()
        _check(self._lib.specverify_bandit_stats(self._state, arm, ctypes.byref(pulls),
                                                 ctypes.byref(total)), "specverify_bandit_stats")
        return pulls.value, total.value


def step_reward(accept_len, gamma: int) -> float:
    """Accepted fraction of a step's draft tokens from its accept lengths (any host array
    or tensor; a device tensor is copied to the host)."""
    if isinstance(accept_len, torch.Tensor):
        accept_len = accept_len.detach().to("cpu")
    arr = torch.as_tensor(accept_len, dtype=torch.int32).contiguous().reshape(-1)
    out = ctypes.c_double()
    _check(load_library().specverify_step_reward(arr.data_ptr(), arr.numel(), gamma,
                                                  ctypes.byref(out)), "specverify_step_reward")
    return out.value


def time_next_stream_kernel(before: torch.cuda.Event | None, after: torch.cuda.Event | None) -> None:
    """The next step or normalise call on this thread records `before` / `after` around its
    streaming kernel (timing events; each must have been recorded once so that it exists)."""
    b = None if before is None else before.cuda_event
    a = None if after is None else after.cuda_event
    if (before is not None and not b) or (after is not None and not a):
        raise SpecVerifyError("record the events once before handing them to the library")
    _check(load_library().specverify_time_next_stream_kernel(b, a),
           "specverify_time_next_stream_kernel")


def check_count(reset: bool = False) -> int | None:
    """Failed device-side index checks so far on the current device, or None when the
    loaded library was built without them (the product build)."""
    n = ctypes.c_uint32()
    st = load_library().specverify_check_count(ctypes.byref(n), int(reset))
    if st == SV_ENOCHECKS:
        return None
    _check(st, "specverify_check_count")
    return int(n.value)


def version() -> int:
    return int(load_library().specverify_version())
