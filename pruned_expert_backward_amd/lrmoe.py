"""Thin Python binding of liblrmoe (C ABI in include/lrmoe.h).

Argument marshalling only: torch tensors supply device memory and the
current HIP stream; every step of the path runs in the library's HIP
kernels.  There is no fallback -- without the built library on a GPU every
call raises.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional, Sequence

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "liblrmoe.so")

F32, BF16 = 0, 1
DW_EXACT, DW_BF16, DW_F16 = 0, 1, 2
SCORE_LRM, SCORE_GRAD_SQNORM, SCORE_GRAD_L1 = 0, 1, 2
QUOTA_RATIO, QUOTA_BUDGET = 0, 1
MAX_EXPERTS = 256
ABI_VERSION = 4

STATUS = {0: "LRMOE_OK", 1: "LRMOE_ERR_NULL", 2: "LRMOE_ERR_INVALID", 3: "LRMOE_ERR_SHAPE",
          4: "LRMOE_ERR_ALIGN", 5: "LRMOE_ERR_DTYPE", 6: "LRMOE_ERR_WORKSPACE",
          7: "LRMOE_ERR_HIP", 8: "LRMOE_ERR_SCRATCH"}

EXPORTS = ["lrmoe_abi_version", "lrmoe_status_string", "lrmoe_plan_quota",
           "lrmoe_workspace_size", "lrmoe_score_select_compact", "lrmoe_select_compact",
           "lrmoe_gather_compact", "lrmoe_grouped_backward", "lrmoe_score_select_compact_timed",
           "lrmoe_select_compact_timed", "lrmoe_grouped_backward_timed", "lrmoe_score_select",
           "lrmoe_mask_alpha", "lrmoe_plan_quota_device", "lrmoe_grouped_backward_glu",
           "lrmoe_grouped_backward_glu_timed", "lrmoe_pruned_backward",
           "lrmoe_pruned_backward_timed", "lrmoe_gather_backward",
           "lrmoe_gather_backward_timed", "lrmoe_grouped_backward_gate_up",
           "lrmoe_grouped_backward_gate_up_timed", "lrmoe_score_select_compact_noalloc"]
TIMING_SLOTS = 8


class LrmoeError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} -> {STATUS.get(status, status)}: {msg}")
        self.status = status


class Problem(C.Structure):
    _fields_ = [("E", C.c_int32), ("dtype", C.c_int32), ("P", C.c_int64), ("T", C.c_int64),
                ("d_out", C.c_int32), ("d_in", C.c_int32),
                ("counts", C.POINTER(C.c_int64)), ("quotas", C.POINTER(C.c_int64)),
                ("dw_mode", C.c_int32), ("score_mode", C.c_int32), ("T_phi", C.c_int64)]


class Timing(C.Structure):
    _fields_ = [("before", C.c_void_p * TIMING_SLOTS), ("after", C.c_void_p * TIMING_SLOTS)]


class QuotaPolicy(C.Structure):
    _fields_ = [("mode", C.c_int32), ("num", C.c_int64), ("den", C.c_int64),
                ("budget_pairs", C.c_int64)]


_lib_handle = None
_P = C.c_void_p


def lib() -> C.CDLL:
    """Load liblrmoe.so once; raise if it has not been built."""
    global _lib_handle
    if _lib_handle is not None:
        return _lib_handle
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} not found: build it with "
                           "`python -m pruned_expert_backward_amd.build`")
    L = C.CDLL(LIB_PATH)
    L.lrmoe_abi_version.restype = C.c_int32
    L.lrmoe_status_string.restype = C.c_char_p
    L.lrmoe_status_string.argtypes = [C.c_int]
    L.lrmoe_plan_quota.restype = C.c_int
    L.lrmoe_plan_quota.argtypes = [C.c_int32, C.POINTER(C.c_int64), C.POINTER(QuotaPolicy),
                                   C.POINTER(C.c_int64)]
    L.lrmoe_workspace_size.restype = C.c_int
    L.lrmoe_workspace_size.argtypes = [C.POINTER(Problem), C.POINTER(C.c_size_t)]
    L.lrmoe_score_select_compact.restype = C.c_int
    L.lrmoe_score_select_compact.argtypes = [C.POINTER(Problem)] + [_P] * 13 + [C.c_size_t, _P]
    L.lrmoe_select_compact.restype = C.c_int
    L.lrmoe_select_compact.argtypes = [C.POINTER(Problem)] + [_P] * 13 + [C.c_size_t, _P]
    L.lrmoe_gather_compact.restype = C.c_int
    L.lrmoe_gather_compact.argtypes = [C.POINTER(Problem)] + [_P] * 12
    L.lrmoe_grouped_backward.restype = C.c_int
    L.lrmoe_grouped_backward.argtypes = [C.POINTER(Problem)] + [_P] * 8 + [C.c_size_t, _P]
    L.lrmoe_score_select_compact_timed.restype = C.c_int
    L.lrmoe_score_select_compact_timed.argtypes = ([C.POINTER(Problem)] + [_P] * 13 +
                                                   [C.c_size_t, _P, C.POINTER(Timing)])
    L.lrmoe_select_compact_timed.restype = C.c_int
    L.lrmoe_select_compact_timed.argtypes = ([C.POINTER(Problem)] + [_P] * 13 +
                                             [C.c_size_t, _P, C.POINTER(Timing)])
    L.lrmoe_score_select.restype = C.c_int
    L.lrmoe_score_select.argtypes = [C.POINTER(Problem)] + [_P] * 9 + [C.c_size_t, _P]
    L.lrmoe_plan_quota_device.restype = C.c_int
    L.lrmoe_plan_quota_device.argtypes = [C.c_int32, _P, C.c_int64, C.POINTER(QuotaPolicy),
                                          _P, _P, _P, _P, _P]
    L.lrmoe_mask_alpha.restype = C.c_int
    L.lrmoe_mask_alpha.argtypes = [C.c_int64, _P, _P, _P, _P, _P]
    L.lrmoe_grouped_backward_timed.restype = C.c_int
    L.lrmoe_grouped_backward_timed.argtypes = ([C.POINTER(Problem)] + [_P] * 8 +
                                               [C.c_size_t, _P, C.POINTER(Timing)])
    L.lrmoe_pruned_backward.restype = C.c_int
    L.lrmoe_pruned_backward.argtypes = [C.POINTER(Problem)] + [_P] * 15 + [C.c_size_t, _P]
    L.lrmoe_pruned_backward_timed.restype = C.c_int
    L.lrmoe_pruned_backward_timed.argtypes = ([C.POINTER(Problem)] + [_P] * 15 +
                                              [C.c_size_t, _P, C.POINTER(Timing)])
    L.lrmoe_gather_backward.restype = C.c_int
    L.lrmoe_gather_backward.argtypes = [C.POINTER(Problem)] + [_P] * 14 + [C.c_size_t, _P]
    L.lrmoe_gather_backward_timed.restype = C.c_int
    L.lrmoe_gather_backward_timed.argtypes = ([C.POINTER(Problem)] + [_P] * 14 +
                                              [C.c_size_t, _P, C.POINTER(Timing)])
    L.lrmoe_grouped_backward_glu.restype = C.c_int
    L.lrmoe_grouped_backward_glu.argtypes = [C.POINTER(Problem)] + [_P] * 10 + [C.c_size_t, _P]
    L.lrmoe_grouped_backward_glu_timed.restype = C.c_int
    L.lrmoe_grouped_backward_glu_timed.argtypes = ([C.POINTER(Problem)] + [_P] * 10 +
                                                   [C.c_size_t, _P, C.POINTER(Timing)])
    L.lrmoe_grouped_backward_gate_up.restype = C.c_int
    L.lrmoe_grouped_backward_gate_up.argtypes = [C.POINTER(Problem)] + [_P] * 8 + [C.c_size_t, _P]
    L.lrmoe_grouped_backward_gate_up_timed.restype = C.c_int
    L.lrmoe_grouped_backward_gate_up_timed.argtypes = ([C.POINTER(Problem)] + [_P] * 8 +
                                                       [C.c_size_t, _P, C.POINTER(Timing)])
    L.lrmoe_score_select_compact_noalloc.restype = C.c_int
    L.lrmoe_score_select_compact_noalloc.argtypes = [C.POINTER(Problem)] + [_P] * 13
    if L.lrmoe_abi_version() != ABI_VERSION:
        raise RuntimeError("liblrmoe ABI version mismatch; rebuild the library")
    _lib_handle = L
    return L


def check(fn: str, status: int) -> None:
    if status != 0:
        raise LrmoeError(fn, status, lib().lrmoe_status_string(status).decode())


# ------------------------------------------------------------------ host side

def _i64_array(vals: Sequence[int]):
    arr = (C.c_int64 * len(vals))(*[int(v) for v in vals])
    return arr


def _policy(policy: tuple) -> QuotaPolicy:
    if policy[0] == "ratio":
        return QuotaPolicy(QUOTA_RATIO, int(policy[1]), int(policy[2]), 0)
    if policy[0] == "budget":
        return QuotaPolicy(QUOTA_BUDGET, 0, 1, int(policy[1]))
    raise ValueError(policy)


def plan_quota(counts: Sequence[int], policy: tuple) -> list:
    """Quotas per expert: policy ("ratio", num, den) or ("budget", pairs)."""
    E = len(counts)
    cnt = _i64_array(counts)
    out = (C.c_int64 * max(E, 1))()
    pol = _policy(policy)
    check("lrmoe_plan_quota", lib().lrmoe_plan_quota(E, cnt, C.byref(pol), out))
    return [int(out[e]) for e in range(E)]


def plan_quota_device(E: int, expert_ids, policy: tuple) -> dict:
    """Counts, quotas and quota offsets on the device from the routing (the
    local expert index of every routed pair); nothing visits the host."""
    dev = expert_ids.device
    out = dict(counts=_empty((E,), torch.int64, dev), quotas=_empty((E,), torch.int64, dev),
               seg_offsets=_empty((E + 1,), torch.int64, dev),
               invalid=_empty((1,), torch.int64, dev))
    pol = _policy(policy)
    st = lib().lrmoe_plan_quota_device(E, _ptr(expert_ids), expert_ids.numel(), C.byref(pol),
                                       _ptr(out["counts"]), _ptr(out["quotas"]),
                                       _ptr(out["seg_offsets"]), _ptr(out["invalid"]), _stream())
    check("lrmoe_plan_quota_device", st)
    return out


class Plan:
    """Host description of one call: counts, quotas, sizes, storage type."""

    def __init__(self, counts, quotas, d_out: int, d_in: int, dtype: int, T: Optional[int] = None,
                 dw_mode: int = DW_EXACT, score_mode: int = SCORE_LRM):
        self.counts = [int(c) for c in counts]
        self.quotas = [int(q) for q in quotas]
        self.E = len(self.counts)
        self.P = sum(self.counts)
        self.M = sum(self.quotas)
        self.T = self.P if T is None else int(T)
        self.d_out, self.d_in, self.dtype, self.dw_mode = int(d_out), int(d_in), int(dtype), int(dw_mode)
        self._cnt = _i64_array(self.counts)
        self._q = _i64_array(self.quotas)
        self.struct = Problem(self.E, self.dtype, self.P, self.T, self.d_out, self.d_in,
                              C.cast(self._cnt, C.POINTER(C.c_int64)),
                              C.cast(self._q, C.POINTER(C.c_int64)), self.dw_mode,
                              int(score_mode), 0)

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == BF16 else torch.float32

    def workspace_bytes(self) -> int:
        n = C.c_size_t(0)
        check("lrmoe_workspace_size", lib().lrmoe_workspace_size(C.byref(self.struct), C.byref(n)))
        return int(n.value)


def storage_dtype(t: torch.dtype) -> int:
    if t == torch.bfloat16:
        return BF16
    if t == torch.float32:
        return F32
    raise TypeError(f"unsupported storage dtype {t}")


# ------------------------------------------------------------------ device side

def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("liblrmoe takes device tensors")
    if not t.is_contiguous():
        raise ValueError("liblrmoe takes contiguous tensors")
    return t.data_ptr() if t.numel() > 0 else None


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _empty(shape, dtype, device):
    return torch.empty(shape, dtype=dtype, device=device)


def alloc_select_outputs(plan: Plan, device, zero_target: bool = True) -> dict:
    """Output buffers of score_select_compact (caller-owned memory)."""
    dt = plan.torch_dtype
    out = dict(scores=_empty((plan.P,), torch.float32, device),
               keep=_empty((plan.P,), torch.uint8, device),
               seg_offsets=_empty((plan.E + 1,), torch.int32, device),
               perm=_empty((plan.M,), torch.int32, device),
               g_c=_empty((plan.M, plan.d_out), dt, device),
               phi_c=_empty((plan.M, plan.d_in), dt, device),
               alpha_c=_empty((plan.M,), torch.float32, device))
    if zero_target:
        out["dphi"] = _empty((plan.P, plan.d_in), torch.float32, device)
    return out


def workspace(plan: Plan, device) -> torch.Tensor:
    return torch.empty((max(plan.workspace_bytes(), 16),), dtype=torch.uint8, device=device)


def score_select_compact(plan: Plan, alpha, g, phi, g_row_index=None, out=None, ws=None,
                         scores=None, timing: Optional["KernelTimer"] = None) -> dict:
    """LRM score -> per-expert top-quota select -> compaction.  With
    `scores` given, the LRM scoring is skipped and those scores are used.
    `timing` (a KernelTimer) records events around each kernel."""
    dev = phi.device
    if out is None:
        out = alloc_select_outputs(plan, dev)
    if ws is None:
        ws = workspace(plan, dev)
    L = lib()
    common = (_ptr(g_row_index), _ptr(alpha), _ptr(g), _ptr(phi))
    tail = (_ptr(out["keep"]), _ptr(out["seg_offsets"]), _ptr(out["perm"]), _ptr(out["g_c"]),
            _ptr(out["phi_c"]), _ptr(out["alpha_c"]), _ptr(out.get("dphi")), _ptr(ws),
            ws.numel(), _stream())
    if scores is None and timing is not None:
        st = L.lrmoe_score_select_compact_timed(C.byref(plan.struct), *common, _ptr(out["scores"]),
                                                *tail, C.byref(timing.next_slots()))
        check("lrmoe_score_select_compact_timed", st)
    elif scores is None:
        st = L.lrmoe_score_select_compact(C.byref(plan.struct), *common, _ptr(out["scores"]), *tail)
        check("lrmoe_score_select_compact", st)
    elif timing is not None:
        st = L.lrmoe_select_compact_timed(C.byref(plan.struct), _ptr(scores), *common, *tail,
                                          C.byref(timing.next_slots()))
        check("lrmoe_select_compact_timed", st)
    else:
        st = L.lrmoe_select_compact(C.byref(plan.struct), _ptr(scores), *common, *tail)
        check("lrmoe_select_compact", st)
    return out


def score_select_compact_noalloc(plan: Plan, alpha, g, phi, g_row_index=None, out=None) -> dict:
    """score_select_compact through the entry point that takes no workspace
    (its selection scratch is the library's static device buffer)."""
    if out is None:
        out = alloc_select_outputs(plan, phi.device)
    st = lib().lrmoe_score_select_compact_noalloc(
        C.byref(plan.struct), _ptr(g_row_index), _ptr(alpha), _ptr(g), _ptr(phi),
        _ptr(out["scores"]), _ptr(out["keep"]), _ptr(out["seg_offsets"]), _ptr(out["perm"]),
        _ptr(out["g_c"]), _ptr(out["phi_c"]), _ptr(out["alpha_c"]), _ptr(out.get("dphi")),
        _stream())
    check("lrmoe_score_select_compact_noalloc", st)
    return out


def score_select(plan: Plan, alpha, g, phi, g_row_index=None, out=None, ws=None) -> dict:
    """Scores and keep flags (with perm and seg_offsets) without compaction."""
    dev = phi.device
    if out is None:
        out = dict(scores=_empty((plan.P,), torch.float32, dev),
                   keep=_empty((plan.P,), torch.uint8, dev),
                   seg_offsets=_empty((plan.E + 1,), torch.int32, dev),
                   perm=_empty((plan.M,), torch.int32, dev))
    if ws is None:
        ws = workspace(plan, dev)
    st = lib().lrmoe_score_select(C.byref(plan.struct), _ptr(g_row_index), _ptr(alpha), _ptr(g),
                                  _ptr(phi), _ptr(out["scores"]), _ptr(out["keep"]),
                                  _ptr(out["seg_offsets"]), _ptr(out["perm"]), _ptr(ws),
                                  ws.numel(), _stream())
    check("lrmoe_score_select", st)
    return out


def mask_alpha(keep, alpha, alpha_masked=None, perm_identity=None, identity: bool = True):
    """alpha where kept, 0 where dropped (and the identity permutation)."""
    P = alpha.numel()
    if alpha_masked is None:
        alpha_masked = _empty((P,), torch.float32, alpha.device)
    if identity and perm_identity is None:
        perm_identity = _empty((P,), torch.int32, alpha.device)
    st = lib().lrmoe_mask_alpha(P, _ptr(keep), _ptr(alpha), _ptr(alpha_masked),
                                _ptr(perm_identity), _stream())
    check("lrmoe_mask_alpha", st)
    return alpha_masked, perm_identity


def masked_dense_backward(plan: Plan, alpha, g, phi, W, out=None, ws=None, dense_ws=None,
                          timing: Optional["KernelTimer"] = None) -> dict:
    """Zero-masked dense alternative to compaction: select the same keep set,
    set alpha of dropped pairs to 0, and run the grouped GEMMs over every
    routed pair of the uncompacted g (one row per pair) and phi.  Same dW and
    dphi as pruned_backward; for timing the two paths against each other."""
    if plan.T != plan.P:
        raise ValueError("the dense path needs one g row per pair (T == P)")
    dense = Plan(plan.counts, plan.counts, plan.d_out, plan.d_in, plan.dtype, dw_mode=plan.dw_mode)
    dev = phi.device
    if out is None:
        out = {}
    sel = score_select(plan, alpha, g, phi, out=out.get("sel"), ws=ws)
    am, pid = mask_alpha(sel["keep"], alpha, out.get("alpha_masked"), out.get("perm_identity"))
    if "dphi" not in out:
        out["dphi"] = _empty((plan.P, plan.d_in), torch.float32, dev)
    out.update(sel=sel, alpha_masked=am, perm_identity=pid, keep=sel["keep"])
    out["dW"] = grouped_backward(dense, pid, am, g, phi, W, dW=out.get("dW"), dphi=out["dphi"],
                                 ws=dense_ws if dense_ws is not None else workspace(dense, dev),
                                 timing=timing)
    return out


def gather_compact(plan: Plan, perm, keep, alpha, g, phi, g_row_index=None, phi_row_index=None,
                   out=None, zero_target: bool = True) -> dict:
    """Kept rows of a projection that inherits a keep set; g=None gathers
    the phi rows and alpha only."""
    dev = phi.device
    dt = plan.torch_dtype
    if out is None:
        out = dict(g_c=_empty((plan.M, plan.d_out), dt, dev) if g is not None else None,
                   phi_c=_empty((plan.M, plan.d_in), dt, dev),
                   alpha_c=_empty((plan.M,), torch.float32, dev))
        if zero_target:
            out["dphi"] = _empty((plan.P, plan.d_in), torch.float32, dev)
    # rows of phi that phi_row_index addresses (the library bounds the index by them)
    plan.struct.T_phi = phi.shape[0] if phi_row_index is not None else 0
    st = lib().lrmoe_gather_compact(C.byref(plan.struct), _ptr(perm), _ptr(keep),
                                    _ptr(g_row_index), _ptr(phi_row_index), _ptr(alpha), _ptr(g),
                                    _ptr(phi), _ptr(out.get("g_c")), _ptr(out["phi_c"]),
                                    _ptr(out["alpha_c"]), _ptr(out.get("dphi")), _stream())
    check("lrmoe_gather_compact", st)
    return out


def grouped_backward(plan: Plan, perm, alpha_c, g_c, phi_c, W, dW=None, dphi=None,
                     ws=None, timing: Optional["KernelTimer"] = None) -> torch.Tensor:
    """dW [E, d_out, d_in] (returned) and the kept rows of dphi (in place)."""
    dev = W.device
    if dW is None:
        dW = _empty((plan.E, plan.d_out, plan.d_in), torch.float32, dev)
    if ws is None:
        ws = workspace(plan, dev)
    args = (C.byref(plan.struct), _ptr(perm), _ptr(alpha_c), _ptr(g_c), _ptr(phi_c), _ptr(W),
            _ptr(dW), _ptr(dphi), _ptr(ws), ws.numel(), _stream())
    if timing is not None:
        check("lrmoe_grouped_backward_timed",
              lib().lrmoe_grouped_backward_timed(*args, C.byref(timing.next_slots())))
    else:
        check("lrmoe_grouped_backward", lib().lrmoe_grouped_backward(*args))
    return dW


def gather_backward(plan: Plan, perm, keep, alpha, g, phi, W, g_row_index=None,
                    phi_row_index=None, out=None, ws=None,
                    timing: Optional["KernelTimer"] = None) -> dict:
    """gather_compact + grouped_backward for a projection on an inherited keep
    set, in one library call (lrmoe_gather_backward): returns g_c, phi_c,
    alpha_c, dW and dphi (dropped rows zero)."""
    dev = phi.device
    dt = plan.torch_dtype
    if out is None:
        out = {}
    for k, shape, t in (("g_c", (plan.M, plan.d_out), dt), ("phi_c", (plan.M, plan.d_in), dt),
                        ("alpha_c", (plan.M,), torch.float32),
                        ("dW", (plan.E, plan.d_out, plan.d_in), torch.float32),
                        ("dphi", (plan.P, plan.d_in), torch.float32)):
        if out.get(k) is None:
            out[k] = _empty(shape, t, dev)
    if ws is None:
        ws = workspace(plan, dev)
    plan.struct.T_phi = phi.shape[0] if phi_row_index is not None else 0
    args = (C.byref(plan.struct), _ptr(perm), _ptr(keep), _ptr(g_row_index), _ptr(phi_row_index),
            _ptr(alpha), _ptr(g), _ptr(phi), _ptr(W), _ptr(out["g_c"]), _ptr(out["phi_c"]),
            _ptr(out["alpha_c"]), _ptr(out["dW"]), _ptr(out["dphi"]), _ptr(ws), ws.numel(),
            _stream())
    if timing is not None:
        check("lrmoe_gather_backward_timed",
              lib().lrmoe_gather_backward_timed(*args, C.byref(timing.next_slots())))
    else:
        check("lrmoe_gather_backward", lib().lrmoe_gather_backward(*args))
    return out


# The one-call entry points (lrmoe_pruned_backward, lrmoe_gather_backward)
# clear the dropped pairs' dphi rows inside the grouped GEMM launch when they
# hold at least this many bytes, else in the gather (the library's rule,
# restated for accounting).
ZERO_IN_GEMM_BYTES = 512 << 20


def zero_fill_in_gemm(plan: Plan) -> bool:
    """Where the one-call entry points clear the dropped dphi rows: True for
    the grouped GEMM launch, False for the gather."""
    return (plan.P - plan.M) * plan.d_in * 4 >= ZERO_IN_GEMM_BYTES


def glu_grad_dtype(plan: Plan) -> torch.dtype:
    """Storage of the SiLU-GLU chain's hand-off gradient: float32, or bf16 in
    the single-rounding dW mode."""
    return torch.bfloat16 if plan.dw_mode == DW_BF16 else torch.float32


def grouped_backward_glu(plan: Plan, perm, alpha_c, g_c, phi_c, W, act_a, act_b, dW=None,
                         dgu_c=None, ws=None, timing: Optional["KernelTimer"] = None):
    """Down projection's dW and, through the SiLU-GLU backward, the gate/up
    output gradient of the kept pairs, compacted: returns (dW, dgu_c) with
    dgu_c [M, 2 d_in] (gate half first, before alpha) in glu_grad_dtype."""
    dev = W.device
    if dW is None:
        dW = _empty((plan.E, plan.d_out, plan.d_in), torch.float32, dev)
    if dgu_c is None:
        dgu_c = _empty((plan.M, 2 * plan.d_in), glu_grad_dtype(plan), dev)
    if ws is None:
        ws = workspace(plan, dev)
    args = (C.byref(plan.struct), _ptr(perm), _ptr(alpha_c), _ptr(g_c), _ptr(phi_c), _ptr(W),
            _ptr(dW), _ptr(act_a), _ptr(act_b), _ptr(dgu_c), _ptr(ws), ws.numel(), _stream())
    if timing is not None:
        check("lrmoe_grouped_backward_glu_timed",
              lib().lrmoe_grouped_backward_glu_timed(*args, C.byref(timing.next_slots())))
    else:
        check("lrmoe_grouped_backward_glu", lib().lrmoe_grouped_backward_glu(*args))
    return dW, dgu_c


def grouped_backward_gate_up(plan: Plan, perm, alpha_c, dgu_c, x_c, W, dW=None, dx=None,
                             ws=None, timing: Optional["KernelTimer"] = None) -> torch.Tensor:
    """The gate/up projection's backward on the float32 output gradient of
    grouped_backward_glu: dW [E, d_out, d_in] (returned) and the kept rows of
    dx (in place)."""
    dev = W.device
    if dW is None:
        dW = _empty((plan.E, plan.d_out, plan.d_in), torch.float32, dev)
    if ws is None:
        ws = workspace(plan, dev)
    args = (C.byref(plan.struct), _ptr(perm), _ptr(alpha_c), _ptr(dgu_c), _ptr(x_c), _ptr(W),
            _ptr(dW), _ptr(dx), _ptr(ws), ws.numel(), _stream())
    if timing is not None:
        check("lrmoe_grouped_backward_gate_up_timed",
              lib().lrmoe_grouped_backward_gate_up_timed(*args, C.byref(timing.next_slots())))
    else:
        check("lrmoe_grouped_backward_gate_up", lib().lrmoe_grouped_backward_gate_up(*args))
    return dW


def glu_chain_backward(plan: Plan, plan2: Plan, alpha, g, phi, W, act_a, act_b, x, W2,
                       g_row_index=None, x_row_index=None, out=None, ws=None) -> dict:
    """The expert MLP's backward on one keep set: score, select, compact
    (down projection), dW, the SiLU-GLU backward into the compacted gate/up
    output gradient, the gather of the gate/up inputs x, and that
    projection's dW2 and dx (dx rows of dropped pairs zeroed).  plan2
    describes the gate/up projection (d_out = 2 d_in of plan, d_in =
    d_model, the same counts and quotas)."""
    dev = phi.device
    if out is None:
        out = alloc_select_outputs(plan, dev, zero_target=False)
    if ws is None:   # one buffer for both projections
        ws = torch.empty((max(plan.workspace_bytes(), plan2.workspace_bytes(), 16),),
                         dtype=torch.uint8, device=dev)
    out = score_select_compact(plan, alpha, g, phi, g_row_index=g_row_index, out=out, ws=ws)
    out["dW"], out["dgu_c"] = grouped_backward_glu(plan, out["perm"], out["alpha_c"], out["g_c"],
                                                   out["phi_c"], W, act_a, act_b, ws=ws)
    c2 = gather_compact(plan2, out["perm"], out["keep"], alpha, None, x,
                        phi_row_index=x_row_index)
    out["x_c"] = c2["phi_c"]
    out["dx"] = c2["dphi"]
    if out["dgu_c"].dtype == torch.float32:   # unrounded hand-off
        out["dW2"] = grouped_backward_gate_up(plan2, out["perm"], c2["alpha_c"], out["dgu_c"],
                                              c2["phi_c"], W2, dx=c2["dphi"], ws=ws)
    else:                                     # single-rounding mode: bf16 hand-off
        out["dW2"] = grouped_backward(plan2, out["perm"], c2["alpha_c"], out["dgu_c"],
                                      c2["phi_c"], W2, dphi=c2["dphi"], ws=ws)
    return out


class KernelTimer:
    """HIP events recorded by the library around each kernel of a call.

    Create one per (call site, number of calls); each call takes the next
    set of slots.  After synchronising, mean_us(slot) is the mean duration of
    that kernel over the calls that launched it."""

    def __init__(self, calls: int, slots=None):
        """slots: the timing slots to record (default all); the library skips
        the others, so they cost nothing."""
        self._hip = C.CDLL("libamdhip64.so")
        self._hip.hipEventCreate.argtypes = [C.POINTER(C.c_void_p)]
        self._hip.hipEventElapsedTime.argtypes = [C.POINTER(C.c_float), C.c_void_p, C.c_void_p]
        self._hip.hipEventQuery.argtypes = [C.c_void_p]
        self._hip.hipEventDestroy.argtypes = [C.c_void_p]
        self.timings = []
        for _ in range(calls):
            t = Timing()
            for k in range(TIMING_SLOTS):
                if slots is not None and k not in slots:
                    continue
                for arr in (t.before, t.after):
                    ev = C.c_void_p()
                    if self._hip.hipEventCreate(C.byref(ev)) != 0:
                        raise RuntimeError("hipEventCreate failed")
                    arr[k] = ev
            self.timings.append(t)
        self._next = 0

    def next_slots(self) -> Timing:
        t = self.timings[self._next]
        self._next += 1
        return t

    def durations_us(self, slot: int) -> list:
        out = []
        for t in self.timings[:self._next]:
            if not t.before[slot]:
                continue
            ms = C.c_float()
            # hipEventElapsedTime fails for events that were never recorded
            # (a kernel the call did not launch); that failure also stays in
            # HIP's last-error slot, where the next launch check of another
            # caller (torch) would report it, so it is cleared here
            if self._hip.hipEventElapsedTime(C.byref(ms), t.before[slot], t.after[slot]) == 0:
                out.append(ms.value * 1e3)
            else:
                self._hip.hipGetLastError()
        return out

    def mean_us(self, slot: int) -> Optional[float]:
        d = self.durations_us(slot)
        return sum(d) / len(d) if d else None

    def close(self):
        for t in self.timings:
            for k in range(TIMING_SLOTS):
                if t.before[k]:
                    self._hip.hipEventDestroy(t.before[k])
                if t.after[k]:
                    self._hip.hipEventDestroy(t.after[k])
        self.timings = []


def pruned_backward(plan: Plan, alpha, g, phi, W, g_row_index=None, out=None, ws=None,
                    timing: Optional["KernelTimer"] = None) -> dict:
    """The whole path in one library call (lrmoe_pruned_backward): score,
    select, compact, dW and dphi.  `out` holds the buffers of
    alloc_select_outputs plus "dW"; missing ones are allocated."""
    dev = phi.device
    if out is None:
        out = alloc_select_outputs(plan, dev)
    if out.get("dW") is None:
        out["dW"] = _empty((plan.E, plan.d_out, plan.d_in), torch.float32, dev)
    if ws is None:
        ws = workspace(plan, dev)
    args = (C.byref(plan.struct), _ptr(g_row_index), _ptr(alpha), _ptr(g), _ptr(phi), _ptr(W),
            _ptr(out["scores"]), _ptr(out["keep"]), _ptr(out["seg_offsets"]), _ptr(out["perm"]),
            _ptr(out["g_c"]), _ptr(out["phi_c"]), _ptr(out["alpha_c"]), _ptr(out["dW"]),
            _ptr(out.get("dphi")), _ptr(ws), ws.numel(), _stream())
    if timing is not None:
        check("lrmoe_pruned_backward_timed",
              lib().lrmoe_pruned_backward_timed(*args, C.byref(timing.next_slots())))
    else:
        check("lrmoe_pruned_backward", lib().lrmoe_pruned_backward(*args))
    return out
