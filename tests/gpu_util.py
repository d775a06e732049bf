"""Helpers for the GPU parity tests: run the HIP path through the C ABI on a
workload and compare it with the CPU oracle.

Comparison rules:
  * keep sets: equal to the oracle's except for pairs whose oracle score is
    within 1e-5 (relative) of that expert's threshold tau_e; every expert
    keeps exactly q_e pairs;
  * offsets, permutation, compacted rows: bit-exact (against the oracle's
    own outputs when the keep sets agree, else against the oracle's
    compaction of the GPU keep set -- "bit-exact given the keep set");
  * dW and dphi: max |err| <= 2e-3 * max |ref| per output tensor.
"""
import numpy as np
import torch

from oracle import lrmoe_oracle as O
from pruned_expert_backward_amd import lrmoe

TOL = 2e-3
BAND = 1e-5
DEV = torch.device("cuda:0")


def dev(a):
    if a is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(a))
    if a.dtype == np.uint16:
        t = t.view(torch.bfloat16)
    return t.to(DEV)


def host_bits(t):
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def dtype_code(p):
    return lrmoe.BF16 if p.dtype == "bf16" else lrmoe.F32


def run_gpu(p, quotas, dw_mode=lrmoe.DW_EXACT, scores=None, score_mode=lrmoe.SCORE_LRM):
    plan = lrmoe.Plan(p.counts, quotas, p.d_out, p.d_in, dtype_code(p), T=p.T, dw_mode=dw_mode,
                      score_mode=score_mode)
    t = dict(alpha=dev(p.alpha), g=dev(p.g), phi=dev(p.phi), W=dev(p.W),
             row=dev(p.row_index))
    sc = dev(scores) if scores is not None else None
    out = lrmoe.score_select_compact(plan, t["alpha"], t["g"], t["phi"], g_row_index=t["row"],
                                     scores=sc)
    out["dW"] = lrmoe.grouped_backward(plan, out["perm"], out["alpha_c"], out["g_c"],
                                       out["phi_c"], t["W"], dphi=out["dphi"])
    torch.cuda.synchronize()
    return plan, out, t


def check_keep(ref_scores, counts, quotas, keep_gpu, keep_ref, taus):
    offs = np.concatenate([[0], np.cumsum(counts)])
    exempt = np.zeros_like(keep_ref)
    for e in range(len(counts)):
        lo, hi = offs[e], offs[e + 1]
        assert int(keep_gpu[lo:hi].sum()) == int(quotas[e]), f"expert {e} keeps the wrong count"
        if 0 < quotas[e] < counts[e]:
            tau = taus[e]
            exempt[lo:hi] = np.abs(ref_scores[lo:hi] - tau) <= BAND * tau
    bad = (keep_gpu != keep_ref) & ~exempt
    assert not bad.any(), f"{int(bad.sum())} keep flags differ outside the threshold band"
    return bool((keep_gpu == keep_ref).all())


def abs_rows(x):
    """|x| of stored rows: clears the sign bit of bf16 bit patterns."""
    return x & np.uint16(0x7FFF) if x.dtype == np.uint16 else np.abs(x)


def single_rounding_bound(sum_abs, k_max):
    """Per-element error bound of the single-rounding dW mode.  Each term
    alpha_j g_j[o] phi_j[i] uses bf16(alpha_j phi_j[i]) (or bf16(alpha_j
    g_j[o])): one round to nearest with 8 significant bits, relative error at
    most 2^-8, on top of the float32 product (2^-24).  The fp32 sum of up to
    k_max terms (MFMA accumulation and the split-K partial sums) adds at most
    k_max * 2^-24 relative per term; doubled here for slack.  sum_abs is
    sum_j |alpha_j g_j[o] phi_j[i]|, computed by the oracle on |inputs|."""
    return (2.0 ** -8 + 2.0 ** -24 + 2 * k_max * 2.0 ** -24) * sum_abs + 1e-30


def check_single_rounding(got, ref, sum_abs, k_max, what):
    bound = single_rounding_bound(sum_abs, k_max)
    excess = np.abs(got.astype(np.float64) - ref) / bound
    assert excess.max() <= 1.0, f"{what}: error {excess.max():.3f} x the single-rounding bound"
    return float(excess.max())


def rel_err(got, ref):
    m = np.abs(ref).max()
    if m == 0:
        return float(np.abs(got).max())
    return float(np.abs(got.astype(np.float64) - ref).max() / m)


def compare_full(p, quotas, out, dw_mode=lrmoe.DW_EXACT, scores_in=None, score_mode="lrm"):
    """Full oracle comparison (small and medium problems)."""
    ref = O.pruned_backward(p.counts, ("ratio", 1, 1), p.alpha, p.g, p.phi, p.W, p.row_index,
                            p.dtype, with_grads=False, score_mode=score_mode)
    R = ref["scores"] if scores_in is None else scores_in.astype(np.float64)
    keep_ref, taus = O.select_top_quota(R, p.counts, quotas)
    keep_gpu = out["keep"].cpu().numpy().astype(bool)
    same = check_keep(R, p.counts, quotas, keep_gpu, keep_ref, taus)
    keep_used = keep_ref if same else keep_gpu
    perm, seg = O.compact(keep_used, p.counts, quotas)
    assert np.array_equal(out["seg_offsets"].cpu().numpy(), seg)
    assert np.array_equal(out["perm"].cpu().numpy(), perm)
    g_c, phi_c, a_c = O.gather(perm, p.row_index, p.g, p.phi, p.alpha)
    assert np.array_equal(host_bits(out["g_c"]), g_c)
    assert np.array_equal(host_bits(out["phi_c"]), phi_c)
    assert np.array_equal(out["alpha_c"].cpu().numpy(), a_c)
    if scores_in is None:
        s = out["scores"].cpu().numpy().astype(np.float64)
        assert np.all(np.abs(s - R) <= 1e-5 * np.maximum(R, 1e-30))
    dW_ref = O.weight_grad(seg, a_c, g_c, phi_c, p.dtype, p.E, p.d_out, p.d_in)
    dphi_ref = O.input_grad(seg, perm, a_c, g_c, p.W, p.dtype, p.P)
    dW_gpu = out["dW"].cpu().numpy()
    errs = dict(dW=rel_err(dW_gpu, dW_ref), dphi=rel_err(out["dphi"].cpu().numpy(), dphi_ref))
    assert errs["dphi"] <= TOL, f"dphi: max err / max|ref| = {errs['dphi']:.3e}"
    if dw_mode == lrmoe.DW_BF16 and p.dtype == "bf16":
        # single rounding of alpha * x to bf16: not within TOL in general (few
        # rows per expert leave the 2^-8 rounding unaveraged), but within its
        # per-element bound
        s_abs = O.weight_grad(seg, np.abs(a_c), abs_rows(g_c), abs_rows(phi_c), p.dtype, p.E,
                              p.d_out, p.d_in)
        k_max = int(np.max(np.diff(seg))) if len(seg) > 1 else 0
        errs["dW_bound_use"] = check_single_rounding(dW_gpu, dW_ref, s_abs, k_max, "dW")
    else:
        assert errs["dW"] <= TOL, f"dW: max err / max|ref| = {errs['dW']:.3e}"
    dphi_gpu = out["dphi"].cpu().numpy()
    assert np.all(dphi_gpu[~keep_used] == 0)
    return errs, same


def check_dgu(got, ref):
    """The chain's compacted gate/up output gradient against the oracle's
    float64 value.  float32 hand-off: float32 arithmetic (the hardware exp2
    and reciprocal in the sigmoid, about one ulp each) within 2^-16 of each
    entry, plus 2e-5 max|ref| for the float32 sum of W^T g.  bf16 hand-off
    (single-rounding mode): one rounding to 8 significant bits on top,
    2^-8 of each entry."""
    if got.dtype == torch.bfloat16:
        v = (host_bits(got).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        rel = 2.0 ** -8
    else:
        assert got.dtype == torch.float32
        v = got.cpu().numpy().astype(np.float64)
        rel = 2.0 ** -16
    if ref.size == 0:
        return 0.0
    bound = rel * np.abs(ref) + 2e-5 * np.abs(ref).max()
    excess = np.abs(v - ref) - bound
    assert np.all(excess <= 0), float(excess.max())
    return float(np.abs(v - ref).max() / max(np.abs(ref).max(), 1e-300))
