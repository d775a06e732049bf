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
    errs = dict(dW=rel_err(out["dW"].cpu().numpy(), dW_ref),
                dphi=rel_err(out["dphi"].cpu().numpy(), dphi_ref))
    for k, v in errs.items():
        assert v <= TOL, f"{k}: max err / max|ref| = {v:.3e}"
    dphi_gpu = out["dphi"].cpu().numpy()
    assert np.all(dphi_gpu[~keep_used] == 0)
    return errs, same
