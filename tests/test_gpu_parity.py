"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Small and medium problems are compared element by element: several 256x256
tiles, ragged row and column tails, empty experts, zero and full quotas,
fp32 and bf16 storage, per-token g (row indirection) and per-pair g, ties,
and a seeded sweep of random shapes.
Full-size workloads are in test_gpu_fullsize.py."""
import numpy as np
import pytest
import torch

from oracle import lrmoe_oracle as O
from pruned_expert_backward_amd import lrmoe
from pruned_expert_backward_amd import workloads as W

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from tests import gpu_util as U  # noqa: E402


def test_tiny_config_fp32_per_token():
    p = W.config(0)
    q = lrmoe.plan_quota(p.counts, p.policy)
    plan, out, _ = U.run_gpu(p, q)
    errs, same = U.compare_full(p, q, out)
    assert same
    print("tiny-fp32", errs)


MEDIUM = [
    # name, kwargs of make_problem, policy
    ("ragged-bf16-c20", dict(P=3000, E=5, d_out=264, d_in=200, dtype="bf16",
                             counts=[1400, 0, 977, 7, 616]), ("ratio", 80, 100)),
    ("ragged-bf16-c30", dict(P=2500, E=6, d_out=136, d_in=392, dtype="bf16", zipf=1.6),
     ("ratio", 70, 100)),
    ("bf16-c0-full", dict(P=1000, E=3, d_out=256, d_in=128, dtype="bf16", zipf=1.0),
     ("ratio", 1, 1)),
    ("bf16-drop-all", dict(P=700, E=4, d_out=128, d_in=128, dtype="bf16", zipf=1.2),
     ("ratio", 0, 1)),
    ("bf16-budget", dict(P=4000, E=16, d_out=256, d_in=176, dtype="bf16", zipf=1.4),
     ("budget", 900)),
    ("fp32-ragged", dict(P=1500, E=4, d_out=196, d_in=140, dtype="f32", zipf=1.2),
     ("ratio", 80, 100)),
    ("bf16-one-expert", dict(P=777, E=1, d_out=128, d_in=264, dtype="bf16", zipf=1.0),
     ("ratio", 1, 2)),
    # float32 storage (four operand planes) with an expert split along K:
    # 2400 kept rows make three chunks whose partial tiles are reduced
    ("fp32-split-k", dict(P=4000, E=3, d_out=136, d_in=200, dtype="f32",
                          counts=[3000, 700, 300]), ("ratio", 80, 100)),
    # 256 experts (the most the ABI takes), 16 row tiles and one column tile:
    # two weight-gradient groups per expert and one input-gradient group make
    # about 768 tile groups, more than the schedule table holds, so the GEMM
    # runs on its formula-order schedule
    ("bf16-256-experts-formula-schedule",
     dict(P=16384, E=256, d_out=4096, d_in=64, dtype="bf16", zipf=1.0), ("ratio", 80, 100)),
]


@pytest.mark.parametrize("idx", range(len(MEDIUM)), ids=[m[0] for m in MEDIUM])
def test_medium(idx):
    name, kw, policy = MEDIUM[idx]
    p = W.make_problem(seed=100 + idx, policy=policy, name=name, **kw)
    q = lrmoe.plan_quota(p.counts, policy)
    assert q == O.plan_quota(p.counts, policy)
    plan, out, _ = U.run_gpu(p, q)
    errs, same = U.compare_full(p, q, out)
    print(name, errs, "keep identical" if same else "keep differs inside band")


MEDIUM_F16 = [(i, m) for i, m in enumerate(MEDIUM) if m[1]["dtype"] == "bf16"]


@pytest.mark.parametrize("j", range(len(MEDIUM_F16)), ids=[m[0] + "-f16" for _, m in MEDIUM_F16])
def test_medium_f16(j):
    """The float16 weight-gradient mode (one matrix-core pass on float16
    planes, alpha * operand rounded once to 11 significant bits, per-expert
    power-of-two scales) on the medium shapes: keep set, compaction and dphi
    as always, dW within 2e-3 max|ref| of the oracle."""
    idx, (name, kw, policy) = MEDIUM_F16[j]
    p = W.make_problem(seed=100 + idx, policy=policy, name=name, **kw)
    q = lrmoe.plan_quota(p.counts, policy)
    plan, out, _ = U.run_gpu(p, q, dw_mode=lrmoe.DW_F16)
    errs, same = U.compare_full(p, q, out, dw_mode=lrmoe.DW_F16)
    print(name, "f16", errs)


def _scaled_rows(x, offsets, factors):
    """bf16 rows of each expert multiplied by its factor (rounded to bf16)."""
    v = (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    for e, f in enumerate(factors):
        v[offsets[e]:offsets[e + 1]] *= f
    return W.to_bf16_bits(v.astype(np.float32))


@pytest.mark.parametrize("d_out,d_in", [(200, 136), (136, 200), (1160, 1040)],
                         ids=["alpha-on-phi", "alpha-on-g", "two-planes"])
def test_f16_wide_range_per_expert(d_out, d_in):
    """The float16 mode on inputs far outside float16's range: every expert's
    g rows and phi rows carry their own power of ten (g from 1e-7 to 1e5,
    phi from 1e-4 to 1e3), so unscaled products would overflow 65504 or
    vanish below float16's smallest normal.  The per-expert scales must map
    each expert into range: every expert's dW within 2e-3 of its own max|ref|
    (not just of the whole tensor's), through both paths (one call, and the
    separate calls whose prologue finds the scales), bit for bit alike.
    Narrow shapes convert the operand without alpha in the GEMM's registers
    (A or B); the last shape reads float16 planes of both."""
    import dataclasses
    counts = [400, 300, 350, 250, 300]
    p = W.make_problem(P=sum(counts), E=5, d_out=d_out, d_in=d_in, dtype="bf16", counts=counts,
                       seed=61, policy=("ratio", 4, 5), name="wide-range")
    off = p.offsets
    p = dataclasses.replace(p, g=_scaled_rows(p.g, off, [1e-7, 1e-2, 1.0, 1e3, 1e5]),
                            phi=_scaled_rows(p.phi, off, [1e3, 1e-4, 1.0, 10.0, 1e-2]))
    q = lrmoe.plan_quota(p.counts, p.policy)
    plan, sep, t = U.run_gpu(p, q, dw_mode=lrmoe.DW_F16)
    one = lrmoe.pruned_backward(plan, t["alpha"], t["g"], t["phi"], t["W"])
    torch.cuda.synchronize()
    for k in ("keep", "perm", "dW", "dphi"):
        assert torch.equal(sep[k], one[k]), k
    keep = sep["keep"].cpu().numpy().astype(bool)
    perm, seg = O.compact(keep, p.counts, q)
    g_c, phi_c, a_c = O.gather(perm, None, p.g, p.phi, p.alpha)
    dW_ref = O.weight_grad(seg, a_c, g_c, phi_c, "bf16", p.E, p.d_out, p.d_in)
    dW = sep["dW"].cpu().numpy()
    per_expert = [U.rel_err(dW[e], dW_ref[e]) for e in range(p.E)]
    print("wide-range per-expert dW err", per_expert)
    assert max(per_expert) <= U.TOL, per_expert
    dphi_ref = O.input_grad(seg, perm, a_c, g_c, p.W, "bf16", p.P)
    dphi = sep["dphi"].cpu().numpy()
    for e in range(p.E):   # dphi per expert block too (bf16 matrix cores, alpha in float32)
        lo, hi = off[e], off[e + 1]
        assert U.rel_err(dphi[lo:hi], dphi_ref[lo:hi]) <= U.TOL, e


def test_f16_token_rows():
    """The float16 mode with per-token g rows through a row index (top-2
    routing of 700 tokens): the score pass takes each pair's g row maximum
    through the index.  Oracle parity, and the one-call path bit for bit the
    separate calls."""
    p = W.make_token_problem(T=700, E=6, topk=2, d_out=48, d_in=40, dtype="bf16", seed=373,
                             policy=("ratio", 3, 4))
    q = lrmoe.plan_quota(p.counts, p.policy)
    plan, sep, t = U.run_gpu(p, q, dw_mode=lrmoe.DW_F16)
    errs, _ = U.compare_full(p, q, sep, dw_mode=lrmoe.DW_F16)
    one = lrmoe.pruned_backward(plan, t["alpha"], t["g"], t["phi"], t["W"], g_row_index=t["row"])
    torch.cuda.synchronize()
    for k in ("keep", "perm", "dW", "dphi"):
        assert torch.equal(sep[k], one[k]), k
    print("f16 token rows", errs)


def test_dw_single_rounding_mode():
    """The one-pass bf16(alpha*x) mode: same keep set and dphi; dW within the
    per-element bound of that one bf16 rounding."""
    p = W.make_problem(P=3000, E=4, d_out=256, d_in=256, dtype="bf16", zipf=1.2, seed=77)
    q = lrmoe.plan_quota(p.counts, ("ratio", 80, 100))
    plan, out, _ = U.run_gpu(p, q, dw_mode=lrmoe.DW_BF16)
    errs, _ = U.compare_full(p, q, out)
    print("dw bf16 mode", errs)


@pytest.mark.parametrize("distinct", [1, 3, 17])
def test_ties_given_scores(distinct):
    """Caller-provided scores with many equal values: the keep set must be
    exactly the oracle's (ties to the lower pair index), no band."""
    p = W.make_problem(P=5000, E=7, d_out=64, d_in=64, dtype="bf16", zipf=1.3, seed=distinct)
    s = W.random_scores(p.P, seed=distinct, distinct=distinct)
    for policy in (("ratio", 80, 100), ("ratio", 1, 3), ("ratio", 1, 1)):
        q = lrmoe.plan_quota(p.counts, policy)
        plan, out, _ = U.run_gpu(p, q, scores=s)
        keep_ref, _ = O.select_top_quota(s.astype(np.float64), p.counts, q)
        assert np.array_equal(out["keep"].cpu().numpy().astype(bool), keep_ref)
        U.compare_full(p, q, out, scores_in=s)


@pytest.mark.parametrize("distinct,layout", [(0, 0), (3, 0), (1, 0), (0, 1), (3, 1), (0, 2),
                                             (3, 2)])
def test_select_large_experts(distinct, layout):
    """An expert above the LDS key cache (24576 pairs) sends the problem
    through the chunked passes (4096-pair chunks of every expert): continuous
    scores, 3 values, or one value for all pairs; experts starting at
    unaligned pair offsets (the scan's second, short tile), of one, two or
    several chunks, empty, keeping nothing or everything; 64 experts (the
    per-expert histograms and state at larger offsets, the chunk-to-expert
    lookup over many experts)."""
    many = [30001] + [((7 * i) % 50) * 37 for i in range(1, 64)]   # zeros among them
    counts = [[90000, 30000, 4000, 1, 0], [30001, 4097, 3, 0, 8190, 2, 4096], many][layout]
    p = W.make_problem(P=sum(counts), E=len(counts), d_out=8, d_in=8, dtype="bf16",
                       counts=counts, seed=40 + layout)
    s = W.random_scores(p.P, seed=40 + distinct, distinct=distinct)
    for policy in (("ratio", 80, 100), ("ratio", 1, 3), ("ratio", 1, 1), ("budget", 5000)):
        q = lrmoe.plan_quota(p.counts, policy)
        plan, out, _ = U.run_gpu(p, q, scores=s)
        keep_ref, _ = O.select_top_quota(s.astype(np.float64), p.counts, q)
        assert np.array_equal(out["keep"].cpu().numpy().astype(bool), keep_ref), policy
        perm, seg = O.compact(keep_ref, p.counts, q)
        assert np.array_equal(out["perm"].cpu().numpy(), perm), policy
        assert np.array_equal(out["seg_offsets"].cpu().numpy(), seg), policy


@pytest.mark.parametrize("mode,name", [(lrmoe.SCORE_GRAD_SQNORM, "sqnorm"),
                                       (lrmoe.SCORE_GRAD_L1, "l1")])
def test_ablation_score_modes(mode, name):
    """Gradient-only scoring rules (the pages' ablation baselines): scores,
    keep sets, compaction and gradients against the oracle's same rule, on a
    bf16 problem and on the per-token float32 one."""
    for p in (W.make_problem(P=4000, E=6, d_out=256, d_in=136, dtype="bf16", zipf=1.3, seed=31),
              W.config(0)):
        q = lrmoe.plan_quota(p.counts, ("ratio", 80, 100))
        plan, out, _ = U.run_gpu(p, q, score_mode=mode)
        errs, _ = U.compare_full(p, q, out, score_mode=name)
        print(name, p.name, errs)


@pytest.mark.parametrize("dw_mode", [lrmoe.DW_EXACT, lrmoe.DW_BF16, lrmoe.DW_F16])
def test_masked_dense_matches_compacted(dw_mode):
    """The zero-masked dense alternative (alpha := 0 on dropped pairs, the
    same GEMMs over every routed pair, nothing compacted) reproduces the
    compacted result: same keep set, dW and dphi within tolerance, dropped
    dphi rows exactly 0."""
    p = W.make_problem(P=3000, E=5, d_out=256, d_in=136, dtype="bf16", zipf=1.3, seed=41)
    policy = ("ratio", 70, 100)
    q = lrmoe.plan_quota(p.counts, policy)
    plan = lrmoe.Plan(p.counts, q, p.d_out, p.d_in, lrmoe.BF16, dw_mode=dw_mode)
    t = dict(alpha=U.dev(p.alpha), g=U.dev(p.g), phi=U.dev(p.phi), W=U.dev(p.W))
    out = lrmoe.masked_dense_backward(plan, t["alpha"], t["g"], t["phi"], t["W"])
    torch.cuda.synchronize()
    ref = O.pruned_backward(p.counts, policy, p.alpha, p.g, p.phi, p.W, None, "bf16",
                            with_grads=False)
    keep = out["keep"].cpu().numpy().astype(bool)
    U.check_keep(ref["scores"], p.counts, q, keep, ref["keep"], ref["taus"])
    perm, seg = O.compact(keep, p.counts, q)
    g_c, phi_c, a_c = O.gather(perm, None, p.g, p.phi, p.alpha)
    dW_ref = O.weight_grad(seg, a_c, g_c, phi_c, "bf16", p.E, p.d_out, p.d_in)
    dphi_ref = O.input_grad(seg, perm, a_c, g_c, p.W, "bf16", p.P)
    dphi = out["dphi"].cpu().numpy()
    assert U.rel_err(dphi, dphi_ref) <= U.TOL
    assert np.all(dphi[~keep] == 0)
    if dw_mode != lrmoe.DW_BF16:
        assert U.rel_err(out["dW"].cpu().numpy(), dW_ref) <= U.TOL
    else:
        # single rounding of alpha * operand: within that rounding's per-element
        # bound around the oracle (dropped pairs enter with alpha = 0, exactly
        # nothing; the float32 sums run over every routed pair of an expert)
        s_abs = O.weight_grad(seg, np.abs(a_c), U.abs_rows(g_c), U.abs_rows(phi_c), "bf16", p.E,
                              p.d_out, p.d_in)
        U.check_single_rounding(out["dW"].cpu().numpy(), dW_ref, s_abs, int(max(p.counts)), "dW")
    am = out["alpha_masked"].cpu().numpy()
    assert np.array_equal(am, np.where(keep, p.alpha, np.float32(0)))
    assert np.array_equal(out["perm_identity"].cpu().numpy(), np.arange(p.P))


def test_negative_and_signed_zero_scores():
    """The order-preserving key handles negative scores and -0.0 == 0.0."""
    p = W.make_problem(P=600, E=3, d_out=32, d_in=32, dtype="bf16", counts=[200, 250, 150], seed=5)
    rng = np.random.default_rng(3)
    s = rng.choice(np.array([-2.5, -1.0, -0.0, 0.0, 1e-30, 3.0], dtype=np.float32), size=p.P)
    q = lrmoe.plan_quota(p.counts, ("ratio", 1, 2))
    plan, out, _ = U.run_gpu(p, q, scores=s)
    keep_ref, _ = O.select_top_quota(s.astype(np.float64), p.counts, q)
    assert np.array_equal(out["keep"].cpu().numpy().astype(bool), keep_ref)


def test_deterministic_bitwise():
    p = W.make_problem(P=4000, E=8, d_out=256, d_in=136, dtype="bf16", zipf=1.2, seed=9)
    q = lrmoe.plan_quota(p.counts, ("ratio", 80, 100))
    _, a, _ = U.run_gpu(p, q)
    _, b, _ = U.run_gpu(p, q)
    for k in ("scores", "keep", "perm", "seg_offsets", "g_c", "phi_c", "alpha_c", "dW", "dphi"):
        assert torch.equal(a[k].view(torch.uint8) if a[k].dtype == torch.bfloat16 else a[k],
                           b[k].view(torch.uint8) if b[k].dtype == torch.bfloat16 else b[k]), k


def test_gate_up_inherits_keep_set():
    """Second projection (gate/up) on the first one's keep set and perm."""
    p = W.make_problem(P=2000, E=4, d_out=128, d_in=96, dtype="bf16", zipf=1.6, seed=12,
                       gate_up=(144, 256))
    q = lrmoe.plan_quota(p.counts, ("ratio", 70, 100))
    plan, out, t = U.run_gpu(p, q)
    gu = p.gate_up
    plan2 = lrmoe.Plan(p.counts, q, gu.d_out, gu.d_in, lrmoe.BF16)
    c2 = lrmoe.gather_compact(plan2, out["perm"], out["keep"], t["alpha"], U.dev(gu.g2),
                              U.dev(gu.x))
    dW2 = lrmoe.grouped_backward(plan2, out["perm"], c2["alpha_c"], c2["g_c"], c2["phi_c"],
                                 U.dev(gu.W2), dphi=c2["dphi"])
    torch.cuda.synchronize()
    ref = O.pruned_backward(p.counts, ("ratio", 70, 100), p.alpha, p.g, p.phi, p.W, None, "bf16",
                            gate_up=(gu.g2, gu.x, gu.W2))
    assert np.array_equal(out["keep"].cpu().numpy().astype(bool), ref["keep"])
    assert np.array_equal(U.host_bits(c2["g_c"]), gu.g2[ref["perm"]])
    assert np.array_equal(U.host_bits(c2["phi_c"]), gu.x[ref["perm"]])
    e1 = U.rel_err(dW2.cpu().numpy(), ref["dW2"])
    e2 = U.rel_err(c2["dphi"].cpu().numpy(), ref["dx"])
    assert e1 <= U.TOL and e2 <= U.TOL, (e1, e2)
    # the same in one call (gather writing the GEMM's operand planes): bit for bit
    one = lrmoe.gather_backward(plan2, out["perm"], out["keep"], t["alpha"], U.dev(gu.g2),
                                U.dev(gu.x), U.dev(gu.W2))
    torch.cuda.synchronize()
    assert torch.equal(one["dW"], dW2) and torch.equal(one["dphi"], c2["dphi"])
    for k in ("g_c", "phi_c"):
        assert torch.equal(one[k].view(torch.int16), c2[k].view(torch.int16)), k


GLU_CASES = [
    # name, make_problem kwargs, dw_mode (the GEMM variant the chain runs in)
    ("glu-alpha-on-phi", dict(P=2400, E=5, d_out=264, d_in=200, counts=[1100, 0, 700, 9, 591],
                              gate_up=(400, 136)), lrmoe.DW_EXACT),
    ("glu-alpha-on-g", dict(P=1800, E=4, d_out=136, d_in=328, zipf=1.6,
                            gate_up=(656, 264)), lrmoe.DW_EXACT),
    ("glu-bf16-single-rounding", dict(P=2000, E=6, d_out=256, d_in=256, zipf=1.2,
                                      gate_up=(512, 128)), lrmoe.DW_BF16),
    ("glu-f16", dict(P=2200, E=5, d_out=264, d_in=200, zipf=1.4, gate_up=(400, 136)),
     lrmoe.DW_F16),
]


@pytest.mark.parametrize("idx", range(len(GLU_CASES)), ids=[c[0] for c in GLU_CASES])
def test_glu_chain(idx):
    """The expert MLP chained on the compacted layout: down projection dW,
    the SiLU-GLU backward written compacted by the input-gradient tiles
    (dgu_c: float32 in the exact mode, bf16 in the single-rounding one), then
    the gate/up projection's dW2 and dx on the same keep set, against the
    oracle's unrounded float64 chain.  dgu_c within check_dgu's bound; dW,
    dW2 and dx within 2e-3 max|ref| (exact mode), or within the
    single-rounding bounds."""
    name, kw, dw_mode = GLU_CASES[idx]
    p = W.make_problem(seed=300 + idx, dtype="bf16", glu=True, policy=("ratio", 70, 100),
                       name=name, **kw)
    gu, gl = p.gate_up, p.glu
    q = lrmoe.plan_quota(p.counts, p.policy)
    plan = lrmoe.Plan(p.counts, q, p.d_out, p.d_in, lrmoe.BF16, dw_mode=dw_mode)
    plan2 = lrmoe.Plan(p.counts, q, gu.d_out, gu.d_in, lrmoe.BF16, dw_mode=dw_mode)
    d = U.dev
    out = lrmoe.glu_chain_backward(plan, plan2, d(p.alpha), d(p.g), d(p.phi), d(p.W), d(gl.a),
                                   d(gl.b), d(gu.x), d(gu.W2))
    torch.cuda.synchronize()
    ref = O.pruned_backward(p.counts, p.policy, p.alpha, p.g, p.phi, p.W, None, "bf16",
                            glu=(gl.a, gl.b, gu.x, gu.W2))
    assert U.check_keep(ref["scores"], p.counts, q, out["keep"].cpu().numpy().astype(bool),
                        ref["keep"], ref["taus"]), "keep set inside the band: reseed"
    assert np.array_equal(out["perm"].cpu().numpy(), ref["perm"])
    assert np.array_equal(U.host_bits(out["x_c"]), gu.x[ref["perm"]])
    assert out["dgu_c"].dtype == (torch.bfloat16 if dw_mode == lrmoe.DW_BF16 else torch.float32)
    e_dgu = U.check_dgu(out["dgu_c"], ref["dgu_c"])
    errs = dict(dW=U.rel_err(out["dW"].cpu().numpy(), ref["dW"]),
                dW2=U.rel_err(out["dW2"].cpu().numpy(), ref["dW2"]),
                dx=U.rel_err(out["dx"].cpu().numpy(), ref["dx"]))
    print(name, dict(dgu=e_dgu, **errs))
    if dw_mode == lrmoe.DW_BF16:   # one bf16 rounding per term: that mode's bounds
        _check_chain_single_rounding(p, ref, out)
        errs = {}
    for k, v in errs.items():
        assert v <= U.TOL, (k, v)
    assert np.all(out["dx"].cpu().numpy()[~ref["keep"]] == 0)


def _check_chain_single_rounding(p, ref, out):
    """The single-rounding chain against the oracle's unrounded chain, per
    element.  dW: one bf16 rounding of alpha * operand per term (the
    oracle's sums of |alpha g phi|).  dW2 and dx: each term carries the bf16
    rounding of dgu (2^-8 relative at most, with the float32 error of dgu
    itself far below it) and, in dW2, that of alpha * dgu again -- three
    times the 2^-8 term (sums of |alpha dgu x| and |alpha W2^T dgu|) covers
    both with room for the float32 sums.  dx rows of dropped pairs are 0."""
    perm, seg = ref["perm"], ref["seg"]
    g_c, phi_c, a_c = O.gather(perm, p.row_index, p.g, p.phi, p.alpha)
    a = np.abs(a_c)
    k_max = int(np.max(np.diff(seg)))
    s1 = O.weight_grad(seg, a, U.abs_rows(g_c), U.abs_rows(phi_c), "bf16", p.E, p.d_out,
                       p.d_in)
    U.check_single_rounding(out["dW"].cpu().numpy(), ref["dW"], s1, k_max, "dW")
    gu = p.gate_up
    adgu = np.abs(ref["dgu_c"]) * (1 + 2.0 ** -8)
    s2 = 3.0 * O.weight_grad(seg, a, adgu, O.to_f64(U.abs_rows(gu.x[perm]), "bf16"), "f64",
                             p.E, gu.d_out, gu.d_in)
    U.check_single_rounding(out["dW2"].cpu().numpy(), ref["dW2"], s2, k_max, "dW2")
    s3 = 3.0 * O.input_grad(seg, perm, a, adgu, O.to_f64(U.abs_rows(gu.W2), "bf16"), "f64", p.P)
    U.check_single_rounding(out["dx"].cpu().numpy(), ref["dx"], s3, gu.d_out, "dx")


def _random_chain_problem(seed):
    """Seeded random MLP-chain shape: P from 1 to 4000, 1 to 10 experts,
    the expert's hidden width d_in (gate and up each), the model width
    d_out, both any multiple of 8 up to 520."""
    rng = np.random.default_rng(7000 + seed)
    E = int(rng.integers(1, 11))
    P = int(rng.integers(1, 64)) if seed % 3 == 1 else int(rng.integers(64, 4001))
    d_out = 8 * int(rng.integers(1, 66))
    d_in = 8 * int(rng.integers(1, 66))
    w = rng.random(E) * (rng.random(E) > 0.2)
    if w.sum() == 0:
        w[0] = 1.0
    counts = rng.multinomial(P, w / w.sum())
    den = int(rng.integers(1, 11))
    policy = ("ratio", int(rng.integers(0, den + 1)), den)
    return W.make_problem(P=P, E=E, d_out=d_out, d_in=d_in, dtype="bf16", counts=counts,
                          seed=600 + seed, policy=policy, glu=True, gate_up=(2 * d_in, d_out),
                          name=f"random-chain-{seed}")


@pytest.mark.parametrize("seed", range(6))
def test_glu_chain_random_shapes(seed):
    """The MLP chain on random shapes: keep set and perm exactly, the float32
    dgu_c within check_dgu's bound, dW, dW2 and dx within 2e-3 max|ref| of
    the oracle's unrounded chain."""
    p = _random_chain_problem(seed)
    gu, gl = p.gate_up, p.glu
    q = lrmoe.plan_quota(p.counts, p.policy)
    print(f"random-chain-{seed}: P={p.P} E={p.E} d_out={p.d_out} d_in={p.d_in} "
          f"{p.policy} M={sum(q)}", flush=True)
    plan = lrmoe.Plan(p.counts, q, p.d_out, p.d_in, lrmoe.BF16)
    plan2 = lrmoe.Plan(p.counts, q, gu.d_out, gu.d_in, lrmoe.BF16)
    d = U.dev
    out = lrmoe.glu_chain_backward(plan, plan2, d(p.alpha), d(p.g), d(p.phi), d(p.W), d(gl.a),
                                   d(gl.b), d(gu.x), d(gu.W2))
    torch.cuda.synchronize()
    ref = O.pruned_backward(p.counts, p.policy, p.alpha, p.g, p.phi, p.W, None, "bf16",
                            glu=(gl.a, gl.b, gu.x, gu.W2))
    same = U.check_keep(ref["scores"], p.counts, q, out["keep"].cpu().numpy().astype(bool),
                        ref["keep"], ref["taus"])
    assert same, "keep set inside the threshold band: reseed"
    assert np.array_equal(out["perm"].cpu().numpy(), ref["perm"])
    U.check_dgu(out["dgu_c"], ref["dgu_c"])
    errs = dict(dW=U.rel_err(out["dW"].cpu().numpy(), ref["dW"]),
                dW2=U.rel_err(out["dW2"].cpu().numpy(), ref["dW2"]),
                dx=U.rel_err(out["dx"].cpu().numpy(), ref["dx"]))
    print(f"random-chain-{seed}", errs)
    for k, v in errs.items():
        assert v <= U.TOL, (k, v)
    assert np.all(out["dx"].cpu().numpy()[~ref["keep"]] == 0)


@pytest.mark.parametrize("seed", range(6))
def test_gate_up_random_shapes(seed):
    """A second projection on the first one's keep set (lrmoe_gather_backward)
    on random shapes, against the oracle."""
    rng = np.random.default_rng(8000 + seed)
    E = int(rng.integers(1, 11))
    P = int(rng.integers(1, 64)) if seed % 3 == 1 else int(rng.integers(64, 4001))
    d_out, d_in = 8 * int(rng.integers(1, 66)), 8 * int(rng.integers(1, 66))
    d2o, d2i = 8 * int(rng.integers(1, 66)), 8 * int(rng.integers(1, 66))
    counts = rng.multinomial(P, np.full(E, 1.0 / E))
    den = int(rng.integers(1, 11))
    policy = ("ratio", int(rng.integers(0, den + 1)), den)
    p = W.make_problem(P=P, E=E, d_out=d_out, d_in=d_in, dtype="bf16", counts=counts,
                       seed=650 + seed, gate_up=(d2o, d2i), name=f"random-gu-{seed}")
    q = lrmoe.plan_quota(p.counts, policy)
    print(f"random-gu-{seed}: P={P} E={E} down {d_out}x{d_in} gate/up {d2o}x{d2i} {policy} "
          f"M={sum(q)}", flush=True)
    plan, out, t = U.run_gpu(p, q)
    gu = p.gate_up
    plan2 = lrmoe.Plan(p.counts, q, gu.d_out, gu.d_in, lrmoe.BF16)
    one = lrmoe.gather_backward(plan2, out["perm"], out["keep"], t["alpha"], U.dev(gu.g2),
                                U.dev(gu.x), U.dev(gu.W2))
    torch.cuda.synchronize()
    ref = O.pruned_backward(p.counts, policy, p.alpha, p.g, p.phi, p.W, None, "bf16",
                            gate_up=(gu.g2, gu.x, gu.W2))
    U.check_keep(ref["scores"], p.counts, q, out["keep"].cpu().numpy().astype(bool),
                 ref["keep"], ref["taus"])
    keep = out["keep"].cpu().numpy().astype(bool)
    # the oracle's compaction of the GPU keep set (equal to its own where the
    # keep sets agree; they may differ only inside the threshold band)
    perm, seg = O.compact(keep, p.counts, q)
    assert np.array_equal(out["perm"].cpu().numpy(), perm)
    g2_c, x_c, a_c = O.gather(perm, None, gu.g2, gu.x, p.alpha)
    assert np.array_equal(U.host_bits(one["g_c"]), g2_c)
    assert np.array_equal(U.host_bits(one["phi_c"]), x_c)
    dW2_ref = O.weight_grad(seg, a_c, g2_c, x_c, "bf16", p.E, gu.d_out, gu.d_in)
    dx_ref = O.input_grad(seg, perm, a_c, g2_c, gu.W2, "bf16", p.P)
    e1 = U.rel_err(one["dW"].cpu().numpy(), dW2_ref)
    e2 = U.rel_err(one["dphi"].cpu().numpy(), dx_ref)
    print(f"random-gu-{seed}", dict(dW2=e1, dx=e2))
    assert e1 <= U.TOL and e2 <= U.TOL, (e1, e2)
    assert np.all(one["dphi"].cpu().numpy()[~keep] == 0)


def test_glu_chain_edges():
    """The MLP chain at its edges: no kept pair at all (M = 0: dW, dW2 and dx
    all zero, nothing else written); tiny ragged shapes (d_in = 8, two
    experts, one of them empty); one expert whose kept rows and columns
    straddle tile edges (q = 301, d_in = 264)."""
    cases = [
        (dict(P=120, E=3, d_out=64, d_in=32, counts=[50, 40, 30], gate_up=(64, 48)), ("ratio", 0, 1)),
        (dict(P=40, E=2, d_out=8, d_in=8, counts=[40, 0], gate_up=(16, 8)), ("ratio", 3, 4)),
        (dict(P=430, E=1, d_out=136, d_in=264, counts=[430], gate_up=(528, 40)), ("ratio", 7, 10)),
    ]
    for i, (kw, policy) in enumerate(cases):
        p = W.make_problem(seed=320 + i, dtype="bf16", glu=True, policy=policy, **kw)
        gu, gl = p.gate_up, p.glu
        q = lrmoe.plan_quota(p.counts, policy)
        plan = lrmoe.Plan(p.counts, q, p.d_out, p.d_in, lrmoe.BF16)
        plan2 = lrmoe.Plan(p.counts, q, gu.d_out, gu.d_in, lrmoe.BF16)
        d = U.dev
        out = lrmoe.glu_chain_backward(plan, plan2, d(p.alpha), d(p.g), d(p.phi), d(p.W),
                                       d(gl.a), d(gl.b), d(gu.x), d(gu.W2))
        torch.cuda.synchronize()
        ref = O.pruned_backward(p.counts, policy, p.alpha, p.g, p.phi, p.W, None, "bf16",
                                glu=(gl.a, gl.b, gu.x, gu.W2))
        assert np.array_equal(out["keep"].cpu().numpy().astype(bool), ref["keep"]), i
        assert np.array_equal(out["perm"].cpu().numpy(), ref["perm"]), i
        assert tuple(out["dgu_c"].shape) == (sum(q), 2 * p.d_in)
        if sum(q) == 0:
            for k in ("dW", "dW2", "dx"):
                assert float(out[k].abs().max()) == 0.0, (i, k)
            continue
        U.check_dgu(out["dgu_c"], ref["dgu_c"])
        for k in ("dW", "dW2", "dx"):
            e = U.rel_err(out[k].cpu().numpy(), ref[k])
            assert e <= U.TOL, (i, k, e)


WHOLE = [
    ("bf16-exact-alpha-on-phi", dict(P=3000, E=5, d_out=264, d_in=200, dtype="bf16",
                                     counts=[1400, 0, 977, 7, 616]), lrmoe.DW_EXACT),
    ("bf16-exact-alpha-on-g", dict(P=2500, E=4, d_out=136, d_in=392, dtype="bf16", zipf=1.6),
     lrmoe.DW_EXACT),
    ("bf16-single-rounding", dict(P=2000, E=3, d_out=256, d_in=128, dtype="bf16", zipf=1.2),
     lrmoe.DW_BF16),
    ("fp32", dict(P=1500, E=4, d_out=196, d_in=140, dtype="f32", zipf=1.2), lrmoe.DW_EXACT),
    ("large-expert", dict(P=40000, E=2, d_out=64, d_in=72, dtype="bf16", counts=[39000, 1000]),
     lrmoe.DW_EXACT),
    # float16 weight gradient: the one call takes the expert scales from the
    # score pass and the select (a large expert's chunks merge them), the
    # separate calls from their own prologue over the compacted rows
    ("f16-alpha-on-phi", dict(P=3000, E=5, d_out=264, d_in=200, dtype="bf16",
                              counts=[1400, 0, 977, 7, 616]), lrmoe.DW_F16),
    ("f16-alpha-on-g", dict(P=2500, E=4, d_out=136, d_in=392, dtype="bf16", zipf=1.6),
     lrmoe.DW_F16),
    ("f16-large-expert", dict(P=40000, E=2, d_out=64, d_in=72, dtype="bf16",
                              counts=[39000, 1000]), lrmoe.DW_F16),
]


@pytest.mark.parametrize("idx", range(len(WHOLE)), ids=[w[0] for w in WHOLE])
def test_whole_path_call_matches_separate_calls(idx):
    """lrmoe_pruned_backward (one call; with bf16 storage the gather writes
    the GEMM's operand planes) gives bit for bit the results of
    lrmoe_score_select_compact followed by lrmoe_grouped_backward, including
    an expert large enough for the multi-workgroup histogram, whose workspace
    the planes reuse afterwards."""
    name, kw, dw_mode = WHOLE[idx]
    p = W.make_problem(seed=340 + idx, policy=("ratio", 4, 5), name=name, **kw)
    q = lrmoe.plan_quota(p.counts, p.policy)
    plan, sep, t = U.run_gpu(p, q, dw_mode=dw_mode)
    one = lrmoe.pruned_backward(plan, t["alpha"], t["g"], t["phi"], t["W"], g_row_index=t["row"])
    torch.cuda.synchronize()
    for k in ("scores", "keep", "perm", "seg_offsets", "g_c", "phi_c", "alpha_c", "dW", "dphi"):
        a, b = sep[k], one[k]
        if a.dtype == torch.bfloat16:
            a, b = a.view(torch.int16), b.view(torch.int16)
        assert torch.equal(a, b), (name, k)
    if idx == 0 or dw_mode == lrmoe.DW_F16:   # and the oracle agrees with both
        errs, _ = U.compare_full(p, q, one, dw_mode=dw_mode)
        print(name, errs)


def _random_problem(seed):
    """Seeded random shape: P from 1 to 6000 (a third of the cases under 64),
    1 to 12 experts with empty ones among them, row widths of any 16-byte
    multiple up to 600 (so tiles are full, ragged or a sliver), bf16 or fp32
    storage, ratio or budget quotas, exact or single-rounding dW."""
    rng = np.random.default_rng(9000 + seed)
    dtype = "f32" if seed % 3 == 0 else "bf16"
    step = 8 if dtype == "bf16" else 4
    E = int(rng.integers(1, 13))
    P = int(rng.integers(1, 64)) if seed % 3 == 1 else int(rng.integers(64, 6001))
    d_out = step * int(rng.integers(1, 600 // step + 1))
    d_in = step * int(rng.integers(1, 600 // step + 1))
    w = rng.random(E) * (rng.random(E) > 0.2)   # about one expert in five empty
    if w.sum() == 0:
        w[0] = 1.0
    counts = rng.multinomial(P, w / w.sum())
    if seed % 4 == 3:
        policy = ("budget", int(rng.integers(0, P + 1)))
    else:
        den = int(rng.integers(1, 11))
        policy = ("ratio", int(rng.integers(0, den + 1)), den)
    dw_mode = lrmoe.DW_BF16 if (dtype == "bf16" and seed % 5 == 2) else lrmoe.DW_EXACT
    p = W.make_problem(P=P, E=E, d_out=d_out, d_in=d_in, dtype=dtype, counts=counts,
                       seed=500 + seed, policy=policy, name=f"random-{seed}")
    return p, policy, dw_mode


def _random_problem_f16(seed):
    """Seeded random bf16 shape for the float16 mode (as _random_problem)."""
    rng = np.random.default_rng(9500 + seed)
    E = int(rng.integers(1, 13))
    P = int(rng.integers(1, 64)) if seed % 3 == 1 else int(rng.integers(64, 6001))
    d_out, d_in = 8 * int(rng.integers(1, 76)), 8 * int(rng.integers(1, 76))
    w = rng.random(E) * (rng.random(E) > 0.2)
    if w.sum() == 0:
        w[0] = 1.0
    counts = rng.multinomial(P, w / w.sum())
    den = int(rng.integers(1, 11))
    policy = ("ratio", int(rng.integers(0, den + 1)), den)
    p = W.make_problem(P=P, E=E, d_out=d_out, d_in=d_in, dtype="bf16", counts=counts,
                       seed=550 + seed, policy=policy, name=f"random-f16-{seed}")
    return p, policy


@pytest.mark.parametrize("seed", range(8))
def test_random_shapes_f16(seed):
    """The float16 mode on random shapes: oracle parity (dW and dphi within
    2e-3 max|ref|) and the one call bit for bit the separate calls."""
    p, policy = _random_problem_f16(seed)
    q = lrmoe.plan_quota(p.counts, policy)
    print(f"random-f16-{seed}: P={p.P} E={p.E} d_out={p.d_out} d_in={p.d_in} {policy} "
          f"M={sum(q)}", flush=True)
    plan, sep, t = U.run_gpu(p, q, dw_mode=lrmoe.DW_F16)
    errs, same = U.compare_full(p, q, sep, dw_mode=lrmoe.DW_F16)
    one = lrmoe.pruned_backward(plan, t["alpha"], t["g"], t["phi"], t["W"])
    torch.cuda.synchronize()
    for k in ("keep", "perm", "seg_offsets", "dW", "dphi"):
        assert torch.equal(sep[k], one[k]), (seed, k)
    print(f"random-f16-{seed}", errs)


@pytest.mark.parametrize("seed", range(10))
def test_random_shapes(seed):
    """Random shapes against the oracle (keep set, perm, offsets and the
    compacted rows exactly, dW and dphi within tolerance), and the one-call
    path bit for bit against the separate calls."""
    p, policy, dw_mode = _random_problem(seed)
    q = lrmoe.plan_quota(p.counts, policy)
    assert q == O.plan_quota(p.counts, policy)
    print(f"random-{seed}: P={p.P} E={p.E} d_out={p.d_out} d_in={p.d_in} {p.dtype} "
          f"{policy} dw_mode={dw_mode} M={sum(q)}", flush=True)
    plan, sep, t = U.run_gpu(p, q, dw_mode=dw_mode)
    errs, same = U.compare_full(p, q, sep, dw_mode=dw_mode)
    one = lrmoe.pruned_backward(plan, t["alpha"], t["g"], t["phi"], t["W"], g_row_index=t["row"])
    torch.cuda.synchronize()
    for k in ("keep", "perm", "seg_offsets", "dW", "dphi"):
        assert torch.equal(sep[k], one[k]), (seed, k)
    print(f"random-{seed}", errs, "keep identical" if same else "keep differs inside band")


@pytest.mark.parametrize("P,E,d_in,frac,dw_mode", [
    (37, 2, 136, (1, 2), lrmoe.DW_F16),       # fewer pairs than one wave's keep bytes
    (4099, 3, 200, (1, 5), lrmoe.DW_EXACT),   # ragged last chunk of 256 pairs
    (9000, 4, 1408, (1, 10), lrmoe.DW_F16),   # GLM-width rows, many chunks
    (777, 3, 72, (0, 1), lrmoe.DW_F16),       # nothing kept: every row dropped
    (120000, 4, 1408, (1, 10), lrmoe.DW_F16), # 608 MB of dropped rows: cleared in the GEMM launch
])
def test_dropped_rows_cleared(P, E, d_in, frac, dw_mode):
    """The one-call path and lrmoe_gather_backward clear the dropped pairs'
    dphi rows: in the gather, or (at least 512 MiB of them) inside the grouped
    GEMM launch, beside its tiles.  On dphi buffers filled with NaN
    beforehand, every dropped row comes back exactly zero and the whole buffer
    equals the separate calls' (whose gather clears the rows)."""
    p = W.make_problem(P=P, E=E, d_out=64, d_in=d_in, dtype="bf16", zipf=1.1, seed=P + d_in)
    q = [c * frac[0] // frac[1] for c in p.counts]
    plan, sep, t = U.run_gpu(p, q, dw_mode=dw_mode)
    print(f"cleared rows: P={P} E={E} d_in={d_in} M={sum(q)} "
          f"in the GEMM launch: {lrmoe.zero_fill_in_gemm(plan)}", flush=True)
    out = lrmoe.alloc_select_outputs(plan, t["g"].device)
    out["dphi"].fill_(float("nan"))
    one = lrmoe.pruned_backward(plan, t["alpha"], t["g"], t["phi"], t["W"], g_row_index=t["row"],
                                out=out)
    gb = lrmoe.gather_backward(plan, sep["perm"], sep["keep"], t["alpha"], t["g"], t["phi"],
                               t["W"], g_row_index=t["row"],
                               out={"dphi": torch.full((P, d_in), float("nan"),
                                                       device=t["g"].device)})
    torch.cuda.synchronize()
    dropped = ~sep["keep"].bool()
    for name, res in (("one call", one["dphi"]), ("gather_backward", gb["dphi"])):
        assert not torch.isnan(res).any(), name
        if bool(dropped.any()):
            assert float(res[dropped].abs().max()) == 0.0, name
        assert torch.equal(res, sep["dphi"]), name


def test_whole_path_call_nothing_kept():
    p = W.make_problem(P=500, E=3, d_out=64, d_in=32, dtype="bf16", counts=[200, 0, 300], seed=9)
    plan = lrmoe.Plan(p.counts, [0, 0, 0], p.d_out, p.d_in, lrmoe.BF16)
    one = lrmoe.pruned_backward(plan, U.dev(p.alpha), U.dev(p.g), U.dev(p.phi), U.dev(p.W))
    torch.cuda.synchronize()
    assert float(one["dW"].abs().max()) == 0.0 and float(one["dphi"].abs().max()) == 0.0
    assert not one["keep"].cpu().numpy().any()


def test_empty_problem_pieces():
    """All experts empty but one; quotas zero everywhere (M = 0)."""
    p = W.make_problem(P=300, E=4, d_out=64, d_in=64, dtype="bf16", counts=[0, 300, 0, 0], seed=2)
    q = [0, 0, 0, 0]
    plan, out, _ = U.run_gpu(p, q)
    assert out["seg_offsets"].cpu().tolist() == [0, 0, 0, 0, 0]
    assert not out["keep"].cpu().numpy().any()
    assert float(out["dW"].abs().max()) == 0.0
    assert float(out["dphi"].abs().max()) == 0.0


@pytest.mark.parametrize("policy", [("ratio", 80, 100), ("ratio", 7, 10), ("budget", 3000),
                                    ("budget", 10**6), ("ratio", 0, 1)])
def test_plan_quota_device(policy):
    """Quotas from the routing on the device equal the oracle's plan on the
    histogram of the same routing (bit-exact), including unrouted indices."""
    rng = np.random.default_rng(5)
    for E, n in ((16, 200003), (1, 17), (5, 0), (256, 4096)):
        ids = rng.integers(0, E, size=n).astype(np.int32)
        if n > 10:
            ids[rng.choice(n, 7, replace=False)] = rng.choice([-1, E, E + 3], size=7)
        out = lrmoe.plan_quota_device(E, torch.from_numpy(ids).to(U.DEV), policy)
        torch.cuda.synchronize()
        valid = ids[(ids >= 0) & (ids < E)]
        counts = np.bincount(valid, minlength=E).astype(np.int64)
        q = np.array(O.plan_quota(counts.tolist(), policy), dtype=np.int64)
        assert np.array_equal(out["counts"].cpu().numpy(), counts)
        assert np.array_equal(out["quotas"].cpu().numpy(), q)
        assert np.array_equal(out["seg_offsets"].cpu().numpy(), np.concatenate([[0], np.cumsum(q)]))
        assert int(out["invalid"].cpu()[0]) == n - valid.size


def test_whole_path_in_a_hip_graph():
    """The one-call path captured in a HIP graph (the library launches only
    kernels on the caller's stream: no allocation, no memset, no host sync)
    and replayed several times, with eager work and synchronisations in
    between: every replay equals the eager result bit for bit."""
    p = W.make_problem(P=3000, E=5, d_out=264, d_in=200, dtype="bf16",
                       counts=[1400, 0, 977, 7, 616], seed=361, policy=("ratio", 4, 5))
    q = lrmoe.plan_quota(p.counts, p.policy)
    plan = lrmoe.Plan(p.counts, q, p.d_out, p.d_in, lrmoe.BF16)
    t = dict(alpha=U.dev(p.alpha), g=U.dev(p.g), phi=U.dev(p.phi), W=U.dev(p.W))
    ws = lrmoe.workspace(plan, U.DEV)
    eager = lrmoe.pruned_backward(plan, t["alpha"], t["g"], t["phi"], t["W"], ws=ws)
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in eager.items()}
    out = {k: torch.empty_like(v) for k, v in eager.items()}
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # warm-up on the capture stream
        lrmoe.pruned_backward(plan, t["alpha"], t["g"], t["phi"], t["W"], out=out, ws=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        lrmoe.pruned_backward(plan, t["alpha"], t["g"], t["phi"], t["W"], out=out, ws=ws)
    for r in range(3):
        for v in out.values():
            v.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k, v in ref.items():
            a, b = v, out[k]
            if a.dtype == torch.bfloat16:
                a, b = a.view(torch.int16), b.view(torch.int16)
            assert torch.equal(a, b), (r, k)
        # eager work between replays, on the same buffers' inputs
        lrmoe.pruned_backward(plan, t["alpha"], t["g"], t["phi"], t["W"], ws=ws)
        torch.cuda.synchronize()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_gather_backward_token_rows(dtype):
    """lrmoe_gather_backward with the second projection's input gathered
    through a row index (x is one row per token, g2 one row per pair), in both
    storage types: bit for bit the separate gather + grouped-backward calls,
    which the oracle checks."""
    p = W.make_token_problem(T=700, E=6, topk=2, d_out=48, d_in=40, dtype=dtype, seed=371,
                             policy=("ratio", 3, 4))
    q = lrmoe.plan_quota(p.counts, p.policy)
    plan, out, t = U.run_gpu(p, q)
    rng = np.random.default_rng(371)
    d2o, d2i = 96, 56
    mk = (lambda a: W.to_bf16_bits(a)) if dtype == "bf16" else (lambda a: a.astype(np.float32))
    g2 = mk(rng.standard_normal((p.P, d2o)).astype(np.float32))
    x = mk(rng.standard_normal((p.T, d2i)).astype(np.float32))
    W2 = mk((0.02 * rng.standard_normal((p.E, d2o, d2i))).astype(np.float32))
    plan2 = lrmoe.Plan(p.counts, q, d2o, d2i, U.dtype_code(p), T=p.P)
    rows = t["row"]
    c2 = lrmoe.gather_compact(plan2, out["perm"], out["keep"], t["alpha"], U.dev(g2), U.dev(x),
                              phi_row_index=rows)
    dW2 = lrmoe.grouped_backward(plan2, out["perm"], c2["alpha_c"], c2["g_c"], c2["phi_c"],
                                 U.dev(W2), dphi=c2["dphi"])
    one = lrmoe.gather_backward(plan2, out["perm"], out["keep"], t["alpha"], U.dev(g2), U.dev(x),
                                U.dev(W2), phi_row_index=rows)
    torch.cuda.synchronize()
    assert torch.equal(one["dW"], dW2) and torch.equal(one["dphi"], c2["dphi"])
    for k in ("g_c", "phi_c", "alpha_c"):
        a, b = one[k], c2[k]
        if a.dtype == torch.bfloat16:
            a, b = a.view(torch.int16), b.view(torch.int16)
        assert torch.equal(a, b), k
    # and the oracle: x rows of the kept pairs' tokens, the second projection's dW and dx
    perm = out["perm"].cpu().numpy()
    seg = out["seg_offsets"].cpu().numpy()
    xr = x[p.row_index.astype(np.int64)]          # x per pair
    ref_dW = O.weight_grad(seg, p.alpha[perm], g2[perm], xr[perm], dtype, p.E, d2o, d2i)
    ref_dx = O.input_grad(seg, perm, p.alpha[perm], g2[perm], W2, dtype, p.P)
    assert U.rel_err(one["dW"].cpu().numpy(), ref_dW) <= U.TOL
    assert U.rel_err(one["dphi"].cpu().numpy(), ref_dx) <= U.TOL


def test_timer_leaves_no_hip_error_for_unlaunched_kernels():
    """Given scores skip the score kernel, so its timing events are never
    recorded.  Reading their duration fails inside HIP; that failure must not
    stay behind for the next torch launch check to report."""
    p = W.make_problem(P=600, E=3, d_out=64, d_in=32, dtype="bf16", counts=[250, 50, 300], seed=21)
    plan = lrmoe.Plan(p.counts, [200, 40, 240], p.d_out, p.d_in, lrmoe.BF16)
    timer = lrmoe.KernelTimer(1)
    try:
        lrmoe.score_select_compact(plan, U.dev(p.alpha), U.dev(p.g), U.dev(p.phi),
                                   scores=U.dev(W.random_scores(p.P, 5)), timing=timer)
        torch.cuda.synchronize()
        assert timer.durations_us(0) == []        # score slot: kernel not launched
        assert len(timer.durations_us(1)) == 1    # select
        x = torch.empty(4096, device="cuda:0")
        x.fill_(2.0)                              # a torch launch checks HIP's last error
        torch.cuda.synchronize()
        assert float(x.sum()) == 8192.0
    finally:
        timer.close()


@pytest.mark.parametrize("dw_mode", [lrmoe.DW_F16, lrmoe.DW_BF16])
def test_half_weight_gradient_edge_tiles(dw_mode):
    """A last column of at most 128 columns (d_in = 1088 = 4 x 256 + 64) with
    one operand plane per side: the weight-gradient tiles of that column are
    256 x 128 (float16 mode with both sides wider than 1024, or single
    rounding).  Expert 0 keeps more than one K chunk, so its half tiles also
    write split-K partial tiles."""
    counts = [2000, 700, 300]
    p = W.make_problem(P=sum(counts), E=3, d_out=1152, d_in=1088, dtype="bf16", counts=counts,
                       seed=91)
    q = lrmoe.plan_quota(p.counts, ("ratio", 4, 5))
    print(f"half dW edge tiles: mode {dw_mode} quotas={q}", flush=True)
    _, out, _ = U.run_gpu(p, q, dw_mode=dw_mode)
    errs, _ = U.compare_full(p, q, out, dw_mode=dw_mode)
    print("half dW edge tiles", errs)


@pytest.mark.parametrize("dtype,d_out,d_in", [("f32", 68, 36), ("bf16", 72, 264)])
def test_epilogue_column_edges(dtype, d_out, d_in):
    """Matrix edges inside the epilogue's 16-column store groups: the last
    tile column holds 4 (float32) or 8 (bfloat16) columns, so in each lane
    pair only some lanes' quads are inside the matrix, for both rows of the
    pair; one expert spans two row tiles."""
    counts = [450, 250]
    p = W.make_problem(P=sum(counts), E=2, d_out=d_out, d_in=d_in, dtype=dtype, counts=counts,
                       seed=77)
    q = lrmoe.plan_quota(p.counts, ("ratio", 4, 5))
    print(f"edges: {dtype} d_out={d_out} d_in={d_in} quotas={q}", flush=True)
    _, out, _ = U.run_gpu(p, q)
    U.compare_full(p, q, out)


@pytest.mark.parametrize("dtype,dw_mode,d_out,d_in", [
    # four column tiles, the last one 32 wide: 3 x 4 groups (an odd number of
    # row tiles per group) with tall 512 x 128 edge tiles of both products in
    # the exact mode, and five row tiles of dW (the last tall dW tile covers a
    # row tile past d_out)
    ("bf16", lrmoe.DW_EXACT, 1280, 800),
    # eight column tiles: 3 x 4 groups, float16 dW converted in registers
    ("bf16", lrmoe.DW_F16, 1024, 2048),
    # six column tiles (the GLM width): 4 x 3 groups, both float16 planes,
    # half dW and tall input-gradient edge tiles
    ("bf16", lrmoe.DW_F16, 2048, 1408),
    # sixteen column tiles, single rounding
    ("bf16", lrmoe.DW_BF16, 768, 4096),
])
def test_group_shapes(dtype, dw_mode, d_out, d_in):
    """Tile groups of every shape the schedule picks for wide problems, with a
    split-K expert (expert 0 keeps more rows than one K chunk)."""
    counts = [3000, 900, 250]
    p = W.make_problem(P=sum(counts), E=3, d_out=d_out, d_in=d_in, dtype=dtype, counts=counts,
                       seed=d_out + d_in)
    q = lrmoe.plan_quota(p.counts, ("ratio", 4, 5))
    print(f"group shapes: mode {dw_mode} d_out={d_out} d_in={d_in} quotas={q}", flush=True)
    _, out, _ = U.run_gpu(p, q, dw_mode=dw_mode)
    errs, _ = U.compare_full(p, q, out, dw_mode=dw_mode)
    print("group shapes", errs)
