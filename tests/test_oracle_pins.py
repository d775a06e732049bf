"""Pins of the CPU oracle to facts outside itself (CPU only).

Each check_* function takes the oracle module so that the mutation tests at
the end can hand it a copy with one planted mistake and confirm that some
check fails.  Sources (page titles):
  [EN] "LRMoE: Trimming Backward Work in Memory-Bound MoE Training"
  [PT] "LRMoE poda a passagem reversa do MoE e acelera o treinamento em 21-45%"
"""
import itertools
import json
import os
import types

import numpy as np
import pytest
import torch

from oracle import lrmoe_oracle as O
from pruned_expert_backward_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def tiny(seed, dtype="f32", E=3, P=None, T=None, d_out=6, d_in=5, counts=None,
         policy=("ratio", 80, 100)):
    if T is not None:
        return W.make_token_problem(T=T, E=E, topk=2, d_out=d_out, d_in=d_in,
                                    dtype=dtype, policy=policy, seed=seed)
    return W.make_problem(P=P or sum(counts), E=E, d_out=d_out, d_in=d_in, dtype=dtype,
                          counts=counts, policy=policy, seed=seed)


def run(orc, p, policy=None, gate_up=None):
    return orc.pruned_backward(p.counts, policy or p.policy, p.alpha, p.g, p.phi, p.W,
                               p.row_index, p.dtype, gate_up=gate_up)


# ------------------------------------------------------------------ checks

def check_quota_example(orc):
    """The pages' figure: loads [4,2,3] become [3,1,2] ([EN] "The part that is
    easy to get wrong"), read as C20 with floor."""
    ex = json.load(open(os.path.join(GOLDEN, "quota_example.json")))
    assert orc.plan_quota(ex["counts"], tuple(ex["policy"])) == ex["quotas"]
    # The same example end to end: segment lengths equal the quotas.
    p = tiny(7, counts=ex["counts"], E=3)
    out = run(orc, p, policy=tuple(ex["policy"]))
    assert np.diff(out["seg"]).tolist() == ex["quotas"]
    # C0 drops nothing.
    assert orc.plan_quota([5, 0, 17, 1], ("ratio", 100, 100)) == [5, 0, 17, 1]


def check_budget_quota(orc):
    """The budget rule (a reading: the pages fix a token-buffer budget for the
    20x batch-pressure run, [EN] "What the measurements show", but give no
    formula for sharing it) against the properties any proportional share of
    a fixed budget must have, on exact integers: no expert keeps more than it
    routed; the kept total never exceeds the budget and loses less than one
    pair per expert to rounding; every expert keeps the same fraction of its
    pairs up to that rounding; a budget of every routed pair is the dense
    backward and an empty budget keeps nothing.  Plus the budget of the
    655 360-pair workload priced from the pages' figures (the fixed-ownership
    token buffer of 12.46 GiB for the 32 768 pairs of a normal step, 8192
    tokens x 4 microbatches per GPU, scaled to 24 GiB)."""
    rng = np.random.default_rng(5)
    cases = [[4, 2, 3], [0, 7, 0, 19, 1], [286057, 8823, 6455, 5898], [1] * 9, [0, 0]]
    cases += [list(rng.integers(0, 400, size=int(rng.integers(1, 12)))) for _ in range(40)]
    for counts in cases:
        counts = [int(c) for c in counts]
        P = sum(counts)
        for Q in sorted({0, 1, P // 7, P // 2, max(P - 1, 0), P, P + 5, 3 * P + 1}):
            q = orc.plan_quota(counts, ("budget", Q))
            assert len(q) == len(counts)
            assert all(0 <= a <= n for a, n in zip(q, counts))
            if Q >= P:   # the budget covers every routed pair: the dense backward
                assert q == counts
                continue
            assert sum(q) <= Q and Q - sum(q) < len([n for n in counts if n > 0])
            for a, n in zip(q, counts):   # a / n = Q / P up to one pair: a <= nQ/P < a + 1
                assert a * P <= n * Q < (a + 1) * P
            if Q == 0:
                assert q == [0] * len(counts)
    # the workload's budget, from the pages' 12.46 GiB at 32 768 pairs
    per_pair_gib = 12.46 / (8192 * 4)
    assert W.GLM45_20X_BUDGET_PAIRS == int(24 / per_pair_gib + 1e-9)
    p4_counts = W.zipf_counts(655360, 16, 1.4, 1004)
    q4 = orc.plan_quota(p4_counts, ("budget", W.GLM45_20X_BUDGET_PAIRS))
    assert W.GLM45_20X_BUDGET_PAIRS - 16 < sum(q4) <= W.GLM45_20X_BUDGET_PAIRS
    # "most experts are cut well beyond 20 %": every expert keeps under 10 %
    assert all(a < 0.1 * n for a, n in zip(q4, p4_counts))


def check_score_bruteforce(orc):
    """R_u equals the squared Frobenius norm of the materialised rank-one
    gradient (alpha_u g_t) phi_u^T ([EN] "LRM: a decomposable contribution
    score")."""
    for dtype in ("f32", "bf16"):
        p = tiny(11, dtype=dtype, T=9, E=4, d_out=7, d_in=16)
        R = orc.lrm_scores(p.alpha, p.g, p.phi, p.row_index, p.dtype)
        gf = O_exact(p.g, dtype)
        pf = O_exact(p.phi, dtype)
        for u in range(p.P):
            t = int(p.row_index[u])
            G = np.zeros((p.d_out, p.d_in))
            for i in range(p.d_out):
                for j in range(p.d_in):
                    G[i, j] = float(p.alpha[u]) * gf[t][i] * pf[u][j]
            ref = sum(G[i, j] ** 2 for i in range(p.d_out) for j in range(p.d_in))
            assert abs(R[u] - ref) <= 1e-12 * ref


def O_exact(a, dtype):
    """Exact values of stored arrays, decoded independently of the oracle:
    a bf16 pattern b has value (-1)^s * 2^(exp-127) * (1 + m/128)."""
    if dtype == "f32":
        return [[float(v) for v in row] for row in a]
    out = []
    for row in a:
        vals = []
        for b in row:
            b = int(b)
            s, ex, m = b >> 15, (b >> 7) & 0xFF, b & 0x7F
            assert ex != 0xFF
            v = (m / 128.0) * 2.0 ** -126 if ex == 0 else (1 + m / 128.0) * 2.0 ** (ex - 127)
            vals.append(-v if s else v)
        out.append(vals)
    return out


def check_gradient_scores(orc):
    """The ablation baselines ([EN] "What the measurements show"): squared
    gradient norm and absolute gradient magnitude (L1), by brute force over
    independently decoded values, through the per-token row index."""
    for dtype in ("f32", "bf16"):
        p = tiny(13, dtype=dtype, T=9, E=4, d_out=7, d_in=16)
        gf = O_exact(p.g, dtype)
        sq = orc.pair_scores("sqnorm", p.alpha, p.g, p.phi, p.row_index, p.dtype)
        l1 = orc.pair_scores("l1", p.alpha, p.g, p.phi, p.row_index, p.dtype)
        for u in range(p.P):
            row = gf[int(p.row_index[u])]
            ref_sq = sum(v * v for v in row)
            ref_l1 = sum(abs(v) for v in row)
            assert abs(sq[u] - ref_sq) <= 1e-12 * ref_sq
            assert abs(l1[u] - ref_l1) <= 1e-12 * ref_l1
        # the method's rule through the same dispatcher
        assert np.array_equal(orc.pair_scores("lrm", p.alpha, p.g, p.phi, p.row_index, p.dtype),
                              orc.lrm_scores(p.alpha, p.g, p.phi, p.row_index, p.dtype))


def check_select_bruteforce(orc):
    """Within a quota the highest-scoring pairs are kept ([PT] "Selecao pela
    metrica LRM"): the kept set maximises the additive objective sum R over
    all subsets of size q; among optimal subsets (ties) the lowest indices."""
    rng = np.random.default_rng(5)
    for trial in range(60):
        n = int(rng.integers(0, 11))
        vals = rng.integers(0, 4, size=n).astype(np.float64) if trial % 2 else rng.random(n)
        for q in range(n + 1):
            keep, taus = orc.select_top_quota(vals, [n], [q])
            best = None
            for sub in itertools.combinations(range(n), q):
                key = (-sum(vals[list(sub)]), sub)
                if best is None or key < best:
                    best = key
            assert sorted(np.nonzero(keep)[0].tolist()) == list(best[1])
            if 0 < q < n:
                assert vals[keep].min() >= vals[~keep].max()
                assert taus[0] == vals[keep].min()
    # All-equal scores keep the first q indices of every expert.
    keep, _ = orc.select_top_quota(np.ones(9), [4, 0, 5], [2, 0, 3])
    assert np.nonzero(keep)[0].tolist() == [0, 1, 4, 5, 6]


def check_compact_invariants(orc):
    """Kept rows packed per expert, unpadded ([EN] "The part that is easy to
    get wrong"): lengths = quotas, offsets = exclusive prefix sums, ascending
    pair index inside a segment, rows copied bit for bit."""
    p = tiny(3, dtype="bf16", E=5, counts=[9, 0, 13, 1, 6], d_out=8, d_in=16)
    out = run(orc, p)
    q = out["quotas"]
    assert out["seg"].tolist() == np.concatenate([[0], np.cumsum(q)]).tolist()
    offs = p.offsets
    for e in range(p.E):
        s, t = out["seg"][e], out["seg"][e + 1]
        seg = out["perm"][s:t]
        assert np.all(np.diff(seg) > 0)
        assert np.all((seg >= offs[e]) & (seg < offs[e + 1]))
    assert out["keep"].sum() == out["seg"][-1] and np.all(out["keep"][out["perm"]])
    g_c, phi_c, a_c = orc.gather(out["perm"], p.row_index, p.g, p.phi, p.alpha)
    for j, u in enumerate(out["perm"]):
        assert np.array_equal(g_c[j], p.g[u]) and np.array_equal(phi_c[j], p.phi[u])
        assert a_c[j] == p.alpha[u]


def dense_autograd(p, alpha_override=None, gate_up=False):
    """torch.autograd (float64) of the dense expert layer
    y_t = sum over pairs u of token t of alpha_u W_e(u) phi_u with upstream
    gradient g_t: returns dL/dW and dL/dphi."""
    E = p.E
    if gate_up:
        gsrc, phisrc, Wsrc = p.gate_up.g2, p.gate_up.x, p.gate_up.W2
    else:
        gsrc, phisrc, Wsrc = p.g, p.phi, p.W
    f = lambda a: torch.tensor(np.array(O_exact(a.reshape(-1, a.shape[-1]), p.dtype)),
                               dtype=torch.float64).reshape(a.shape)
    Wt = f(Wsrc).requires_grad_(True)
    phi = f(phisrc).requires_grad_(True)
    g = f(gsrc)
    alpha = torch.tensor(p.alpha if alpha_override is None else alpha_override, dtype=torch.float64)
    e_of_u = torch.tensor(np.repeat(np.arange(E), p.counts))
    rows = torch.arange(p.P) if p.row_index is None else torch.tensor(p.row_index.astype(np.int64))
    contrib = alpha[:, None] * torch.einsum("pij,pj->pi", Wt[e_of_u], phi)
    y = torch.zeros(g.shape[0], g.shape[1], dtype=torch.float64).index_add(0, rows, contrib)
    (y * g).sum().backward()
    return Wt.grad.numpy(), phi.grad.numpy()


def check_dense_equivalence(orc):
    """(i) With q = n (C0) the pruned backward is the dense backward of the
    layer; (ii) with a real quota it equals the dense backward with the
    routing weight of dropped pairs set to 0 -- the zero-masking the pages
    contrast with compaction ([EN] "The part that is easy to get wrong")."""
    for dtype, kw in (("f32", dict(T=10, E=4)), ("bf16", dict(counts=[5, 0, 7, 2], E=4))):
        p = tiny(21, dtype=dtype, d_out=6, d_in=5, **kw)
        full = run(orc, p, policy=("ratio", 1, 1))
        dW, dphi = dense_autograd(p)
        assert np.abs(full["dW"] - dW).max() <= 1e-12 * np.abs(dW).max()
        assert np.abs(full["dphi"] - dphi).max() <= 1e-12 * np.abs(dphi).max()
        cut = run(orc, p, policy=("ratio", 3, 5))
        assert cut["keep"].sum() < p.P
        dWm, dphim = dense_autograd(p, alpha_override=np.where(cut["keep"], p.alpha, 0.0))
        assert np.abs(cut["dW"] - dWm).max() <= 1e-12 * np.abs(dWm).max()
        assert np.abs(cut["dphi"] - dphim).max() <= 1e-12 * np.abs(dphim).max()
        assert np.all(cut["dphi"][~cut["keep"]] == 0)


def check_drop_identities(orc):
    """dW_kept = dW_dense - sum over dropped pairs of G_u, and the Frobenius
    error of pruning is at most sum over dropped pairs of sqrt(R_u)
    (triangle inequality on the rank-one terms)."""
    p = tiny(33, dtype="bf16", E=3, counts=[8, 6, 9], d_out=8, d_in=8)
    full = run(orc, p, policy=("ratio", 1, 1))
    cut = run(orc, p, policy=("ratio", 1, 2))
    gf, pf = np.array(O_exact(p.g, "bf16")), np.array(O_exact(p.phi, "bf16"))
    offs = p.offsets
    err_bound = 0.0
    acc = full["dW"].copy()
    for u in np.nonzero(~cut["keep"])[0]:
        e = int(np.searchsorted(offs, u, side="right") - 1)
        acc[e] -= float(p.alpha[u]) * np.outer(gf[u], pf[u])
        err_bound += np.sqrt(cut["scores"][u])
    assert np.abs(acc - cut["dW"]).max() <= 1e-12 * np.abs(full["dW"]).max()
    assert np.linalg.norm(full["dW"] - cut["dW"]) <= err_bound * (1 + 1e-12)


def check_gate_up_inherits(orc):
    """The second projection reuses the keep set: with q = n it is the dense
    backward of h = W2 x, and dropped pairs get zero input gradient."""
    p = W.make_problem(P=14, E=3, d_out=6, d_in=5, dtype="bf16", counts=[6, 3, 5],
                       seed=44, gate_up=(4, 7))
    gu = (p.gate_up.g2, p.gate_up.x, p.gate_up.W2)
    full = run(orc, p, policy=("ratio", 1, 1), gate_up=gu)
    dW2, dx = dense_autograd(p, gate_up=True)
    assert np.abs(full["dW2"] - dW2).max() <= 1e-12 * np.abs(dW2).max()
    assert np.abs(full["dx"] - dx).max() <= 1e-12 * np.abs(dx).max()
    cut = run(orc, p, policy=("ratio", 1, 2), gate_up=gu)
    dW2m, dxm = dense_autograd(p, alpha_override=np.where(cut["keep"], p.alpha, 0.0), gate_up=True)
    assert np.abs(cut["dW2"] - dW2m).max() <= 1e-12 * np.abs(dW2m).max()
    assert np.abs(cut["dx"] - dxm).max() <= 1e-12 * np.abs(dxm).max()


def _mlp_moe(seed, T=10, E=3, topk=2, d_model=7, d_in=5, d_out=6):
    """Token-routed expert MLP in float64: routing from the workload
    generator, x, W_gate, W_up, W_down, g drawn here."""
    p = W.make_token_problem(T=T, E=E, topk=topk, d_out=d_out, d_in=d_in, seed=seed)
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, d_model))
    Wg = 0.5 * rng.standard_normal((E, d_in, d_model))
    Wu = 0.5 * rng.standard_normal((E, d_in, d_model))
    Wd = 0.5 * rng.standard_normal((E, d_out, d_in))
    g = rng.standard_normal((T, d_out))
    e_of_u = np.repeat(np.arange(E), p.counts)
    xt = x[p.row_index.astype(np.int64)]                       # hidden state of each pair
    a = np.einsum("pij,pj->pi", Wg[e_of_u], xt)
    b = np.einsum("pij,pj->pi", Wu[e_of_u], xt)
    phi = a / (1.0 + np.exp(-a)) * b
    return p, x, xt, Wg, Wu, Wd, g, a, b, phi, e_of_u


def _mlp_autograd(p, x, Wg, Wu, Wd, g, e_of_u, alpha):
    """torch.autograd (float64) of y_t = sum over pairs u of token t of
    alpha_u W_down,e (SiLU(W_gate,e x_t) * (W_up,e x_t)), loss sum(y * g)."""
    t = lambda v: torch.tensor(v, dtype=torch.float64, requires_grad=True)
    xt, Wgt, Wut, Wdt = t(x), t(Wg), t(Wu), t(Wd)
    eu = torch.tensor(e_of_u)
    rows = torch.tensor(p.row_index.astype(np.int64))
    h = xt[rows]
    a = torch.einsum("pij,pj->pi", Wgt[eu], h)
    b = torch.einsum("pij,pj->pi", Wut[eu], h)
    phi = torch.nn.functional.silu(a) * b
    contrib = torch.tensor(alpha, dtype=torch.float64)[:, None] * torch.einsum(
        "pij,pj->pi", Wdt[eu], phi)
    y = torch.zeros(x.shape[0], Wd.shape[1], dtype=torch.float64).index_add(0, rows, contrib)
    (y * torch.tensor(g)).sum().backward()
    return (Wdt.grad.numpy(), np.concatenate([Wgt.grad.numpy(), Wut.grad.numpy()], axis=1),
            xt.grad.numpy())


def check_glu_chain_autograd(orc):
    """The chained MLP backward (down -> SiLU-GLU -> gate/up on the compacted
    layout): with q = n it is torch.autograd of the routed expert MLP, the
    token's input gradient being the sum of its pairs' dx; with a real quota
    it is the same autograd with the routing weight of dropped pairs set to 0,
    and dropped pairs get zero dx.  Gate rows come first in W2."""
    p, x, xt, Wg, Wu, Wd, g, a, b, phi, e_of_u = _mlp_moe(51)
    W2 = np.concatenate([Wg, Wu], axis=1)
    tok = p.row_index.astype(np.int64)
    for policy in (("ratio", 1, 1), ("ratio", 1, 2)):
        out = orc.pruned_backward(p.counts, policy, p.alpha, g, phi, Wd, p.row_index, "f64",
                                  glu=(a, b, xt, W2))
        keep = out["keep"]
        if policy[1] != policy[2]:
            assert 0 < keep.sum() < p.P
        dWd, dW2, dx = _mlp_autograd(p, x, Wg, Wu, Wd, g, e_of_u, np.where(keep, p.alpha, 0.0))
        assert np.abs(out["dW"] - dWd).max() <= 1e-12 * np.abs(dWd).max()
        assert np.abs(out["dW2"] - dW2).max() <= 1e-12 * np.abs(dW2).max()
        dx_tok = np.zeros_like(x)
        np.add.at(dx_tok, tok, out["dx"])
        assert np.abs(dx_tok - dx).max() <= 1e-12 * np.abs(dx).max()
        assert np.all(out["dx"][~keep] == 0)
        assert out["dgu_c"].shape == (int(keep.sum()), 2 * a.shape[1])


def check_glu_chain_sampled(orc):
    """The sampled chain helpers agree with the full chain."""
    p = W.make_problem(P=60, E=3, d_out=16, d_in=8, counts=[30, 5, 25], gate_up=(16, 12),
                       glu=True, seed=8)
    gu, gl = p.gate_up, p.glu
    out = orc.pruned_backward(p.counts, ("ratio", 3, 4), p.alpha, p.g, p.phi, p.W, None,
                              p.dtype, glu=(gl.a, gl.b, gu.x, gu.W2))
    o_idx, i_idx = [0, 3, 9, 15], [2, 11]
    for e in range(p.E):
        blk = orc.glu_weight_grad_block(out["seg"], out["perm"], None, p.alpha, p.g, p.W,
                                        gl.a, gl.b, gu.x, p.dtype, e, o_idx, i_idx)
        assert np.allclose(blk, out["dW2"][e][np.ix_(o_idx, i_idx)], rtol=1e-13, atol=1e-300)
    js = [0, 7, len(out["perm"]) - 1]
    rows = orc.glu_chain_rows(out["seg"], out["perm"], None, p.g, p.W, gl.a, gl.b, p.dtype, js)
    assert np.allclose(rows, out["dgu_c"][js], rtol=1e-13, atol=0)
    pairs = [0, 4, 31, 36, 59]
    dx = orc.glu_input_grad_rows(p.counts, out["keep"], None, p.alpha, p.g, p.W, gl.a, gl.b,
                                 gu.W2, p.dtype, pairs)
    assert np.allclose(dx, out["dx"][pairs], rtol=1e-13, atol=0)


def check_sampled_match_full(orc):
    """The sampled-output helpers agree with the full computation."""
    p = tiny(9, dtype="bf16", E=4, counts=[30, 0, 17, 21], d_out=24, d_in=16)
    out = run(orc, p)
    o_idx, i_idx = [0, 5, 23], [1, 15]
    for e in range(p.E):
        blk = orc.weight_grad_block(out["seg"], out["perm"], p.row_index, p.alpha, p.g, p.phi,
                                    p.dtype, e, o_idx, i_idx)
        assert np.allclose(blk, out["dW"][e][np.ix_(o_idx, i_idx)], rtol=1e-13, atol=0)
    pairs = [0, 3, 31, 50, 67]
    rows = orc.input_grad_rows(p.counts, out["keep"], p.row_index, p.alpha, p.g, p.W, p.dtype, pairs)
    assert np.allclose(rows, out["dphi"][pairs], rtol=1e-13, atol=0)


CHECKS = [check_quota_example, check_budget_quota, check_score_bruteforce, check_gradient_scores,
          check_select_bruteforce,
          check_compact_invariants, check_dense_equivalence, check_drop_identities,
          check_gate_up_inherits, check_glu_chain_autograd, check_glu_chain_sampled,
          check_sampled_match_full]


@pytest.mark.parametrize("check", CHECKS, ids=lambda c: c.__name__)
def test_oracle_pin(check):
    check(O)


def test_workload_counts_and_ranges():
    """Generator sanity: exact Zipf counts and the expected value ranges."""
    c = W.zipf_counts(32768, 16, 1.6, 0)
    assert c.sum() == 32768 and sorted(c)[-1] == 16584
    p = W.config(0)
    assert p.P == 512 and p.counts.sum() == 512 and p.g.shape == (256, 64)
    # Routing weights of a top-2 softmax pair sum to 1 per token.
    s = np.zeros(256)
    np.add.at(s, p.row_index, p.alpha)
    assert np.allclose(s, 1.0, atol=1e-6)


# ------------------------------------------------------------------ mutations

def _mutant(**overrides):
    """A copy of the oracle module with some functions replaced; the copied
    oracle functions resolve names in the copy, so internal calls reach the
    replacements."""
    m = types.ModuleType("oracle_mutant")
    for k, v in O.__dict__.items():
        if k.startswith("__"):
            continue
        if isinstance(v, types.FunctionType):
            v = types.FunctionType(v.__code__, m.__dict__, v.__name__, v.__defaults__,
                                   v.__closure__)
        m.__dict__[k] = v
    m.__dict__.update(overrides)
    return m


def _scores_alpha_not_squared(alpha, g, phi, row_index, dtype, block_rows=4096):
    return O.lrm_scores(alpha, g, phi, row_index, dtype) / np.maximum(alpha.astype(np.float64), 1e-30)


def _scores_no_phi(alpha, g, phi, row_index, dtype, block_rows=4096):
    a = alpha.astype(np.float64)
    gg = to_f64(g, dtype)
    rows = np.arange(phi.shape[0]) if row_index is None else row_index.astype(np.int64)
    return a * a * (gg * gg).sum(1)[rows]


def _select_keep_lowest(scores, counts, quotas):
    return O.select_top_quota(-scores, counts, quotas)


def _select_tie_high(scores, counts, quotas):
    P = scores.shape[0]
    keep, taus = O.select_top_quota(scores[::-1].copy(), counts[::-1], quotas[::-1])
    return keep[::-1].copy(), taus[::-1]


def _input_grad_wrong_expert(seg, perm, alpha_c, g_c, W, dtype, P):
    return O.input_grad(seg, perm, alpha_c, g_c, np.roll(W, 1, axis=0), dtype, P)


def _weight_grad_no_alpha(seg, alpha_c, g_c, phi_c, dtype, E, d_out, d_in):
    return O.weight_grad(seg, np.ones_like(alpha_c), g_c, phi_c, dtype, E, d_out, d_in)


def _compact_unsorted(keep, counts, quotas):
    perm, seg = O.compact(keep, counts, quotas)
    out = perm.copy()
    for e in range(len(seg) - 1):
        out[seg[e]:seg[e + 1]] = out[seg[e]:seg[e + 1]][::-1]
    return out, seg


def _quota_round(counts, policy):
    if policy[0] == "ratio":
        return [min(int(c), int(round(c * policy[1] / policy[2]))) for c in counts]
    return O.plan_quota(counts, policy)


def _quota_budget_ceil(counts, policy):
    if policy[0] == "budget":
        Q, P = int(policy[1]), int(sum(counts))
        return [int(c) if P == 0 else min(int(c), -(-int(c) * Q // P)) for c in counts]
    return O.plan_quota(counts, policy)


def _quota_budget_even(counts, policy):
    if policy[0] == "budget":
        per = int(policy[1]) // max(len(counts), 1)
        return [min(int(c), per) for c in counts]
    return O.plan_quota(counts, policy)


def _input_grad_keep_dropped_rows(seg, perm, alpha_c, g_c, W, dtype, P):
    d = O.input_grad(seg, perm, alpha_c, g_c, W, dtype, P)
    d[d == 0] = 1e-3
    return d


to_f64 = O.to_f64


def _gradient_scores_l1_squares(g, row_index, dtype, P, rule, block_rows=4096):
    return O.gradient_scores(g, row_index, dtype, P, "sqnorm", block_rows)


def _gradient_scores_unsquared(g, row_index, dtype, P, rule, block_rows=4096):
    v = O.gradient_scores(g, row_index, dtype, P, rule, block_rows)
    return np.sqrt(v) if rule == "sqnorm" else v

def _glu_derivative_is_sigmoid(dphi, a, b):
    s = 1.0 / (1.0 + np.exp(-a))
    return np.concatenate([dphi * b * s, dphi * a * s], axis=1)


def _glu_halves_swapped(dphi, a, b):
    d = a.shape[1]
    r = O.silu_glu_grad(dphi, a, b)
    return np.concatenate([r[:, d:], r[:, :d]], axis=1)


def _glu_up_uses_b(dphi, a, b):
    r = O.silu_glu_grad(dphi, a, b)
    r[:, a.shape[1]:] = dphi * b
    return r


def _glu_chain_transposed_ab(seg, perm, g_c, W, a, b, dtype):
    return O.glu_chain_grad(seg, perm, g_c, W, b, a, dtype)


def _glu_chain_rounded_handoff(seg, perm, g_c, W, a, b, dtype):
    # the gate/up output gradient rounded to 8 significant bits on the way
    # to the gate/up backward (a storage rounding nothing on the pages fixes)
    out = O.glu_chain_grad(seg, perm, g_c, W, a, b, dtype)
    m, e = np.frexp(out)
    return np.ldexp(np.round(m * 256.0) / 256.0, e)


MUTANTS = {
    "score_alpha_not_squared": dict(lrm_scores=_scores_alpha_not_squared),
    "score_drops_phi_term": dict(lrm_scores=_scores_no_phi),
    "select_keeps_lowest": dict(select_top_quota=_select_keep_lowest),
    "select_tie_to_higher_index": dict(select_top_quota=_select_tie_high),
    "dphi_wrong_expert_weight": dict(input_grad=_input_grad_wrong_expert),
    "dW_drops_alpha": dict(weight_grad=_weight_grad_no_alpha),
    "perm_descending": dict(compact=_compact_unsorted),
    "quota_rounds": dict(plan_quota=_quota_round),
    "budget_rounds_up": dict(plan_quota=_quota_budget_ceil),
    "budget_split_evenly": dict(plan_quota=_quota_budget_even),
    "dropped_rows_nonzero": dict(input_grad=_input_grad_keep_dropped_rows),
    "l1_rule_uses_squares": dict(gradient_scores=_gradient_scores_l1_squares),
    "sqnorm_rule_not_squared": dict(gradient_scores=_gradient_scores_unsquared),
    "glu_derivative_is_sigmoid": dict(silu_glu_grad=_glu_derivative_is_sigmoid),
    "glu_halves_swapped": dict(silu_glu_grad=_glu_halves_swapped),
    "glu_up_uses_b": dict(silu_glu_grad=_glu_up_uses_b),
    "glu_chain_swaps_a_b": dict(glu_chain_grad=_glu_chain_transposed_ab),
    "glu_handoff_rounded": dict(glu_chain_grad=_glu_chain_rounded_handoff),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    m = _mutant(**MUTANTS[name])
    failed = []
    for check in CHECKS:
        try:
            check(m)
        except (AssertionError, ValueError, IndexError):
            failed.append(check.__name__)
    assert failed, f"mutant {name} passed every pin"
