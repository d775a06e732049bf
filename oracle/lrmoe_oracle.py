"""CPU oracle for LRMoE's pruned MoE expert backward -- TEST INFRASTRUCTURE.

Only the test suite, the smoke check and the CPU-baseline leg of the benchmark
may import this module.  The product path (the HIP library and its Python
binding) never calls it, and this module imports nothing from the product.

It is a plain, slow, step-by-step restatement of what the pages describe,
in float64 arithmetic with exact Python/numpy integers for quotas and
indices.  Page titles used in citations:

  [EN] "LRMoE: Trimming Backward Work in Memory-Bound MoE Training"
       (aimodeling.com news article, English text).
  [PT] "LRMoE poda a passagem reversa do MoE e acelera o treinamento em 21-45%"
       (news.hamidun.com, Portuguese write-up).

Steps, in the pages' order:
  plan_quota      quota q_e per expert, fixed before the backward
                  ([EN] "Backward demand is not a constant"; [PT] bullet
                  "Cotas antes do calculo").
  lrm_scores      R_u = alpha_u^2 * ||g_t||^2 * ||phi_u||^2
                  ([EN] "LRM: a decomposable contribution score").
  gradient_scores the ablation baselines ||g_t||^2 and sum_i |g_t,i|
                  ([EN] "What the measurements show").
  select_top_quota  per expert, keep the q_e highest-scoring pairs
                  ([PT] bullet "Selecao pela metrica LRM").
  compact         pack kept rows into contiguous expert segments
                  ([EN] "The part that is easy to get wrong"; [PT] bullet
                  "Compactacao fisica").
  weight_grad     dW_e = sum over kept u of (alpha_u g_t) phi_u^T
                  ([EN] "LRM: ..." defines the per-pair outer product).
  input_grad      dphi_u = alpha_u W_e^T g_t for kept u, zero for dropped u,
                  in the original pair layout ([PT] "Compactacao fisica":
                  the result goes back to the original layout afterwards).
  silu_glu_grad   the expert MLP's activation backward between the down and
                  the gate/up projection, phi = SiLU(a) * b; the pages imply
                  this step without spelling it out.  On the compacted
                  layout (glu_chain_grad) it feeds the gate/up projection's
                  backward on the same keep set.

Readings where the pages are silent (each also listed in the design notes):
  * quota rounding: q_e = floor(n_e * num / den) for a keep ratio num/den,
    or floor(n_e * Q / P) for a budget of Q pairs over P routed pairs;
  * ties in R go to the lower original pair index;
  * segments in ascending expert id, ascending pair index inside a segment;
  * dropped pairs contribute nothing: their dphi rows are zero;
  * the routing weight enters the MLP chain once: the gate/up output gradient
    is formed from W_e^T g before alpha, and the gate/up backward applies
    alpha, as for a projection whose output gradient is given pre-alpha;
  * that gate/up output gradient goes on to the gate/up backward as the
    exact float64 value: the pages fix no storage rounding for it (they only
    say the result returns to the original layout afterwards, [PT]
    "Compactacao fisica").

Pins: every function here is checked in tests/test_oracle_pins.py against
something other than itself (brute force of the definition, the pages'
worked example, autograd of the dense layer, algebraic identities).  The
budget quota rule is a reading (the pages give a budget but no formula for
sharing it); its implementation is pinned by the properties every
proportional share of a fixed budget has and by the pages' figures for the
workload's budget, not by a value the pages print for it.
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np


# ---------------------------------------------------------------- storage

def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of stored inputs: bfloat16 bit patterns (uint16)
    are widened by placing them in the top half of a float32."""
    if dtype == "bf16":
        assert a.dtype == np.uint16
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if dtype == "f64":   # values the oracle itself produced
        assert a.dtype == np.float64
        return a
    assert a.dtype == np.float32
    return a.astype(np.float64)


# ---------------------------------------------------------------- a0: quota

def plan_quota(counts: Sequence[int], policy: tuple) -> list:
    """Per-expert backward retention quota, fixed before the backward.

    ("ratio", num, den): keep floor(n_e * num / den) pairs -- C-level Cx keeps
    (100 - x)/100 of each expert's pairs ([EN] "What the measurements show"
    names C0..C30 by the fraction of backward pairs dropped).
    ("budget", Q): a fixed number Q of pairs for the layer call, shared in
    proportion to demand, q_e = floor(n_e * Q / P)."""
    n = [int(c) for c in counts]
    assert all(c >= 0 for c in n)
    if policy[0] == "ratio":
        num, den = int(policy[1]), int(policy[2])
        assert den > 0 and 0 <= num <= den
        q = [(c * num) // den for c in n]
    elif policy[0] == "budget":
        Q, P = int(policy[1]), sum(n)
        assert Q >= 0
        q = [c if P == 0 else min(c, (c * Q) // P) for c in n]
    else:
        raise ValueError(policy)
    return q


# ---------------------------------------------------------------- a1: score

def lrm_scores(alpha, g, phi, row_index, dtype, block_rows: int = 4096) -> np.ndarray:
    """R_u = alpha_u^2 * ||g_t(u)||_2^2 * ||phi_u||_2^2 for every pair u.

    This is the squared Frobenius norm of the rank-one per-pair weight
    gradient (alpha_u g_t) phi_u^T, factorised ([EN] "LRM: a decomposable
    contribution score")."""
    P = phi.shape[0]
    a = alpha.astype(np.float64)
    gsq = np.empty(g.shape[0])
    for lo in range(0, g.shape[0], block_rows):
        gb = to_f64(g[lo:lo + block_rows], dtype)
        gsq[lo:lo + block_rows] = np.einsum("ij,ij->i", gb, gb)
    psq = np.empty(P)
    for lo in range(0, P, block_rows):
        pb = to_f64(phi[lo:lo + block_rows], dtype)
        psq[lo:lo + block_rows] = np.einsum("ij,ij->i", pb, pb)
    rows = np.arange(P) if row_index is None else row_index.astype(np.int64)
    assert np.all(np.isfinite(a)) and np.all(np.isfinite(gsq)) and np.all(np.isfinite(psq))
    return a * a * gsq[rows] * psq


def gradient_scores(g, row_index, dtype, P: int, rule: str, block_rows: int = 4096) -> np.ndarray:
    """Ablation baselines that score a pair by its upstream gradient alone
    ([EN] "What the measurements show": squared gradient norm and absolute
    gradient magnitude).  rule "sqnorm": ||g_t||_2^2.  rule "l1": the sum of
    |g_t,i| -- read as the L1 norm, since the Euclidean norm ranks pairs
    exactly like its square."""
    assert rule in ("sqnorm", "l1")
    v = np.empty(g.shape[0])
    for lo in range(0, g.shape[0], block_rows):
        gb = to_f64(g[lo:lo + block_rows], dtype)
        v[lo:lo + block_rows] = (np.einsum("ij,ij->i", gb, gb) if rule == "sqnorm"
                                 else np.abs(gb).sum(axis=1))
    rows = np.arange(P) if row_index is None else row_index.astype(np.int64)
    assert np.all(np.isfinite(v))
    return v[rows]


def pair_scores(mode: str, alpha, g, phi, row_index, dtype) -> np.ndarray:
    """Scores of the selectable rules: "lrm" (the method) or a gradient-only
    ablation ("sqnorm", "l1")."""
    if mode == "lrm":
        return lrm_scores(alpha, g, phi, row_index, dtype)
    return gradient_scores(g, row_index, dtype, phi.shape[0], mode)


# ---------------------------------------------------------------- a2: select

def select_top_quota(scores: np.ndarray, counts, quotas):
    """Per expert, keep the q_e pairs with the highest score; equal scores
    are ordered by ascending pair index.  Returns (keep bool[P],
    tau list): tau[e] is the score of the q_e-th kept pair (None when
    q_e is 0)."""
    P = scores.shape[0]
    keep = np.zeros(P, dtype=bool)
    taus = []
    lo = 0
    for n, q in zip(counts, quotas):
        n, q = int(n), int(q)
        assert 0 <= q <= n
        idx = np.arange(lo, lo + n)
        order = np.lexsort((idx, -scores[lo:lo + n]))   # by (-R, u)
        chosen = idx[order[:q]]
        keep[chosen] = True
        taus.append(float(scores[chosen[-1]]) if q > 0 else None)
        lo += n
    assert lo == P
    return keep, taus


# ---------------------------------------------------------------- a3: compact

def compact(keep: np.ndarray, counts, quotas):
    """Kept pair indices packed per expert (ascending expert, ascending pair
    index inside), and the segment offsets [0, q_0, q_0+q_1, ...]."""
    perm, seg = [], [0]
    lo = 0
    for n, q in zip(counts, quotas):
        kept = lo + np.nonzero(keep[lo:lo + int(n)])[0]      # ascending u
        assert len(kept) == int(q)
        perm.append(kept)
        seg.append(seg[-1] + len(kept))
        lo += int(n)
    perm = np.concatenate(perm) if perm else np.zeros(0)
    return perm.astype(np.int64), np.array(seg, dtype=np.int64)


def gather(perm, row_index, g, phi, alpha):
    """The compacted buffers: rows of g and phi and entries of alpha of the
    kept pairs, in segment order.  Pure copies of the stored values."""
    rows = perm if row_index is None else row_index.astype(np.int64)[perm]
    return g[rows], phi[perm], alpha[perm]


# ---------------------------------------------------------------- a4/a5: GEMMs

def weight_grad(seg, alpha_c, g_c, phi_c, dtype, E: int, d_out: int, d_in: int):
    """dW_e = sum over the kept pairs j of expert e of (alpha_j g_j) phi_j^T,
    i.e. G_e^T diag(alpha) Phi_e; zero for an expert that keeps nothing."""
    dW = np.zeros((E, d_out, d_in))
    for e in range(E):
        s, t = int(seg[e]), int(seg[e + 1])
        if t > s:
            ga = alpha_c[s:t].astype(np.float64)[:, None] * to_f64(g_c[s:t], dtype)
            dW[e] = ga.T @ to_f64(phi_c[s:t], dtype)
    return dW


def input_grad(seg, perm, alpha_c, g_c, W, dtype, P: int):
    """dphi_u = alpha_u W_e^T g_t for kept pairs, written back at the pair's
    original row; rows of dropped pairs stay zero."""
    E, d_out, d_in = W.shape
    dphi = np.zeros((P, d_in))
    for e in range(E):
        s, t = int(seg[e]), int(seg[e + 1])
        if t > s:
            rows = to_f64(g_c[s:t], dtype) @ to_f64(W[e], dtype)
            dphi[perm[s:t]] = alpha_c[s:t].astype(np.float64)[:, None] * rows
    return dphi


# ---------------------------------------------------------------- SiLU-GLU chain

def silu_glu_grad(dphi, a, b) -> np.ndarray:
    """Backward of phi = SiLU(a) * b (SiLU(a) = a sigmoid(a)) for float64
    rows: with s = sigmoid(a), d phi/d a = b s (1 + a (1 - s)) and
    d phi/d b = SiLU(a).  Returns [dL/da | dL/db], gate part first."""
    s = 1.0 / (1.0 + np.exp(-a))
    return np.concatenate([dphi * b * s * (1.0 + a * (1.0 - s)), dphi * a * s], axis=1)


def glu_chain_grad(seg, perm, g_c, W, a, b, dtype) -> np.ndarray:
    """Gate/up output gradient of every kept pair, in segment order: row j
    (pair u = perm[j] of expert e) is silu_glu_grad(W_e^T g_j, a_u, b_u),
    before the routing weight.  a, b [P, d_in] are the pair's saved gate and
    up pre-activations."""
    E, d_out, d_in = W.shape
    out = np.zeros((len(perm), 2 * d_in))
    for e in range(E):
        s, t = int(seg[e]), int(seg[e + 1])
        if t > s:
            u = perm[s:t]
            dphi = to_f64(g_c[s:t], dtype) @ to_f64(W[e], dtype)
            out[s:t] = silu_glu_grad(dphi, to_f64(a[u], dtype), to_f64(b[u], dtype))
    return out


# ---------------------------------------------------------------- whole path

def pruned_backward(counts, policy, alpha, g, phi, W, row_index, dtype,
                    with_grads: bool = True, gate_up=None, score_mode: str = "lrm",
                    glu=None) -> dict:
    """plan -> score -> select -> compact -> dW, dphi (and, when gate_up =
    (g2, x, W2) is given, the second projection's dW and dx on the same keep
    set and permutation).  score_mode picks the scoring rule (pair_scores).
    glu = (a, b, x, W2) chains the MLP instead: the gate/up output gradient
    of the kept pairs comes from the down projection through the SiLU-GLU
    backward (dgu_c, compacted) and drives the gate/up projection's dW2 and
    dx; x [P, d_model] is the hidden state each pair saw and W2 [E, 2 d_in,
    d_model] stacks the gate rows over the up rows."""
    E, d_out, d_in = W.shape
    P = phi.shape[0]
    q = plan_quota(counts, policy)
    R = pair_scores(score_mode, alpha, g, phi, row_index, dtype)
    keep, taus = select_top_quota(R, counts, q)
    perm, seg = compact(keep, counts, q)
    out = dict(quotas=q, scores=R, keep=keep, taus=taus, perm=perm, seg=seg)
    if with_grads:
        g_c, phi_c, alpha_c = gather(perm, row_index, g, phi, alpha)
        out["dW"] = weight_grad(seg, alpha_c, g_c, phi_c, dtype, E, d_out, d_in)
        out["dphi"] = input_grad(seg, perm, alpha_c, g_c, W, dtype, P)
        if gate_up is not None:
            g2, x, W2 = gate_up
            g2_c, x_c, _ = gather(perm, None, g2, x, alpha)
            out["dW2"] = weight_grad(seg, alpha_c, g2_c, x_c, dtype, E, W2.shape[1], W2.shape[2])
            out["dx"] = input_grad(seg, perm, alpha_c, g2_c, W2, dtype, P)
        if glu is not None:
            a, b, x, W2 = glu
            dgu_c = glu_chain_grad(seg, perm, g_c, W, a, b, dtype)
            out["dgu_c"] = dgu_c
            out["dW2"] = weight_grad(seg, alpha_c, dgu_c, to_f64(x[perm], dtype), "f64", E,
                                     W2.shape[1], W2.shape[2])
            out["dx"] = input_grad(seg, perm, alpha_c, dgu_c, to_f64(W2, dtype), "f64", P)
    return out


# ---------------------------------------------------------------- sampled outputs

def weight_grad_block(seg, perm, row_index, alpha, g, phi, dtype, e: int,
                      o_idx, i_idx) -> np.ndarray:
    """dW_e[o_idx][:, i_idx] for large problems: the same sum over the kept
    pairs of expert e, restricted to the requested rows and columns."""
    s, t = int(seg[e]), int(seg[e + 1])
    o_idx, i_idx = np.asarray(o_idx), np.asarray(i_idx)
    if t == s:
        return np.zeros((len(o_idx), len(i_idx)))
    u = perm[s:t]
    rows = u if row_index is None else row_index.astype(np.int64)[u]
    ga = alpha[u].astype(np.float64)[:, None] * to_f64(g[rows][:, o_idx], dtype)
    return ga.T @ to_f64(phi[u][:, i_idx], dtype)


def input_grad_rows(counts, keep, row_index, alpha, g, W, dtype, pairs) -> np.ndarray:
    """dphi for the requested original pair indices (zero rows for dropped
    pairs)."""
    offs = np.concatenate([[0], np.cumsum(np.asarray(counts, dtype=np.int64))])
    out = np.zeros((len(pairs), W.shape[2]))
    expert = np.searchsorted(offs, np.asarray(pairs, dtype=np.int64), side="right") - 1
    for e in np.unique(expert):
        We = to_f64(W[e], dtype)
        for k in np.nonzero(expert == e)[0]:
            u = int(pairs[k])
            if not keep[u]:
                continue
            r = u if row_index is None else int(row_index[u])
            out[k] = float(alpha[u]) * (We.T @ to_f64(g[r], dtype))
    return out


def _expert_of_rows(seg, js) -> np.ndarray:
    return np.searchsorted(np.asarray(seg, dtype=np.int64), np.asarray(js, dtype=np.int64),
                           side="right") - 1


def glu_chain_rows(seg, perm, row_index, g, W, a, b, dtype, js) -> np.ndarray:
    """Rows js of the compacted gate/up output gradient (glu_chain_grad),
    each computed on its own from the original-layout inputs."""
    out = np.zeros((len(js), 2 * W.shape[2]))
    for k, (j, e) in enumerate(zip(js, _expert_of_rows(seg, js))):
        u = int(perm[j])
        r = u if row_index is None else int(row_index[u])
        dphi = to_f64(g[r:r + 1], dtype) @ to_f64(W[e], dtype)
        out[k] = silu_glu_grad(dphi, to_f64(a[u:u + 1], dtype), to_f64(b[u:u + 1], dtype))[0]
    return out


def glu_weight_grad_block(seg, perm, row_index, alpha, g, W, a, b, x, dtype, e: int,
                          o_idx, i_idx) -> np.ndarray:
    """dW2_e[o_idx][:, i_idx] of the chained gate/up projection: the sum over
    expert e's kept pairs of alpha_u dgu_u[o] x_u[i], with only the needed
    gate/up columns of dgu formed (gate column c and up column c both need
    column c of W_e^T g)."""
    s, t = int(seg[e]), int(seg[e + 1])
    o_idx, i_idx = np.asarray(o_idx), np.asarray(i_idx)
    if t == s:
        return np.zeros((len(o_idx), len(i_idx)))
    d_in = W.shape[2]
    u = perm[s:t]
    rows = u if row_index is None else row_index.astype(np.int64)[u]
    cols = np.unique(o_idx % d_in)
    dphi = to_f64(g[rows], dtype) @ to_f64(W[e][:, cols], dtype)
    full = silu_glu_grad(dphi, to_f64(a[u][:, cols], dtype), to_f64(b[u][:, cols], dtype))
    pos = np.searchsorted(cols, o_idx % d_in) + np.where(o_idx >= d_in, len(cols), 0)
    ga = alpha[u].astype(np.float64)[:, None] * full[:, pos]
    return ga.T @ to_f64(x[u][:, i_idx], dtype)


def glu_input_grad_rows(counts, keep, row_index, alpha, g, W, a, b, W2, dtype, pairs) -> np.ndarray:
    """dx of the chained gate/up projection for the requested original pair
    indices: alpha_u W2_e^T dgu_u, zero rows for dropped pairs."""
    offs = np.concatenate([[0], np.cumsum(np.asarray(counts, dtype=np.int64))])
    out = np.zeros((len(pairs), W2.shape[2]))
    expert = np.searchsorted(offs, np.asarray(pairs, dtype=np.int64), side="right") - 1
    for k, (u, e) in enumerate(zip(pairs, expert)):
        u = int(u)
        if not keep[u]:
            continue
        r = u if row_index is None else int(row_index[u])
        dphi = to_f64(g[r:r + 1], dtype) @ to_f64(W[e], dtype)
        dgu = silu_glu_grad(dphi, to_f64(a[u:u + 1], dtype), to_f64(b[u:u + 1], dtype))
        out[k] = float(alpha[u]) * (to_f64(W2[e], dtype).T @ dgu[0])
    return out
