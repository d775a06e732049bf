"""Seeded synthetic workloads for the pruned MoE expert backward.

This module only *draws inputs*: routing (expert counts and routing weights
alpha), upstream gradients g, saved projection inputs phi and expert weights
W.  It holds none of the method's arithmetic (no scores, quotas, selection,
compaction or gradients); the CPU oracle and the HIP path both consume what
it returns, and neither is imported here.

Shapes and distributions follow the one-GPU expert-parallel shares used to
evaluate LRMoE ("LRMoE: Trimming Backward Work in Memory-Bound MoE Training",
section "What the measurements show": Qwen3-30B-A3B and GLM4.5-106B-A12B,
BF16, sequence 8192, microbatch 4 per GPU, EP8).  The pages trained on a
preprocessed Alpaca corpus with real weights; neither is available, so these
seeded tensors of the same shapes stand in for them.

Recipe (all draws from numpy's PCG64, one stream per (seed, tensor, block)):
  * expert counts: truncated Zipf p_e ~ (rank+1)^-s over the local experts,
    exact integer counts by largest remainder (ties to the lower rank), and a
    seeded permutation decides which expert gets which rank;
  * alpha (bf16 configs): per pair, 128 N(0,1) router logits, keep the top 8,
    softmax over those 8, and take the weight of one of them chosen uniformly;
  * alpha (tiny config): per token, 8 N(0,1) logits, top-2 experts, softmax
    over the two selected logits;
  * g rows: N(0,1) elementwise times one lognormal(0, 0.5) factor per row;
  * phi: SiLU(z) with z ~ N(0,1) elementwise;
  * W: N(0, 0.02) elementwise;
  * MLP-chain variant: saved gate and up pre-activations a, b ~ N(0,1)
    elementwise (stored), and phi = SiLU(a) * b from the stored a, b in
    float32, then stored;
  * bf16 storage: draw in float32 and round to nearest even (kept as uint16
    bit patterns, since numpy has no bfloat16).
"""
from __future__ import annotations

import concurrent.futures as _fut
import dataclasses
import os
from typing import Optional

import numpy as np

BLOCK_ROWS = 2048  # rows per independent random stream (thread-count independent)

_TENSOR_IDS = {"counts": 1, "alpha": 2, "g": 3, "phi": 4, "W": 5,
               "g2": 6, "x": 7, "W2": 8, "route": 9, "scores": 10,
               "glu_a": 11, "glu_b": 12}


def _rng(seed: int, tensor: str, block: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(
        [int(seed), _TENSOR_IDS[tensor], int(block)])))


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); return uint16 bits.

    Inputs are finite by construction, so NaN handling is not needed."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def _workers() -> int:
    return max(1, min(16, os.cpu_count() or 1))


@dataclasses.dataclass
class GateUp:
    """Second projection sharing the first one's keep set (gate/up of the MLP).

    g2 [P, d_out] is the gradient w.r.t. the gate/up output *before* the
    routing weight (so alpha is applied once, by the backward), x [P, d_in]
    is the token hidden state each pair saw, W2 [E, d_out, d_in]."""
    d_out: int
    d_in: int
    g2: np.ndarray
    x: np.ndarray
    W2: np.ndarray


@dataclasses.dataclass
class Glu:
    """Saved pre-activations of the expert MLP phi = SiLU(a) * b, one row per
    pair: a (gate) and b (up), each [P, d_in] like phi."""
    a: np.ndarray
    b: np.ndarray


@dataclasses.dataclass
class Problem:
    name: str
    dtype: str                 # "bf16" (uint16 bit arrays) or "f32"
    E: int
    P: int
    T: int                     # rows of g
    d_out: int                 # length of g rows, rows of W_e
    d_in: int                  # length of phi rows, columns of W_e
    counts: np.ndarray         # int64 [E], pairs routed to each local expert
    row_index: Optional[np.ndarray]  # int32 [P] g row of each pair, None = identity
    alpha: np.ndarray          # float32 [P] routing weight of each pair
    g: np.ndarray              # [T, d_out]
    phi: np.ndarray            # [P, d_in]
    W: np.ndarray              # [E, d_out, d_in]
    policy: tuple              # ("ratio", num, den) or ("budget", pairs)
    gate_up: Optional[GateUp] = None
    glu: Optional[Glu] = None   # phi = SiLU(a) * b; gate_up.W2 stacks gate over up

    @property
    def offsets(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.counts)]).astype(np.int64)

    def nbytes(self) -> int:
        n = self.g.nbytes + self.phi.nbytes + self.W.nbytes + self.alpha.nbytes
        if self.gate_up is not None:
            n += self.gate_up.g2.nbytes + self.gate_up.x.nbytes + self.gate_up.W2.nbytes
        if self.glu is not None:
            n += self.glu.a.nbytes + self.glu.b.nbytes
        return n


def zipf_counts(P: int, E: int, s: float, seed: int) -> np.ndarray:
    """Exact per-expert counts for a truncated Zipf(s) law over E experts."""
    w = (np.arange(E, dtype=np.float64) + 1.0) ** (-float(s))
    raw = P * w / w.sum()
    base = np.floor(raw).astype(np.int64)
    rem = raw - base
    short = int(P - base.sum())
    order = sorted(range(E), key=lambda e: (-rem[e], e))
    for e in order[:short]:
        base[e] += 1
    perm = _rng(seed, "counts").permutation(E)
    counts = np.empty(E, dtype=np.int64)
    counts[perm] = base            # rank r goes to expert perm[r]
    return counts


def _fill_rows(out: np.ndarray, seed: int, tensor: str, make_block) -> None:
    """Fill out[rows] block by block, each block from its own stream."""
    n = out.shape[0]
    nblk = (n + BLOCK_ROWS - 1) // BLOCK_ROWS

    def work(b):
        lo, hi = b * BLOCK_ROWS, min(n, (b + 1) * BLOCK_ROWS)
        out[lo:hi] = make_block(_rng(seed, tensor, b), hi - lo)

    if nblk == 1:
        work(0)
        return
    with _fut.ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(work, range(nblk)))


def _store(x32: np.ndarray, dtype: str) -> np.ndarray:
    return to_bf16_bits(x32) if dtype == "bf16" else x32.astype(np.float32)


def _g_block(d: int, dtype: str):
    def mk(rng, rows):
        z = rng.standard_normal((rows, d), dtype=np.float32)
        s = np.exp(0.5 * rng.standard_normal((rows, 1), dtype=np.float32))
        return _store(z * s, dtype)
    return mk


def _phi_block(d: int, dtype: str):
    def mk(rng, rows):
        z = rng.standard_normal((rows, d), dtype=np.float32)
        return _store(z / (np.float32(1.0) + np.exp(-z)), dtype)
    return mk


def _normal_block(d: int, dtype: str, std: float):
    def mk(rng, rows):
        return _store(rng.standard_normal((rows, d), dtype=np.float32) * np.float32(std), dtype)
    return mk


def _alpha_topk_of_128(rng, rows):
    logits = rng.standard_normal((rows, 128))
    top = np.partition(logits, 120, axis=1)[:, 120:]          # the 8 largest
    w = np.exp(top - top.max(axis=1, keepdims=True))
    w /= w.sum(axis=1, keepdims=True)
    pick = rng.integers(0, 8, size=rows)
    return w[np.arange(rows), pick].astype(np.float32)


def _load(x: np.ndarray, dtype: str) -> np.ndarray:
    """float32 values of stored inputs (bf16 bits widened)."""
    if dtype == "bf16":
        return (x.astype(np.uint32) << np.uint32(16)).view(np.float32)
    return x


def _glu_forward(a32: np.ndarray, b32: np.ndarray) -> np.ndarray:
    """The MLP forward's activation, float32: SiLU(a) * b."""
    return a32 / (np.float32(1.0) + np.exp(-a32)) * b32


def _tensor(shape, dtype, seed, tensor, make_block):
    out = np.empty(shape, dtype=np.uint16 if dtype == "bf16" else np.float32)
    flat = out.reshape(-1, shape[-1])
    _fill_rows(flat, seed, tensor, make_block)
    return out


def make_problem(*, P: int, E: int, d_out: int, d_in: int, dtype: str = "bf16",
                 zipf: float = 1.2, counts=None, policy=("ratio", 80, 100),
                 seed: int = 0, name: str = "custom", gate_up=None, glu: bool = False) -> Problem:
    """Expert-sorted pairs with one g row per pair (the expert side's view
    after the expert-parallel dispatch).  glu=True (with gate_up = (2 d_in,
    d_model)) makes phi the SiLU-GLU of saved pre-activations, so that the
    down projection's input gradient chains into the gate/up projection."""
    if counts is None:
        counts = zipf_counts(P, E, zipf, seed)
    counts = np.asarray(counts, dtype=np.int64)
    assert counts.shape == (E,) and int(counts.sum()) == P
    alpha = np.empty((P, 1), dtype=np.float32)
    _fill_rows(alpha, seed, "alpha", lambda r, n: _alpha_topk_of_128(r, n)[:, None])
    alpha = alpha[:, 0].copy()
    g = _tensor((P, d_out), dtype, seed, "g", _g_block(d_out, dtype))
    W = _tensor((E, d_out, d_in), dtype, seed, "W", _normal_block(d_in, dtype, 0.02))
    gl = None
    if glu:
        assert gate_up is not None and gate_up[0] == 2 * d_in
        gl = Glu(_tensor((P, d_in), dtype, seed, "glu_a", _normal_block(d_in, dtype, 1.0)),
                 _tensor((P, d_in), dtype, seed, "glu_b", _normal_block(d_in, dtype, 1.0)))
        phi = _store(_glu_forward(_load(gl.a, dtype), _load(gl.b, dtype)), dtype)
    else:
        phi = _tensor((P, d_in), dtype, seed, "phi", _phi_block(d_in, dtype))
    gu = None
    if gate_up is not None:
        d2o, d2i = gate_up
        gu = GateUp(d2o, d2i,
                    _tensor((P, d2o), dtype, seed, "g2", _g_block(d2o, dtype)),
                    _tensor((P, d2i), dtype, seed, "x", _normal_block(d2i, dtype, 1.0)),
                    _tensor((E, d2o, d2i), dtype, seed, "W2", _normal_block(d2i, dtype, 0.02)))
    return Problem(name, dtype, E, P, P, d_out, d_in, counts, None, alpha, g, phi, W,
                   tuple(policy), gu, gl)


def make_token_problem(*, T: int, E: int, topk: int, d_out: int, d_in: int,
                       dtype: str = "f32", policy=("ratio", 80, 100), seed: int = 0,
                       name: str = "token") -> Problem:
    """Per-token routing: each of T tokens picks its top-k experts from N(0,1)
    logits (ties to the lower expert), alpha is the softmax over the k chosen
    logits, and g is one row per token shared by the token's k pairs."""
    rng = _rng(seed, "route")
    logits = rng.standard_normal((T, E))
    chosen = np.argsort(-logits, axis=1, kind="stable")[:, :topk]
    sel = np.take_along_axis(logits, chosen, axis=1)
    w = np.exp(sel - sel.max(axis=1, keepdims=True))
    w /= w.sum(axis=1, keepdims=True)
    tok = np.repeat(np.arange(T), topk)
    exp = chosen.reshape(-1)
    a = w.reshape(-1)
    order = np.lexsort((tok, exp))                 # expert-sorted, ascending token
    tok, exp, a = tok[order], exp[order], a[order]
    counts = np.bincount(exp, minlength=E).astype(np.int64)
    P = T * topk
    g = _tensor((T, d_out), dtype, seed, "g", _g_block(d_out, dtype))
    phi = _tensor((P, d_in), dtype, seed, "phi", _phi_block(d_in, dtype))
    W = _tensor((E, d_out, d_in), dtype, seed, "W", _normal_block(d_in, dtype, 0.02))
    return Problem(name, dtype, E, P, T, d_out, d_in, counts, tok.astype(np.int32),
                   a.astype(np.float32), g, phi, W, tuple(policy))


# Budget of config "glm45-20x": a fixed 24 GiB token buffer, priced at the
# per-pair token-buffer cost of the normal batch (12.46 GiB for 32768 pairs
# per GPU share, from the memory paragraph of "What the measurements show"):
# Q = floor(24 * 32768 / 12.46) pairs.
GLM45_20X_BUDGET_PAIRS = (24 * 32768 * 100) // 1246

CONFIGS = {
    0: dict(kind="token", name="tiny-fp32", T=256, E=8, topk=2, d_out=64, d_in=32,
            dtype="f32", policy=("ratio", 80, 100)),
    1: dict(kind="pairs", name="qwen3-30b-a3b-down-c20", P=32768, E=16, d_out=2048,
            d_in=768, dtype="bf16", zipf=1.2, policy=("ratio", 80, 100)),
    2: dict(kind="pairs", name="qwen3-30b-a3b-down-c30+gateup", P=32768, E=16,
            d_out=2048, d_in=768, dtype="bf16", zipf=1.6, policy=("ratio", 70, 100),
            gate_up=(1536, 2048)),
    3: dict(kind="pairs", name="glm45-106b-a12b-down-c20", P=32768, E=16, d_out=4096,
            d_in=1408, dtype="bf16", zipf=1.2, policy=("ratio", 80, 100)),
    4: dict(kind="pairs", name="glm45-106b-a12b-20x-budget", P=655360, E=16,
            d_out=4096, d_in=1408, dtype="bf16", zipf=1.4,
            policy=("budget", GLM45_20X_BUDGET_PAIRS)),
}


def config(c: int, glu: bool = False) -> Problem:
    """The named workload c (0 tiny fp32, 1-4 one-GPU shares), seed 1000+c.
    glu=True (config 2 only) draws the MLP-chain variant: phi from saved
    gate/up pre-activations, for the down -> SiLU-GLU -> gate/up chain."""
    spec = dict(CONFIGS[c])
    kind = spec.pop("kind")
    seed = 1000 + c
    if glu:
        assert "gate_up" in spec
        spec["glu"] = True
        spec["name"] = spec["name"] + "-glu-chain"
    if kind == "token":
        return make_token_problem(seed=seed, **spec)
    return make_problem(seed=seed, **spec)


def random_scores(n: int, seed: int, distinct: int = 0) -> np.ndarray:
    """Non-negative float32 scores for selection tests; distinct>0 draws from
    only that many values so that ties are frequent."""
    rng = _rng(seed, "scores")
    if distinct:
        vals = np.abs(rng.standard_normal(distinct)).astype(np.float32)
        vals[0] = 0.0
        return vals[rng.integers(0, distinct, size=n)]
    return (rng.standard_normal(n) ** 2).astype(np.float32)
