"""lrmoe_score_select_compact_noalloc (no workspace argument: the selection
scratch is the library's static device array) against
lrmoe_score_select_compact with a caller workspace, on two calls in a row,
the second smaller, both with experts above 24576 pairs so that the scratch
is used (the chunked passes' digit histograms, select state and chunk
counts).  Results must be bit
for bit the same: both run the same kernels on the same inputs."""
import numpy as np
import pytest
import torch

from pruned_expert_backward_amd import lrmoe
from pruned_expert_backward_amd import workloads as W
from tests import gpu_util as U

pytestmark = pytest.mark.gpu
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

CASES = [  # first call, then a smaller one on the same GPU
    dict(P=70000, E=3, d_out=64, d_in=40, counts=[52000, 13000, 5000], seed=901),
    dict(P=36000, E=2, d_out=32, d_in=24, counts=[27000, 9000], seed=902),
]


def _same(a, b, what):
    if a.dtype == torch.bfloat16:
        a, b = a.view(torch.int16), b.view(torch.int16)
    assert torch.equal(a, b), what


def test_noalloc_matches_workspace_call_twice():
    for i, kw in enumerate(CASES):
        p = W.make_problem(dtype="bf16", **kw)
        q = lrmoe.plan_quota(p.counts, ("ratio", 4, 5))
        plan = lrmoe.Plan(p.counts, q, p.d_out, p.d_in, lrmoe.BF16)
        print(f"noalloc call {i}: P={p.P} counts={list(p.counts)} M={sum(q)}", flush=True)
        alpha, g, phi = U.dev(p.alpha), U.dev(p.g), U.dev(p.phi)
        ref = lrmoe.score_select_compact(plan, alpha, g, phi)
        ref["dphi"].fill_(7.0)
        ref = lrmoe.score_select_compact(plan, alpha, g, phi, out=ref)
        got = lrmoe.alloc_select_outputs(plan, alpha.device)
        got["dphi"].fill_(7.0)   # rows of kept pairs are left alone, dropped ones zeroed
        lrmoe.score_select_compact_noalloc(plan, alpha, g, phi, out=got)
        torch.cuda.synchronize()
        for k in ("scores", "keep", "seg_offsets", "perm", "g_c", "phi_c", "alpha_c", "dphi"):
            _same(got[k], ref[k], (i, k))
        keep = got["keep"].cpu().numpy().astype(bool)
        assert int(keep.sum()) == sum(q)
        d = got["dphi"].cpu().numpy()
        assert np.all(d[~keep] == 0) and np.all(d[keep] == 7.0)
