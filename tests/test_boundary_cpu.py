"""C-ABI library: loads, exports what include/lrmoe.h declares, plans quotas,
and rejects every host-detectable bad argument before launching anything.
CPU only: the calls below fail validation, so no kernel is launched."""
import ctypes as C
import os
import re

import pytest

from pruned_expert_backward_amd import lrmoe as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lrmoe.h")

if not os.path.exists(L.LIB_PATH):
    pytest.skip("liblrmoe.so not built (run __graft_entry__.build())", allow_module_level=True)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lrmoe_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    lib = L.lib()
    names = declared_functions()
    assert set(names) == set(L.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n
    assert lib.lrmoe_abi_version() == L.ABI_VERSION
    for s in range(9):
        assert lib.lrmoe_status_string(s)


def test_plan_quota_matches_pages_example_and_rules():
    assert L.plan_quota([4, 2, 3], ("ratio", 80, 100)) == [3, 1, 2]
    assert L.plan_quota([5, 0, 17, 1], ("ratio", 100, 100)) == [5, 0, 17, 1]
    assert L.plan_quota([1, 9, 10], ("ratio", 80, 100)) == [0, 7, 8]
    assert L.plan_quota([10, 30, 60], ("budget", 50)) == [5, 15, 30]
    assert L.plan_quota([10, 30, 60], ("budget", 1000)) == [10, 30, 60]
    # Large counts: exact integer arithmetic (no float products).
    n = [2**31 - 1, 3]
    assert L.plan_quota(n, ("ratio", 7, 9)) == [(2**31 - 1) * 7 // 9, 2]
    assert L.plan_quota(n, ("budget", 2**31 - 5)) == [
        (2**31 - 1) * (2**31 - 5) // (2**31 + 2), 3 * (2**31 - 5) // (2**31 + 2)]


def test_plan_quota_matches_oracle_on_workloads():
    from oracle import lrmoe_oracle as O
    from pruned_expert_backward_amd import workloads as W
    for c, spec in W.CONFIGS.items():
        counts = W.zipf_counts(spec.get("P", 512), spec["E"], spec.get("zipf", 1.0), 1000 + c)
        assert L.plan_quota(counts, spec["policy"]) == O.plan_quota(counts, spec["policy"])


@pytest.mark.parametrize("policy,code", [
    (L.QuotaPolicy(L.QUOTA_RATIO, 5, 4, 0), 2), (L.QuotaPolicy(L.QUOTA_RATIO, -1, 4, 0), 2),
    (L.QuotaPolicy(L.QUOTA_RATIO, 1, 0, 0), 2), (L.QuotaPolicy(L.QUOTA_BUDGET, 0, 1, -3), 2),
    (L.QuotaPolicy(7, 1, 1, 0), 2)])
def test_plan_quota_rejects_bad_policy(policy, code):
    cnt = (C.c_int64 * 3)(4, 2, 3)
    out = (C.c_int64 * 3)()
    assert L.lib().lrmoe_plan_quota(3, cnt, C.byref(policy), out) == code


def test_plan_quota_rejects_bad_counts():
    pol = L.QuotaPolicy(L.QUOTA_RATIO, 1, 2, 0)
    out = (C.c_int64 * 3)()
    assert L.lib().lrmoe_plan_quota(3, (C.c_int64 * 3)(4, -2, 3), C.byref(pol), out) == 2
    assert L.lib().lrmoe_plan_quota(0, (C.c_int64 * 3)(4, 2, 3), C.byref(pol), out) == 2
    assert L.lib().lrmoe_plan_quota(300, (C.c_int64 * 300)(), C.byref(pol), out) == 2
    assert L.lib().lrmoe_plan_quota(3, None, C.byref(pol), out) == 1


# A fake, 16-byte-aligned device address: validation fails before any use.
FAKE = 0x7F0000001000


def sscc(plan, **over):
    args = dict(row=None, alpha=FAKE, g=FAKE, phi=FAKE, scores=FAKE, keep=FAKE, seg=FAKE,
                perm=FAKE, g_c=FAKE, phi_c=FAKE, alpha_c=FAKE, dphi=None, ws=None, ws_bytes=0)
    args.update(over)
    return L.lib().lrmoe_score_select_compact(
        C.byref(plan.struct), args["row"], args["alpha"], args["g"], args["phi"], args["scores"],
        args["keep"], args["seg"], args["perm"], args["g_c"], args["phi_c"], args["alpha_c"],
        args["dphi"], args["ws"], args["ws_bytes"], None)


def plan(counts=(4, 2, 3), quotas=(3, 1, 2), d_out=16, d_in=8, dtype=L.BF16, **kw):
    return L.Plan(list(counts), list(quotas), d_out, d_in, dtype, **kw)


@pytest.mark.parametrize("mutate,code", [
    (lambda p: setattr(p.struct, "E", 0), 2),
    (lambda p: setattr(p.struct, "E", 257), 2),
    (lambda p: setattr(p.struct, "dtype", 9), 5),
    (lambda p: setattr(p.struct, "dw_mode", 3), 2),
    (lambda p: setattr(p.struct, "score_mode", 3), 2),
    (lambda p: setattr(p.struct, "score_mode", -1), 2),
    (lambda p: setattr(p.struct, "P", 8), 3),             # sum of counts != P
    (lambda p: setattr(p.struct, "P", 2**31), 3),
    (lambda p: setattr(p.struct, "d_out", 12), 4),        # not a multiple of 8 (bf16)
    (lambda p: setattr(p.struct, "d_in", 0), 3),
    (lambda p: setattr(p.struct, "counts", None), 1),
    (lambda p: setattr(p.struct, "quotas", None), 1),
])
def test_problem_validation(mutate, code):
    p = plan()
    mutate(p)
    assert sscc(p) == code


def test_quota_bounds_validation():
    assert sscc(plan(quotas=(5, 1, 2))) == 2          # q_e > n_e
    assert sscc(plan(quotas=(-1, 1, 2))) == 2         # q_e < 0
    assert sscc(plan(counts=(4, -2, 3))) == 2


def test_fp32_row_length_rule():
    # 12 % 4 == 0 passes the row rule, so the next check (alpha) reports.
    assert sscc(plan(dtype=L.F32, d_out=12, d_in=4), alpha=None) == 1
    assert sscc(plan(dtype=L.F32, d_out=10, d_in=4)) == 4


@pytest.mark.parametrize("field", ["alpha", "g", "phi", "scores", "keep", "seg", "perm", "g_c",
                                   "phi_c", "alpha_c"])
def test_null_and_misaligned_pointers(field):
    assert sscc(plan(), **{field: None}) == 1
    assert sscc(plan(), **{field: FAKE + 4}) == 4


def test_row_index_required_when_g_is_per_token():
    assert sscc(plan(T=5)) == 3
    assert sscc(plan(), row=FAKE + 8) == 4


def test_row_index_needs_rows_to_index():
    """With a g row index, g must have at least one row when any pair is
    read (T = 0 would let a NULL g through to the kernels); with a phi row
    index, phi's row count T_phi must be given when rows are gathered.  The
    index values themselves live on the device: the kernels bound them by T
    and T_phi (reading a zero row), which no CPU test can launch."""
    assert sscc(plan(T=0), row=FAKE) == 3
    assert sscc(plan(T=0), row=FAKE, g=None) == 3
    gc = L.lib().lrmoe_gather_compact
    # perm keep g_row phi_row alpha g phi g_c phi_c alpha_c dphi_zero stream
    ok = [FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None]
    p = plan(T=0)
    assert gc(C.byref(p.struct), *ok) == 3                  # g rows gathered, T = 0
    a = list(ok)
    a[3] = FAKE                                            # phi row index ...
    p = plan(T=4)
    p.struct.T_phi = 0
    assert gc(C.byref(p.struct), *a) == 3                  # ... with no phi rows
    p.struct.T_phi = 2**31
    assert gc(C.byref(p.struct), *a) == 3
    gb = L.lib().lrmoe_gather_backward
    p = plan(T=0)
    n = p.workspace_bytes()
    okb = [FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE,
           n, None]
    assert gb(C.byref(p.struct), *okb) == 3
    pb = L.lib().lrmoe_pruned_backward
    okp = [FAKE] + [FAKE] * 14 + [n, None]
    assert pb(C.byref(p.struct), *okp) == 3


def test_workspace_size_and_check():
    p = plan(counts=(40, 20, 30), quotas=(30, 10, 20), d_out=64, d_in=32)
    n = p.workspace_bytes()
    # exact mode, bf16: the plain grouped backward keeps alpha * phi (the
    # narrower operand) as hi + lo planes; the gate/up variant (float32 g_c)
    # alpha * g_c as hi + lo planes; no split-K partials at this size, then
    # the GEMM's queue counters (256 bytes) and the float16 mode's expert
    # maxima (2 floats for each of up to 256 experts).  One size serves every
    # call: the larger.
    heads = 256 + 2 * 256 * 4
    plane_phi = (60 * 32 * 2 + 255) // 256 * 256
    plane_g = (60 * 64 * 2 + 255) // 256 * 256
    assert select_bytes((40, 20, 30)) == 0   # small experts: the selection needs none
    assert n == max(2 * plane_phi, 2 * plane_g) + heads
    for f in (L.lib().lrmoe_grouped_backward, L.lib().lrmoe_grouped_backward_gate_up):
        assert f(C.byref(p.struct), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, n - 1,
                 None) == 6
        assert f(C.byref(p.struct), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, n, None) == 1
    p1 = plan(counts=(40, 20, 30), quotas=(30, 10, 20), d_out=64, d_in=32, dw_mode=L.DW_BF16)
    assert p1.workspace_bytes() == max(plane_phi, plane_g) + heads
    # float16 mode: counters and maxima, the score pass's per-pair row maxima
    # (8 bytes per routed pair), then the float16 plane of alpha * phi (the
    # narrower operand; the GEMM converts g_c in registers)
    p2 = plan(counts=(40, 20, 30), quotas=(30, 10, 20), d_out=64, d_in=32, dw_mode=L.DW_F16)
    f16 = (heads + 90 * 8 + 255) // 256 * 256 + plane_phi
    assert p2.workspace_bytes() == max(f16, 2 * plane_g + heads)
    # with the narrower operand wider than 1024, both float16 planes
    p3 = plan(counts=(40, 20, 30), quotas=(30, 10, 20), d_out=2048, d_in=1152, dw_mode=L.DW_F16)
    wide_g = (60 * 2048 * 2 + 255) // 256 * 256
    wide_phi = (60 * 1152 * 2 + 255) // 256 * 256
    f16 = (heads + 90 * 8 + 255) // 256 * 256 + wide_g + wide_phi
    assert p3.workspace_bytes() == max(f16, 2 * wide_g + heads)


def test_grouped_backward_gate_up_validation():
    """The MLP chain's gate/up call: bf16 x and W only (the float32 output
    gradient is the only float32 operand); the usual pointer rules."""
    f = L.lib().lrmoe_grouped_backward_gate_up
    p = plan()
    n = p.workspace_bytes()
    ok = [FAKE] * 6 + [None, FAKE, n, None]   # perm alpha_c dgu_c x_c W dW dx ws
    assert f(C.byref(plan(dtype=L.F32).struct), *ok) == 5
    for i in (1, 2, 3, 4, 5, 7):
        a = list(ok)
        a[i] = None
        assert f(C.byref(p.struct), *a) == 1, i
    a = list(ok)
    a[0], a[6] = None, FAKE        # perm needed when dx is requested
    assert f(C.byref(p.struct), *a) == 1
    a = list(ok)
    a[2] = FAKE + 4
    assert f(C.byref(p.struct), *a) == 4
    assert f(None, *ok) == 1


def select_bytes(counts):
    """The selection's workspace: none when every expert has at most 24576
    pairs (one workgroup per expert, keys in LDS); else, for the chunked
    passes, per expert two 4096-bin and one 256-bin digit histogram and 8
    words of select state, per 4096-pair chunk two counts (32-bit words)."""
    if max(counts) <= 24576:
        return 0
    chunks = sum((n + 4095) // 4096 for n in counts)
    return (len(counts) * (2 * 4096 + 256 + 8) + 2 * chunks) * 4


def test_select_workspace():
    """A problem with an expert above 24576 pairs is selected in chunked
    passes over 4096-pair chunks of every expert, which keep their digit
    histograms, state and chunk counts in the workspace: the selection calls
    then need that much.  Otherwise they need none."""
    counts, quotas = (60000, 24576, 100), (48000, 19660, 80)
    p = plan(counts=counts, quotas=quotas, d_out=8, d_in=8)
    sel = select_bytes(counts)
    assert sel == (3 * 8456 + 2 * (15 + 6 + 1)) * 4
    n = p.workspace_bytes()
    assert n >= sel
    assert sscc(p, ws=FAKE, ws_bytes=sel - 1) == 6
    assert sscc(p, ws=None, ws_bytes=sel) == 1
    assert sscc(p, ws=FAKE + 4, ws_bytes=sel) == 4
    # no expert above 24576 pairs: no workspace (the only error is the NULL alpha)
    assert sscc(plan(counts=(24576, 10), quotas=(10, 5), d_out=8, d_in=8), alpha=None,
                ws=None, ws_bytes=0) == 1
    assert sscc(plan(counts=(24576, 10), quotas=(10, 5), d_out=8, d_in=8), alpha=None,
                ws=FAKE + 4, ws_bytes=0) == 1   # and its alignment is not checked either


def test_grouped_backward_validation():
    p = plan()
    f = L.lib().lrmoe_grouped_backward
    args = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, None]
    for i, code in [(1, 1), (2, 1), (3, 1), (4, 1), (5, 1)]:
        a = list(args)
        a[i] = None
        assert f(C.byref(p.struct), *a) == code, i
    a = list(args)
    a[0], a[6] = None, FAKE        # perm needed when dphi is requested
    assert f(C.byref(p.struct), *a) == 1
    a = list(args)
    a[6] = FAKE + 2
    assert f(C.byref(p.struct), *a) == 4


def test_grouped_backward_glu_validation():
    """The SiLU-GLU chain entry point: bf16 only; the saved pre-activations,
    the gate/up output and perm are required; the usual workspace and
    alignment rules hold."""
    f = L.lib().lrmoe_grouped_backward_glu
    p = plan()
    n = p.workspace_bytes()
    ok = [FAKE] * 10 + [n, None]   # perm alpha_c g_c phi_c W dW act_a act_b dgu_c ws
    assert f(C.byref(plan(dtype=L.F32).struct), *ok) == 5
    for i in (0, 1, 2, 3, 4, 5, 6, 7, 8, 9):
        a = list(ok)
        a[i] = None
        assert f(C.byref(p.struct), *a) == 1, i
    for i in (6, 7, 8):
        a = list(ok)
        a[i] = FAKE + 4
        assert f(C.byref(p.struct), *a) == 4, i
    a = list(ok)
    a[10] = n - 1
    assert f(C.byref(p.struct), *a) == 6
    assert f(None, *ok) == 1


def test_pruned_backward_validation():
    """The whole-path call checks what its two steps check, before any launch."""
    f = L.lib().lrmoe_pruned_backward
    p = plan()
    n = p.workspace_bytes()
    # g_row_index alpha g phi W scores keep seg perm g_c phi_c alpha_c dW dphi ws
    ok = [None] + [FAKE] * 14 + [n, None]
    for i in (1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 14):   # 13: dphi may be NULL
        a = list(ok)
        a[i] = None
        assert f(C.byref(p.struct), *a) == 1, i
    a = list(ok)
    a[15] = n - 1
    assert f(C.byref(p.struct), *a) == 6
    a = list(ok)
    a[12] = FAKE + 4
    assert f(C.byref(p.struct), *a) == 4
    assert f(None, *ok) == 1


def test_gather_backward_validation():
    f = L.lib().lrmoe_gather_backward
    p = plan()
    n = p.workspace_bytes()
    # perm keep g_row phi_row alpha g phi W g_c phi_c alpha_c dW dphi ws
    ok = [FAKE, FAKE, None, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE,
          n, None]
    for i in (0, 4, 5, 6, 7, 8, 9, 10, 11, 13):   # g is required here (the GEMM reads g_c)
        a = list(ok)
        a[i] = None
        assert f(C.byref(p.struct), *a) == 1, i
    a = list(ok)
    a[14] = n - 1
    assert f(C.byref(p.struct), *a) == 6
    a = list(ok)
    a[1], a[12] = None, FAKE   # zero target needs the keep flags
    assert f(C.byref(p.struct), *a) == 1


def test_gather_compact_validation():
    p = plan()
    f = L.lib().lrmoe_gather_compact
    ok = [FAKE, FAKE, None, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None]
    for i in (0, 4, 5, 6, 7, 8, 9):
        a = list(ok)
        a[i] = None
        assert f(C.byref(p.struct), *a) == 1, i
    a = list(ok)
    a[1] = None
    a[10] = FAKE       # zero target needs the keep flags
    assert f(C.byref(p.struct), *a) == 1
    a = list(ok)
    a[5], a[7], a[8] = None, None, None   # g and g_c both NULL: phi rows only ...
    assert f(C.byref(p.struct), *a) == 1  # ... and phi_c is still required


def test_mask_alpha_and_score_select_validation():
    f = L.lib().lrmoe_mask_alpha
    assert f(-1, FAKE, FAKE, FAKE, None, None) == 3
    assert f(2**31, FAKE, FAKE, FAKE, None, None) == 3
    assert f(10, None, FAKE, FAKE, None, None) == 1
    assert f(10, FAKE, FAKE, FAKE + 4, None, None) == 4
    assert f(10, FAKE, FAKE, FAKE, FAKE + 8, None) == 4
    g = L.lib().lrmoe_score_select
    p = plan()
    # required: alpha, g, phi, scores, keep, seg_offsets, perm (compacted rows are not)
    args = [None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, None]
    for i in range(1, 8):
        a = list(args)
        a[i] = None
        assert g(C.byref(p.struct), *a) == 1, i


def test_plan_quota_device_validation():
    f = L.lib().lrmoe_plan_quota_device
    ok = L.QuotaPolicy(L.QUOTA_RATIO, 80, 100, 0)
    bad = L.QuotaPolicy(L.QUOTA_RATIO, 120, 100, 0)
    assert f(4, FAKE, 10, None, FAKE, FAKE, FAKE, None, None) == 1
    assert f(0, FAKE, 10, C.byref(ok), FAKE, FAKE, FAKE, None, None) == 2
    assert f(4, FAKE, 10, C.byref(bad), FAKE, FAKE, FAKE, None, None) == 2
    assert f(4, FAKE, -1, C.byref(ok), FAKE, FAKE, FAKE, None, None) == 3
    assert f(4, None, 10, C.byref(ok), FAKE, FAKE, FAKE, None, None) == 1
    assert f(4, FAKE, 10, C.byref(ok), FAKE + 4, FAKE, FAKE, None, None) == 4
    assert f(4, FAKE, 10, C.byref(ok), FAKE, FAKE, FAKE, FAKE + 8, None) == 4


def test_noalloc_rejects_problems_beyond_its_scratch():
    """The entry point without a workspace holds the selection scratch of the
    chunked passes in an 8 MiB static device buffer: a problem needing more
    (here 250 experts, one above 24576 pairs: 33 KiB of digit histograms and
    state each) is rejected before any HIP call; so are the usual bad
    arguments.  A 9-million-pair expert fits."""
    f = L.lib().lrmoe_score_select_compact_noalloc
    many = (30000,) + (4,) * 249
    assert select_bytes((9_000_000, 5)) <= 8 << 20 < select_bytes(many)
    big = plan(counts=many, quotas=(2,) * 250, d_out=8, d_in=8)
    args = [None] + [FAKE] * 11 + [None, None]   # row alpha g phi scores keep seg perm g_c phi_c alpha_c dphi
    assert f(C.byref(big.struct), *args) == 8
    assert L.lib().lrmoe_status_string(8)
    p = plan()
    a = list(args)
    a[1] = None                                   # alpha
    assert f(C.byref(p.struct), *a) == 1
    a = list(args)
    a[5] = FAKE + 4                               # keep misaligned
    assert f(C.byref(p.struct), *a) == 4
    assert f(None, *args) == 1
