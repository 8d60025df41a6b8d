"""Host-side checks of the C-ABI library (no GPU needed): it loads, exports every entry point
include/cf.h declares, and rejects bad arguments before enqueuing anything."""
import ctypes
import os
import re

import pytest

import oracle
import synth
import selective_recompute_cf_amd as cf

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "cf.h")).read()
    return sorted(set(re.findall(r"\b(cf_[a-z_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(cf.LIB_PATH):
        from selective_recompute_cf_amd import build
        build.build()
    return cf.lib()


def test_library_exports_every_declared_symbol(L):
    names = _declared()
    assert len(names) >= 12
    for n in names:
        assert hasattr(L, n), n
    assert sorted(cf.EXPORTS) == names


def test_version_string(L):
    assert "gfx950" in cf.version()


def test_topk_validation(L):
    assert L.cf_topk_select(None, 10, 11, 0, None, 0, None, None, 0, None) == cf.CF_EINVAL
    assert "k" in L.cf_last_error().decode()
    assert L.cf_topk_select(None, 10, -1, 0, None, 0, None, None, 0, None) == cf.CF_EINVAL
    assert L.cf_topk_select(None, 10, 2, 7, None, 0, None, None, 0, None) == cf.CF_EINVAL
    # k = 0 enqueues nothing and succeeds
    assert L.cf_topk_select(None, 10, 0, 0, None, 0, None, None, 0, None) == cf.CF_OK
    # span bounds must start at 0, end at n and increase strictly
    for b in ([0, 5, 9], [1, 5, 10], [0, 5, 5, 10], [0, 12]):
        arr = (ctypes.c_int32 * len(b))(*b)
        assert L.cf_topk_select(None, 10, 0, 1, arr, len(b) - 1, None, None, 0, None) == cf.CF_EINVAL, b
    good = (ctypes.c_int32 * 3)(0, 4, 10)
    assert L.cf_topk_select(None, 10, 3, 1, good, 2, None, None, 0, None) == cf.CF_EWORKSPACE
    assert cf.topk_workspace_size(10, "doc") >= 88 and cf.topk_workspace_size(10, "token") == 0
    # token mode from n = 65536 on runs on the whole GPU and needs a workspace
    assert cf.topk_workspace_size(65535, "token") == 0 and cf.topk_workspace_size(65536, "token") > 0
    assert L.cf_topk_select(None, 1 << 20, 5, 0, None, 0, None, None, 0, None) == cf.CF_EWORKSPACE
    # from the minimum (the 2-bit map of the n values, per-range counts, 128 KB of sampled keys) up
    # any workspace is accepted; the rest holds candidates: a list of n / 16 and slices of 1 / 16
    # of each range at the full size
    for n in (1 << 16, 1 << 20, 3000017, (1 << 28) + 5):
        lo, hi = cf.topk_workspace_min_size(n, "token"), cf.topk_workspace_size(n, "token")
        assert n // 4 <= lo < n // 4 + (n // 1024) * 24 + (192 << 10) and hi >= lo + 4 * (n // 16) + 4 * (n // 16), n
    for mode in ("doc", "ranked", "heads"):
        assert cf.topk_workspace_min_size(1000, mode) == cf.topk_workspace_size(1000, mode)
    assert cf.topk_workspace_min_size(65535, "token") == 0
    # the no-allocation entry point holds the token-mode minimum (mostly the 2-bit map) up to about
    # 15.8 million values; beyond, it refuses on the host before anything is enqueued
    hdr = open(os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "cf.h")).read()
    assert "#define CF_NOALLOC_SCRATCH_BYTES (4u << 20)" in hdr and cf.CF_NOALLOC_SCRATCH_BYTES == 4 << 20
    big = 16_000_000
    assert cf.topk_workspace_min_size(big, "token") > cf.CF_NOALLOC_SCRATCH_BYTES
    assert L.cf_topk_select_noalloc(None, big, 5, 0, None, 0, None, None) == cf.CF_EWORKSPACE
    assert cf.topk_workspace_min_size(15_000_000, "token") <= cf.CF_NOALLOC_SCRATCH_BYTES
    assert L.cf_topk_select_noalloc(None, 15_000_000, 5, 0, None, 0, None, None) == cf.CF_EINVAL  # null values
    fake = ctypes.c_void_p(1 << 20)  # never dereferenced: both calls fail on the host
    lo = cf.topk_workspace_min_size(1 << 20, "token")
    assert L.cf_topk_select(None, 1 << 20, 5, 0, None, 0, None, fake, lo - 1, None) == cf.CF_EWORKSPACE
    assert L.cf_topk_select(None, 1 << 20, 5, 0, None, 0, None, fake, lo, None) == cf.CF_EINVAL  # null values


def test_deviation_validation(L):
    assert L.cf_kv_deviation(None, 5, 8, None, 0, 8, None, 4, 8, None) == cf.CF_EDTYPE
    assert L.cf_kv_deviation(None, 0, 8, None, 0, 8, None, 4, 12, None) == cf.CF_ESHAPE
    assert L.cf_kv_deviation(None, 0, 8, None, 0, 8, None, 0, 8, None) == cf.CF_OK
    assert L.cf_kv_deviation(None, 0, 8, None, 0, 8, None, 4, 8, None) == cf.CF_EINVAL


def test_null_context_rejected(L):
    assert L.cf_rope_reposition(None, None, None, 0, 0, None, None, 0, 0, None, 0, 0, 0, None) == cf.CF_EINVAL
    assert L.cf_blend_layer(None, None, None, None, None, None, 0, 1, None, 0, None) == cf.CF_EINVAL
    assert L.cf_blend_prefill(None, None, None, None, None, 1, 0, None, None, 0, 0, None, 0, 0, 0, 0, None, 0,
                              None, None, 0, None, None, None, None, 0, None) == cf.CF_EINVAL
    assert L.cf_blend_layer_workspace_size(None, 10, 5) == 0
    assert L.cf_blend_prefill_workspace_size(None, 10, 5, 3, 0) == 0
    sched = (ctypes.c_int32 * 2)(3, 2)
    assert L.cf_blend_prefill_gradual(None, None, None, None, None, 10, 5, None, None, 0, 0, None, 0, 1, sched, None,
                                      None, 0, None, None, None, None, 0, None) == cf.CF_EINVAL
    assert L.cf_blend_prefill_gradual_workspace_size(None, 10, 5, 1, sched) == 0
    assert L.cf_blend_prefill_streamed(None, None, None, None, None, 1, 0, None, None, 0, 0, None, 0, 0, 0, 0, None,
                                       0, None, None, 0, None, None, None, None, 0, None) == cf.CF_EINVAL
    assert L.cf_blend_prefill_streamed_workspace_size(None, 10, 5, 3, 0, 10) == 0
    lset = (ctypes.c_int32 * 1)(0)
    assert L.cf_query_scores(None, None, None, None, 10, 5, None, None, 0, lset, 1, None, None, 0, None) == cf.CF_EINVAL
    assert L.cf_query_scores_workspace_size(None, 10, 5) == 0


def test_loading_controller_host_logic_agrees_with_oracle():
    import itertools
    tables = [{(5, 100): 1.0, (15, 100): 3.0, (30, 100): 6.0, (100, 100): 20.0},
              {(1, 3): 2.0, (1, 2): 2.0, (3, 4): 9.0}, {}]
    for t, load, floor in itertools.product(tables, [0.1, 2.0, 3.0, 6.5, 50.0], [(15, 100), (0, 1), (1, 3)]):
        assert cf.loading_controller(load, t, floor) == oracle.loading_ratio(load, t, floor)


def test_gradual_schedule_host_logic_agrees_with_oracle():
    for n in [0, 1, 10, 512, 3072, 10240]:
        for first, keep, final in [((20, 100), (9, 10), (15, 100)), ((30, 100), (1, 2), (5, 100)),
                                   ((15, 100), (1, 1), (15, 100)), ((0, 100), (1, 2), (0, 100)),
                                   ((100, 100), (0, 1), (1, 100))]:
            for n_sched in [1, 3, 31]:
                assert cf.gradual_schedule(n, n_sched, first, keep, final) == \
                    oracle.gradual_schedule(n, n_sched, first, keep, final)
    with pytest.raises(cf.CfError) as e:
        cf.gradual_schedule(100, 3, (10, 100), (1, 2), (20, 100))
    assert e.value.status == cf.CF_EINVAL


def test_context_rejects_bad_shapes(L):
    h = ctypes.c_void_p()
    bad = [cf.ModelCfg(2, 256, 4, 2, 96, 688, 1000, 0, 1e4, 1e-5, 0),    # head_dim 96
           cf.ModelCfg(2, 256, 4, 3, 64, 688, 1000, 0, 1e4, 1e-5, 0),    # 4 % 3
           cf.ModelCfg(2, 256, 4, 2, 64, 688, 1000, 0, 1e4, 1e-5, 7),    # dtype
           cf.ModelCfg(2, 260, 4, 2, 64, 688, 1000, 0, 1e4, 1e-5, 0)]    # d % 8
    want = [cf.CF_EUNSUPPORTED, cf.CF_ESHAPE, cf.CF_EDTYPE, cf.CF_EUNSUPPORTED]
    for c, w in zip(bad, want):
        assert L.cf_ctx_create(ctypes.byref(c), 1024, 0, ctypes.byref(h)) == w


def test_budget_host_logic_agrees_with_oracle():
    for n in [0, 1, 7, 10, 512, 3072, 7720, 10240, 16384]:
        for num, den in [(0, 100), (1, 100), (5, 100), (15, 100), (29, 100), (30, 100), (1, 3), (100, 100)]:
            assert cf.budget(n, num, den) == oracle.budget(n, num, den)
    for args in [(10, 101, 100), (10, -1, 100), (10, 1, 0), (-1, 1, 2)]:
        with pytest.raises(cf.CfError) as e:
            cf.budget(*args)
        assert e.value.status == cf.CF_EINVAL


def test_span_policy_host_logic_agrees_with_oracle():
    import numpy as np
    for n in [1, 30, 92, 300, 3072, 7728]:
        for size, off in [(92, 46), (92, 0), (7, 3), (64, 63)]:
            assert cf.fixed_chunk_bounds(n, size, off) == oracle.fixed_chunk_bounds(n, size, off)
        assert cf.single_window_bounds(n) == oracle.single_window_bounds(n)
    rng = np.random.default_rng(2)
    for _ in range(100):
        d = rng.random(50).astype(np.float32)
        d[rng.integers(0, 50, 3)] = np.nan
        sel = np.unique(rng.integers(0, 50, 12))
        a, b = cf.selection_stats(sel, d), oracle.selection_stats(sel, d)
        assert a[0] == b[0] and (a[1] == b[1] or abs(a[1] - b[1]) < 1e-12 or (np.isnan(a[1]) and np.isnan(b[1])))


def test_policy_calls_validate_and_report_sizes(L):
    """The policy arithmetic entry points reject bad arguments with CF_EINVAL and report the
    number of bounds a too-small array would have needed."""
    k = ctypes.c_int32(-7)
    assert L.cf_budget(10, 1, 2, None) == cf.CF_EINVAL
    assert L.cf_budget(10, 3, 2, ctypes.byref(k)) == cf.CF_EINVAL and k.value == -7
    assert "ratio" in L.cf_last_error().decode()
    assert L.cf_budget(3072, 15, 100, ctypes.byref(k)) == cf.CF_OK and k.value == 460 and L.cf_last_error() == b""
    nb = ctypes.c_int32(0)
    small = (ctypes.c_int32 * 2)()
    assert L.cf_fixed_chunk_bounds(300, 92, 46, small, 2, ctypes.byref(nb)) == cf.CF_EINVAL and nb.value == 5
    assert L.cf_fixed_chunk_bounds(300, 92, 92, small, 2, ctypes.byref(nb)) == cf.CF_EINVAL
    assert L.cf_single_window_bounds(5, small, 2, ctypes.byref(nb)) == cf.CF_OK and list(small) == [0, 5]
    sched = (ctypes.c_int32 * 3)()
    assert L.cf_gradual_schedule(100, 3, 20, 100, 3, 2, 15, 100, sched) == cf.CF_EINVAL  # keep > 1
    seg, cap = ctypes.c_int32(0), ctypes.c_double(0)
    dup = (ctypes.c_int32 * 2)(3, 3)
    dev = (ctypes.c_float * 5)(1, 2, 3, 4, 5)
    assert L.cf_selection_stats(dup, 2, dev, 5, ctypes.byref(seg), ctypes.byref(cap)) == cf.CF_EINVAL
    out = (ctypes.c_int32 * 2)(1, 5)
    assert L.cf_selection_stats(out, 2, dev, 5, ctypes.byref(seg), ctypes.byref(cap)) == cf.CF_EINVAL
    ok = (ctypes.c_int32 * 2)(4, 3)
    assert L.cf_selection_stats(ok, 2, dev, 5, ctypes.byref(seg), ctypes.byref(cap)) == cf.CF_OK
    assert seg.value == 1 and abs(cap.value - 9 / 15) < 1e-15
    rat = (ctypes.c_int32 * 2)(1, 0)
    ms = (ctypes.c_double * 1)(1.0)
    a, b = ctypes.c_int32(0), ctypes.c_int32(0)
    assert L.cf_loading_ratio(2.0, rat, ms, 1, 15, 100, ctypes.byref(a), ctypes.byref(b)) == cf.CF_EINVAL


def test_ranked_span_order_validation(L):
    bad = (ctypes.c_int32 * 7)(0, 3, 8, 10, 1, 1, 0)   # bounds then a non-permutation
    assert L.cf_topk_select(None, 10, 3, cf.CF_SEL_RANKED_SPANS, bad, 3, None, None, 0, None) == cf.CF_EINVAL
    assert "permutation" in L.cf_last_error().decode()
    good = (ctypes.c_int32 * 7)(0, 3, 8, 10, 2, 0, 1)
    assert L.cf_topk_select(None, 10, 0, cf.CF_SEL_RANKED_SPANS, good, 3, None, None, 0, None) == cf.CF_OK
    assert L.cf_topk_select(None, 10, 3, cf.CF_SEL_SPAN_HEADS, good, 3, None, None, 0, None) == cf.CF_EINVAL
    assert cf.topk_workspace_size(10, "ranked") == 0 and cf.topk_workspace_size(10, "heads") == 0


def test_binding_checks_buffer_extent_and_dtype():
    """The binding's buffer check: the storage from a tensor's data pointer must hold the elements
    the call will touch (a view's offset counts), and the dtype must be the expected one."""
    import torch
    base = torch.zeros(3, 10, 4)
    cf._room(base, 120, "a", torch.float32)
    cf._room(base[:, 2:], 120 - 8, "view")  # from element 8 on
    cf._room(None, 10**9, "absent")
    cf._room(base, 0, "nothing touched")
    with pytest.raises(cf.CfError) as e:
        cf._room(base, 121, "a")
    assert e.value.status == cf.CF_EINVAL and "121" in str(e.value)
    with pytest.raises(cf.CfError) as e:
        cf._room(base[1:], 120 - 39, "view")
    assert e.value.status == cf.CF_EINVAL
    with pytest.raises(cf.CfError) as e:
        cf._room(base.to(torch.bfloat16), 1, "a", torch.float32)
    assert e.value.status == cf.CF_EDTYPE


def test_product_path_fails_loudly_without_the_library(monkeypatch):
    """No fallback: with libcf.so absent, every entry point raises instead of computing anything."""
    monkeypatch.setattr(cf, "LIB_PATH", os.path.join(os.path.dirname(cf.LIB_PATH), "absent", "libcf.so"))
    monkeypatch.setattr(cf, "_lib", None)
    for call in (cf.lib, cf.version, lambda: cf.topk_workspace_size(10, "token"), lambda: cf.budget(10, 1, 2),
                 lambda: cf.gradual_schedule(10, 2), lambda: cf.fixed_chunk_bounds(100),
                 lambda: cf.Context.from_model_cfg(synth.TINY, max_pos=64)):
        with pytest.raises(RuntimeError, match="missing"):
            call()


def _oracle_imports(path):
    """(enclosing function or None, line) of every import of the oracle package in a source file."""
    import ast
    tree = ast.parse(open(path).read())
    found = []

    def walk(node, fn):
        for child in ast.iter_child_nodes(node):
            f = child.name if isinstance(child, (ast.FunctionDef, ast.AsyncFunctionDef)) else fn
            names = []
            if isinstance(child, ast.Import):
                names = [a.name for a in child.names]
            elif isinstance(child, ast.ImportFrom):
                names = [child.module or ""]
            if any(n == "oracle" or n.startswith("oracle.") for n in names):
                found.append((f, child.lineno))
            walk(child, f)
    walk(tree, None)
    return found


def test_oracle_only_reached_from_tests_smoke_and_cpu_baseline():
    """The product package never imports the oracle; bench.py only in its cpu_baseline leg and
    __graft_entry__.py only in smoke()."""
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    pkg = os.path.join(root, "selective_recompute_cf_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith(".py"):
                assert _oracle_imports(os.path.join(dirpath, f)) == [], f
    assert {fn for fn, _ in _oracle_imports(os.path.join(root, "bench.py"))} <= {"cpu_baseline"}
    assert {fn for fn, _ in _oracle_imports(os.path.join(root, "__graft_entry__.py"))} <= {"smoke"}


def test_anchor_positions_host_logic_agrees_with_oracle():
    """cf_anchor_positions (QCFuse Eq. 14-15) against oracle.select_anchors chunk by chunk: Sink and
    both key-norm directions, ragged chunks stored out of request order, integer-valued scores with
    many ties (lower position first), anchor ratios from 0 to 1."""
    import numpy as np
    rng = np.random.default_rng(31)
    for trial in range(40):
        m = int(rng.integers(1, 7))
        lens = rng.integers(1, 60, m).tolist()
        order = rng.permutation(m)  # store rows in a shuffled order; request positions in chunk order
        rows, at = {}, 0
        for i in order:
            rows[i] = at
            at += lens[i]
        dst = np.concatenate([[0], np.cumsum(lens)[:-1]]).tolist()
        tab = [(rows[i], int(rng.integers(0, 5)), dst[i], lens[i]) for i in range(m)]
        scores = rng.integers(0, 6, at).astype(np.float32)
        for ratio in [(0, 1), (1, 10), (1, 3), (7, 10), (1, 1)]:
            for rule in ("sink", "knorm", "knorm_low"):
                got = cf.anchor_positions(rule, tab, ratio, scores if rule != "sink" else None, at)
                want = np.concatenate([dst[i] + oracle.select_anchors(
                    lens[i], ratio[0], ratio[1], rule, scores[rows[i]:rows[i] + lens[i]]) for i in range(m)])
                assert got == sorted(want.tolist()), (trial, ratio, rule)
    with pytest.raises(cf.CfError):
        cf.anchor_positions("knorm", [(0, 0, 0, 10)], (1, 10), None, 10)  # key norms need scores
    with pytest.raises(cf.CfError):
        cf.anchor_positions("sink", [(0, 0, 0, 10)], (11, 10))
