"""GPU parity of the HBM-bound steps through the C ABI: RoPE re-position + stitch, KV deviation,
token top-k and document-aligned selection (bit-exact on identical deviation arrays)."""
import numpy as np
import pytest

import oracle
import synth
import selective_recompute_cf_amd as cf
from tests import _golden
from tests._gpu import compare, context, host, say, torch_dtype

pytestmark = pytest.mark.gpu


def _torch():
    import torch
    return torch


@pytest.mark.parametrize("dtype,hd", [("f32", 64), ("bf16", 64), ("bf16", 128)])
def test_reposition_matches_oracle(dtype, hd):
    """QCFuse Eq. 4 with rotation composition: chunks of ragged length, negative and positive
    offsets, a layer range that leaves layer 0 untouched."""
    torch = _torch()
    cfg = synth.TINY.replace(head_dim=hd, n_kv_heads=2, dtype=dtype, n_layers=3)
    kvd = cfg.kv_dim
    Ly, rows, L = 3, 300, 400
    say(f"reposition dtype={dtype} hd={hd}")
    ctx = context(cfg, max_pos=2048)
    ks = synth.normal_array([7, 1], (Ly, rows, cfg.n_kv_heads, hd))
    vs = synth.normal_array([7, 2], (Ly, rows, cfg.n_kv_heads, hd))
    if dtype == "bf16":
        ks, vs = synth.bf16_round(ks), synth.bf16_round(vs)
    table = [(0, 0, 0, 37), (37, 0, 37, 100), (137, 512, 137, 61), (198, 1000, 198 + 50, 102), (10, 3, 380, 20)]
    dt = torch_dtype(dtype)
    k_store = torch.from_numpy(ks.reshape(Ly, rows, kvd)).to(dt).cuda()
    v_store = torch.from_numpy(vs.reshape(Ly, rows, kvd)).to(dt).cuda()
    k_blend = torch.full((Ly, L, kvd), 7.0, dtype=dt, device="cuda")
    v_blend = torch.full((Ly, L, kvd), 7.0, dtype=dt, device="cuda")
    ctx.rope_reposition(k_store, v_store, k_blend, v_blend, table, 1, 3)
    torch.cuda.synchronize()
    kref, vref = oracle.stitch(ks, vs, table, L, range(1, 3), cfg.rope_theta,
                               np.float64, n_total=L)
    kb, vb = host(k_blend).reshape(Ly, L, cfg.n_kv_heads, hd), host(v_blend).reshape(Ly, L, cfg.n_kv_heads, hd)
    covered = np.zeros(L, bool)
    for _, _, dst, ln in table:
        covered[dst:dst + ln] = True
    tol = (1e-5, 1e-5) if dtype == "f32" else (1e-6, 2.0 ** -8)
    compare("K", kb[1:, covered], kref[1:, covered], atol=tol[0], rtol=tol[1])
    np.testing.assert_array_equal(vb[1:, covered], vref[1:, covered])
    assert np.all(kb[0] == 7.0) and np.all(kb[1:, ~covered] == 7.0)


@pytest.mark.parametrize("Ly,N,chunk", [(31, 3072, 512), (79, 16384, 1024)])
def test_reposition_full_size_sampled_layers(Ly, N, chunk):
    """The launch the sweep times: every layer after the selection layer of the Llama-3-8B-shaped
    request (31 x 6 x 512 rows) and of the 70B-shaped one (79 x 16 x 1024 rows) re-positioned in one
    call, chunks encoded at position 0 and placed at their request offsets. Seeded bf16 inputs drawn
    on the GPU; the first, a middle and the last layer are compared with the oracle over every row."""
    torch = _torch()
    cfg = synth.LLAMA3_8B.replace(n_layers=Ly)
    H, hd, kvd = cfg.n_kv_heads, cfg.head_dim, cfg.kv_dim
    say(f"reposition full size Ly={Ly} N={N}")
    ctx = context(cfg, max_pos=2 * N + 1)
    g = torch.Generator(device="cuda").manual_seed(N + Ly)
    ks = torch.randn((Ly, N, kvd), device="cuda", generator=g).to(torch.bfloat16)
    vs = torch.randn((Ly, N, kvd), device="cuda", generator=g).to(torch.bfloat16)
    kb, vb = torch.empty_like(ks), torch.empty_like(vs)
    table = [(i * chunk, 0, i * chunk, chunk) for i in range(N // chunk)]
    ctx.rope_reposition(ks, vs, kb, vb, table, 0, Ly)
    torch.cuda.synchronize()
    for layer in (0, Ly // 2, Ly - 1):
        k_in = host(ks[layer]).reshape(1, N, H, hd)
        v_in = host(vs[layer]).reshape(1, N, H, hd)
        kref, vref = oracle.stitch(k_in, v_in, table, N, [0], cfg.rope_theta, np.float64, n_total=N)
        compare(f"K layer {layer}", host(kb[layer]).reshape(N, H, hd), kref[0], atol=1e-6, rtol=2.0 ** -8)
        np.testing.assert_array_equal(host(vb[layer]).reshape(N, H, hd), vref[0])
    ctx.close()


@pytest.mark.parametrize("n", [32 * 3072, 1 << 20])
def test_deviation_full_size_sampled_rows(n):
    """The deviation launches the sweep times (all 32 layers of the request's 3072 rows at once, and
    a million rows), kvd = 1024, bf16 inputs drawn on the GPU from a seed; 2000 sampled rows against
    the oracle."""
    torch = _torch()
    say(f"deviation full size n={n}")
    g = torch.Generator(device="cuda").manual_seed(n)
    kn = torch.randn((n, 1024), device="cuda", generator=g).to(torch.bfloat16)
    kr = torch.randn((n, 1024), device="cuda", generator=g).to(torch.bfloat16)
    dev = torch.empty(n, dtype=torch.float32, device="cuda")
    cf.kv_deviation(kn, kr, dev)
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(n).choice(n, 2000, replace=False))
    idx = torch.from_numpy(rows).cuda()
    want = oracle.kv_deviation(host(kn[idx]), host(kr[idx]))
    compare("dev", host(dev[idx]), want, atol=0.0, rtol=1e-5)


def test_reposition_rejects_bad_chunks():
    torch = _torch()
    cfg = synth.TINY
    ctx = context(cfg, max_pos=1024)
    a = torch.zeros(2, 64, cfg.kv_dim, device="cuda")
    with pytest.raises(cf.CfError):
        ctx.rope_reposition(a, a, a, a, [(0, 0, 40, 30)], 0, 2)   # dst past the blended rows
    with pytest.raises(cf.CfError):
        ctx.rope_reposition(a, a, a, a, [(0, 0, 0, 10), (10, 0, 5, 10)], 0, 2)  # overlap
    with pytest.raises(cf.CfError):
        ctx.rope_reposition(a, a, a, a, [(0, 2000, 0, 10)], 0, 2)  # offset beyond max_pos


@pytest.mark.parametrize("dn,dr", [("f32", "f32"), ("bf16", "bf16"), ("f32", "bf16")])
def test_deviation_matches_oracle(dn, dr):
    torch = _torch()
    n, kvd = 777, 1024
    a = synth.normal_array([8, 1], (n, kvd))
    b = a + 0.3 * synth.normal_array([8, 2], (n, kvd))
    if dn == "bf16":
        a = synth.bf16_round(a)
    if dr == "bf16":
        b = synth.bf16_round(b)
    ta = torch.from_numpy(a).to(torch_dtype(dn)).cuda()
    tb = torch.from_numpy(b).to(torch_dtype(dr)).cuda()
    dev = torch.zeros(n, device="cuda")
    cf.kv_deviation(ta, tb, dev)
    torch.cuda.synchronize()
    compare("dev", dev.cpu().numpy(), oracle.kv_deviation(a, b), atol=0.0, rtol=1e-5)


def _gpu_topk(d, k, mode="token", bounds=None):
    torch = _torch()
    dev = torch.from_numpy(np.asarray(d, np.float32)).cuda()
    out = torch.full((max(k, 1),), -1, dtype=torch.int32, device="cuda")
    ws = torch.empty(max(cf.topk_workspace_size(len(d), mode), 1), dtype=torch.uint8, device="cuda")
    cf.topk_select(dev, k, out, mode, bounds, ws)
    torch.cuda.synchronize()
    return out.cpu().numpy()[:k].tolist()


@pytest.mark.parametrize("case", _golden.topk_cases())
def test_topk_golden(case):
    d, k, want = case
    assert _gpu_topk(d, k) == want


@pytest.mark.parametrize("n", [1, 7, 100, 1000, 1025, 3072, 10240, 16384, 100003])
def test_topk_bit_exact_vs_oracle(n):
    rng = np.random.default_rng(n)
    say(f"topk n={n}")
    for trial in range(3):
        if trial == 0:
            d = rng.random(n).astype(np.float32)
        elif trial == 1:  # heavy ties, zeros of both signs, inf, nan, denormals
            d = rng.choice(np.array([0.0, -0.0, 1e-45, 3e-45, 0.5, 2.0, np.inf, np.nan], np.float32), n)
        else:  # sums of squares: skewed, as deviations are
            d = (rng.standard_normal(n).astype(np.float32) ** 2) * np.float32(3.0)
        for k in sorted({0, 1, n // 7, n // 2, n - 1, n}):
            if 0 <= k <= n:
                assert _gpu_topk(d, k) == oracle.select_topk(d, k).tolist(), (n, trial, k)


@pytest.mark.parametrize("n", [(1 << 20) + 3, 3000017])
def test_topk_large_n_multiblock_bit_exact(n):
    """From n = 65536 on the selection runs on the whole GPU (a sampled band around the threshold,
    a collect pass, digit passes over the candidates, per-range counts, a scan and an ordered
    write; histogram passes over all n values when the band misses or does not fit); it must give
    the same unique answer as the oracle. Uniform values take the sampled route; values sorted by
    index put every undecided value into a few ranges, whose candidate slices overflow and are
    read again; heavy ties and a constant array leave the band too large for the list."""
    rng = np.random.default_rng(n)
    say(f"topk large n={n}")
    for trial in range(4):
        if trial == 0:
            d = rng.random(n).astype(np.float32)
        elif trial == 1:
            d = rng.choice(np.array([0.0, -0.0, 1e-45, 0.5, 2.0, np.inf, np.nan], np.float32), n)
        elif trial == 2:  # ascending with runs of equal values
            d = np.sort(rng.integers(0, n // 3, n)).astype(np.float32)
        else:
            d = np.full(n, 0.25, np.float32)
        for k in sorted({1, n // 100, n // 2, n}):
            assert _gpu_topk(d, k) == oracle.select_topk(d, k).tolist(), (n, trial, k)


def test_topk_whole_gpu_16m_bit_exact():
    """n = 2^24 + 7: sub-ranges of 4096 indices (four write steps each, a ragged last one), against the
    oracle on skewed values like squared key deviations and on values with runs of ties."""
    n = (1 << 24) + 7
    rng = np.random.default_rng(24)
    say(f"topk 16M n={n}")
    for trial in range(2):
        d = ((rng.standard_normal(n).astype(np.float32) ** 2) * np.float32(3.0) if trial == 0 else
             np.round(rng.random(n) * 1000).astype(np.float32))
        for k in (n * 15 // 100, n // 2 + 1):
            assert _gpu_topk(d, k) == oracle.select_topk(d, k).tolist(), (trial, k)


def _order_keys(d):
    """Order-preserving 32-bit keys of float32 values (NaN as +inf, -0 as +0), for the test to find
    how many values share the threshold key's top 16 bits."""
    u = np.asarray(d, np.float32).view(np.uint32).copy()
    u[(u & 0x7FFFFFFF) > 0x7F800000] = 0x7F800000
    u[(u & 0x7FFFFFFF) == 0] = 0
    neg = (u & 0x80000000) != 0
    return np.where(neg, ~u, u | 0x80000000).astype(np.uint32)


@pytest.mark.parametrize("n", [(1 << 18) + 5, 2000003])
def test_topk_candidate_list_capacity_edges(n):
    """When the sampled band does not fit the workspace's candidate list, the whole-GPU selection
    falls back to the values that share the threshold key's top 16 bits, and when those do not fit
    either, it reads all n values twice more. Workspaces with list room (4 bytes a value, the first
    n / 16 entries ahead of the per-range slices) for exactly that many, one fewer, none, and the
    full size, and a value array 4 bytes off 16-byte alignment, must all give the oracle's unique
    answer."""
    torch = _torch()
    rng = np.random.default_rng(n)
    d = rng.standard_normal(n).astype(np.float32) ** 2  # skewed, as deviations are
    d[rng.integers(0, n, n // 100)] = np.float32(1.0)   # a block of ties
    d[rng.integers(0, n, 50)] = np.nan
    buf = torch.from_numpy(np.concatenate([np.zeros(1, np.float32), d])).cuda()
    aligned = buf[1:].clone()
    keys = _order_keys(d)
    srt = np.sort(keys)[::-1]
    base = cf.topk_workspace_min_size(n, "token")
    for k in (1, n // 7, n // 2, n):
        want = oracle.select_topk(d, k).tolist()
        h = int(np.count_nonzero((keys >> 16) == (srt[k - 1] >> 16)))
        assert h <= n // 16  # so that room for h list entries is exactly h
        say(f"topk capacity n={n} k={k} h={h}")
        for room in (h, h - 1, 0, None):
            nbytes = cf.topk_workspace_size(n, "token") if room is None else base + 4 * room
            ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
            for vals in (aligned, buf[1:]):
                out = torch.full((k,), -1, dtype=torch.int32, device="cuda")
                cf.topk_select(vals, k, out, "token", None, ws)
                torch.cuda.synchronize()
                assert out.cpu().numpy().tolist() == want, (n, k, room, vals.data_ptr() % 16)


def test_topk_whole_gpu_at_int32_max():
    """n = 2^31 - 1, the largest n the ABI takes (the index arithmetic of every pass in 64 bits where it
    can pass INT_MAX): too large for the oracle, so the unique answer is pinned by its properties,
    checked on the GPU with torch: k positions strictly ascending, every selected value at least every
    unselected one, and among the values equal to the threshold exactly the lowest-index ones taken.
    Uniform [0, 1) float32 values tie often at this n, so the tie rule is exercised."""
    torch = _torch()
    n = (1 << 31) - 1
    k = n * 15 // 100
    say(f"topk int32 max n={n} k={k}")
    g = torch.Generator(device="cuda").manual_seed(11)
    d = torch.rand(n, device="cuda", generator=g)
    out = torch.empty(k, dtype=torch.int32, device="cuda")
    ws = torch.empty(cf.topk_workspace_size(n, "token"), dtype=torch.uint8, device="cuda")
    cf.topk_select(d, k, out, "token", None, ws)
    torch.cuda.synchronize()
    del ws
    sel = out.long()
    del out
    assert bool((sel[1:] > sel[:-1]).all()) and int(sel[0]) >= 0 and int(sel[-1]) < n
    mask = torch.zeros(n, dtype=torch.bool, device="cuda")
    mask[sel] = True
    t = d[sel].min()
    assert float(d.masked_fill(mask, -1.0).max()) <= float(t)  # values lie in [0, 1)
    eq = torch.nonzero(d == t).squeeze(1)  # ascending; a few hundred at this n
    eq_sel = sel[d[sel] == t]
    assert len(eq_sel) >= 1 and torch.equal(eq_sel, eq[: len(eq_sel)])


def _sample_positions(n, s=32768):
    """The whole-GPU selection's stratified sample: stratum j of s gives the value at a hashed offset
    inside [j n / s, (j + 1) n / s) (Wellons' lowbias32 integer hash of j, scaled to n)."""
    j = np.arange(s, dtype=np.uint64)
    x = j.astype(np.uint32)
    x ^= x >> np.uint32(16)
    x = (x * np.uint32(0x7FEB352D)).astype(np.uint32)
    x ^= x >> np.uint32(15)
    x = (x * np.uint32(0x846CA68B)).astype(np.uint32)
    x ^= x >> np.uint32(16)
    jit = (x.astype(np.uint64) * np.uint64(n)) >> np.uint64(32)
    return ((j * np.uint64(n) + jit) // np.uint64(s)).astype(np.int64)


@pytest.mark.parametrize("direction", ["sample_low", "sample_high"])
def test_topk_sampled_band_that_misses(direction):
    """Values planted at exactly the sampled positions make the sample misjudge the distribution: too
    many values lie above its band (sample_low) or too few at or above it (sample_high), so the
    selection must take the fallback route (histograms over all n values, then the threshold's 16-bit
    bin) and still give the oracle's unique answer."""
    n = (1 << 20) + 3
    rng = np.random.default_rng(7)
    d = rng.random(n).astype(np.float32) + np.float32(1.0)
    pos = _sample_positions(n)
    assert pos.min() >= 0 and pos.max() < n and np.all(np.diff(pos) >= 0)
    d[pos] = np.float32(1e-3) if direction == "sample_low" else np.float32(1e3)
    say(f"topk band miss {direction} n={n}")
    for k in (n // 7, n // 2):
        assert _gpu_topk(d, k) == oracle.select_topk(d, k).tolist(), (direction, k)


@pytest.mark.parametrize("case", _golden.doc_span_cases())
def test_doc_spans_golden(case):
    d, b, k, want = case
    assert _gpu_topk(d, k, "doc", b) == want


@pytest.mark.parametrize("policy", ["single-window", "fixed-chunk", "random-document", "heads"])
@pytest.mark.parametrize("n_spans,span_len", [(1, 50), (6, 512), (84, 92), (256, 40)])
def test_span_policies_bit_exact_vs_oracle(policy, n_spans, span_len):
    """The ablation policies of Request Order Matters §2.3 (single-window and fixed-chunk through
    the document-aligned mode over generated bounds, random-document as a ranked order drawn here)
    and EPIC's chunk heads, against the oracle on the same arrays; ragged documents, ties."""
    rng = np.random.default_rng(n_spans * 7 + span_len)
    lens = np.maximum(1, rng.integers(span_len // 2, span_len * 3 // 2 + 1, n_spans))
    docs = [0] + np.cumsum(lens).tolist()
    n = docs[-1]
    say(f"{policy} n_spans={n_spans} n={n}")
    for trial in range(2):
        d = rng.random(n).astype(np.float32) if trial == 0 else rng.integers(0, 3, n).astype(np.float32)
        for k in sorted({0, 1, n // 20, n // 3, n - 1, n}):
            if policy == "single-window":
                b = cf.single_window_bounds(n)
                want = oracle.select_doc_spans(d, k, oracle.single_window_bounds(n))
                got = _gpu_topk(d, k, "doc", b)
            elif policy == "fixed-chunk":
                b = cf.fixed_chunk_bounds(n, 92, 46)
                assert b == oracle.fixed_chunk_bounds(n, 92, 46)
                want = oracle.select_doc_spans(d, k, b)
                assert len(b) - 1 <= 256
                got = _gpu_topk(d, k, "doc", b)
            elif policy == "random-document":
                order = rng.permutation(n_spans).tolist()
                want = oracle.select_ranked_spans(n, k, docs, order)
                got = _gpu_topk(d, k, "ranked", (docs, order))
            else:
                want = oracle.select_span_heads(n, k, docs)
                got = _gpu_topk(d, k, "heads", docs)
            assert got == want.tolist(), (trial, k)


@pytest.mark.parametrize("n_spans,span_len", [(1, 50), (5, 7), (20, 512), (84, 92), (256, 40)])
def test_doc_spans_bit_exact_vs_oracle(n_spans, span_len):
    rng = np.random.default_rng(n_spans * 1000 + span_len)
    lens = np.maximum(1, rng.integers(span_len // 2, span_len * 3 // 2 + 1, n_spans))
    bounds = [0] + np.cumsum(lens).tolist()
    n = bounds[-1]
    say(f"spans n_spans={n_spans} n={n}")
    for trial in range(3):
        if trial == 0:
            d = rng.random(n).astype(np.float32)
        elif trial == 1:
            d = rng.integers(0, 3, n).astype(np.float32)
        else:
            d = (rng.standard_normal(n).astype(np.float32) ** 2)
        for k in sorted({0, 1, n // 20, n // 3, n - 1, n}):
            assert _gpu_topk(d, k, "doc", bounds) == oracle.select_doc_spans(d, k, bounds).tolist(), (trial, k)
