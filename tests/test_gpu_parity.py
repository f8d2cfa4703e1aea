"""GPU parity: the HIP path (through the C-ABI) against the CPU oracle.

Bar: routing outputs (route bits, C_struct numerator, block masses, totals)
and index sets bit-exact; attention max-abs 2e-2 for bf16 and 1e-5 for fp32
against the fp64 oracle on the same index sets.  Below 128K every row is
checked; at 128K and above the full index sets plus 256 seeded rows per head.
"""
import gc
import os

import numpy as np
import pytest

import dynamic_sparse_attention_proxy_amd as crisp
import oracle
import synth
from gpu_harness import (DeviceInputs, Timer, compare_index_sets, download_index_sets, log, rows_of,
                         run_dense, run_route_select, run_sparse, spec_for)

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 2e-2}

_cache = {}


def _case(name, wl=None, select_mode=crisp.SELECT_NOISE_FLOOR):
    key = (name, select_mode)
    if key in _cache:
        return _cache[key]
    _cache.clear()
    gc.collect()
    wl = wl or synth.WORKLOADS[name]
    log("case", name, "mode", select_mode, "n", wl.n, "heads", wl.hq, wl.hkv, "d", wl.d, wl.dtype)
    with Timer(f"inputs {name}"):
        I = synth.make_inputs(wl)
    with Timer(f"upload {name}"):
        X = DeviceInputs(I)
    spec = spec_for(wl, select_mode)
    with Timer(f"gpu route+select {name}"):
        bufs = run_route_select(spec, X)
    with Timer(f"oracle index sets {name}"):
        ref = oracle.index_sets(I.q, I.k, wl.block, wl.w_sink, wl.w_local, synth.TAU, synth.ALPHA, synth.GAMMA,
                                I.bias_offsets, I.bias_values,
                                keep_all=select_mode == crisp.SELECT_KEEP_ALL,
                                cumulative=select_mode == crisp.SELECT_CUMULATIVE)
    _cache[key] = (wl, I, X, spec, bufs, ref)
    return _cache[key]


def _check_attention(wl, I, X, spec, bufs, ref, rows, what, heads=None):
    """Sparse and dense GPU outputs against the fp64 oracle at the given rows / heads."""
    import torch
    specs = oracle.specs_from_index_sets(ref)
    hs = list(range(len(specs))) if heads is None else list(heads)
    hsel = torch.as_tensor(hs, device="cuda")
    with Timer(f"gpu sparse {what}"):
        o_sp = rows_of(run_sparse(spec, X, bufs)[hsel], rows)
    with Timer(f"oracle sparse {what}"):
        r_sp = oracle.attention(I.q, I.k, I.v, wl.block, specs, rows=rows, bias_offsets=I.bias_offsets,
                                bias_values=I.bias_values, heads=hs, chunk=512)
    err_sp = np.abs(o_sp - r_sp).max()
    with Timer(f"gpu dense {what}"):
        o_de = rows_of(run_dense(spec, X)[hsel], rows)
    with Timer(f"oracle dense {what}"):
        r_de = oracle.attention(I.q, I.k, I.v, wl.block, [dict(kind="dense")] * len(specs), rows=rows,
                                bias_offsets=I.bias_offsets, bias_values=I.bias_values, heads=hs, chunk=512)
    err_de = np.abs(o_de - r_de).max()
    log(what, "max-abs sparse", err_sp, "dense", err_de)
    assert np.isfinite(o_sp).all() and np.isfinite(o_de).all()
    if wl.dtype == "f32" and wl.qk_scale > 1.0:
        tol = _peaked_f32_tolerance(wl, I, rows, hs)[:, :, None]
        log(what, "row tolerance", float(tol.min()), float(tol.max()))
        assert np.all(np.abs(o_sp - r_sp) <= tol), f"sparse max-abs {err_sp}"
        assert np.all(np.abs(o_de - r_de) <= tol), f"dense max-abs {err_de}"
        return
    assert err_sp <= TOL[wl.dtype], f"sparse max-abs {err_sp}"
    assert err_de <= TOL[wl.dtype], f"dense max-abs {err_de}"


def _peaked_f32_tolerance(wl, I, rows, heads):
    """Per-row fp32 bar for inputs with logits of thousands of nats.

    An fp32 logit s = fl(q . k) c + bias carries an absolute rounding error up to
    E = gamma_(d+2) (c sum_t |q_t k_t| + |bias|), gamma_m = m u / (1 - m u),
    u = 2^-24: proportional to the logit's size, not bounded by the 1e-5 bar.  A
    softmax-weighted mean moves by at most 2 max_j |ds_j| max_j |v_j| under
    logit perturbations ds, so each row is held to 1e-5 (the rounding of the
    probabilities and of the weighted sum, as for every other fp32 case) plus
    that first-order term with the row's largest E over its causal keys.
    """
    n, d = wl.n, wl.d
    rows = np.arange(n) if rows is None else np.asarray(rows)
    G = wl.hq // wl.hkv
    u = 2.0 ** -24
    gam = (d + 2) * u / (1 - (d + 2) * u)
    c = 1.0 / np.sqrt(d)
    out = np.empty((len(heads), len(rows)))
    causal = np.arange(n)[None, :] <= rows[:, None]
    for hi, h in enumerate(heads):
        g = h // G
        mag = c * (np.abs(I.q[h][rows].astype(np.float64)) @ np.abs(I.k[g].astype(np.float64)).T)
        bmax = float(np.abs(I.bias_values[h]).max()) if I.bias_values.size else 0.0
        E = gam * (np.where(causal, mag, 0.0).max(axis=1) + bmax)
        out[hi] = TOL["f32"] + 2.0 * E * float(np.abs(I.v[g]).max())
    return out


ALL = ["tiny", "llama_32k", "llama_128k", "qwen_128k", "llama_512k"]

JSD_TAU = (1, 100)


def _check_jsd(wl, I, X, spec, bufs, ref):
    """crisp_route_jsd on the proxy that crisp_route left in bufs, against the oracle's
    divergence router on the oracle's own block masses: bit-exact J, route and pooled row."""
    import torch
    bh, nb = spec.heads, spec.num_blocks
    r_gpu = torch.zeros(bh, dtype=torch.uint8, device="cuda")
    j_gpu = torch.zeros(bh, dtype=torch.int64, device="cuda")
    p_gpu = torch.zeros(bh, nb, dtype=torch.int64, device="cuda")
    crisp.route_jsd(spec, X.q, X.k, bufs, r_gpu, j_gpu, JSD_TAU, p_gpu)
    torch.cuda.synchronize()
    with Timer("oracle jsd"):
        want = oracle.jsd_route(I.q, I.k, wl.block, ref["proxy"], JSD_TAU)
    assert np.array_equal(p_gpu.cpu().numpy(), want["abar"]), "pooled estimate"
    assert np.array_equal(j_gpu.cpu().numpy(), want["jsd"]), (j_gpu.cpu().numpy()[:4], want["jsd"][:4])
    assert np.array_equal(r_gpu.cpu().numpy(), want["route"])
    # the pooled estimate is an optional output: without it the router gives the same bits
    r2 = torch.zeros_like(r_gpu)
    j2 = torch.zeros_like(j_gpu)
    crisp.route_jsd(spec, X.q, X.k, bufs, r2, j2, JSD_TAU, None)
    torch.cuda.synchronize()
    assert torch.equal(r2, r_gpu) and torch.equal(j2, j_gpu)
    return want


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ALL)
def test_index_sets_bit_exact(name):
    wl, I, X, spec, bufs, ref = _case(name)
    gpu = download_index_sets(bufs)
    bad = compare_index_sets(gpu, ref)
    assert not bad, "\n".join(bad[:20])
    # the planted heads route to VS, the i.i.d. heads to pooled estimation
    expect = [1 if h in wl.planted_heads else 0 for h in range(wl.hq)]
    assert gpu["route"].tolist() == expect
    if name == "tiny":
        _check_attention(wl, I, X, spec, bufs, ref, None, f"{name} all rows")
    else:
        _check_attention(wl, I, X, spec, bufs, ref, synth.sample_rows(wl), f"{name} 256 sampled rows")
    if name == "llama_32k":
        # every row of two VS and two PE heads (both kinds of KV group)
        _check_attention(wl, I, X, spec, bufs, ref, None, f"{name} all rows, heads 0 1 16 17",
                         heads=[0, 1, 16, 17])


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ALL[::-1])  # the largest case is still cached from the test above
def test_jsd_router(name):
    """The divergence router bit-exact against the oracle; on the planted layers it makes
    the same decisions as C_struct (planted heads diverge from their pooled estimate)."""
    wl, I, X, spec, bufs, ref = _case(name)
    want = _check_jsd(wl, I, X, spec, bufs, ref)
    log(name, "JSD (nats) per head", (want["jsd"] * 2.0 ** -53).round(5).tolist())
    assert want["route"].tolist() == ref["proxy"]["route"].tolist()


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["tiny", "llama_32k"])
def test_keep_all_equals_dense(name):
    """With every block kept, the sparse path is dense causal attention, bit for bit."""
    wl, I, X, spec, bufs, ref = _case(name, select_mode=crisp.SELECT_KEEP_ALL)
    gpu = download_index_sets(bufs)
    bad = compare_index_sets(gpu, ref)
    assert not bad, "\n".join(bad[:20])
    o_sp = run_sparse(spec, X, bufs)
    o_de = run_dense(spec, X)
    import torch
    assert torch.equal(o_sp, o_de)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["tiny", "llama_32k", "qwen_128k"])
def test_cumulative_mode(name):
    """The cumulative-coverage comparison mode: VS lists bit-exact against the oracle's
    cumulative rule on the same masses, attention within tolerance."""
    wl, I, X, spec, bufs, ref = _case(name, select_mode=crisp.SELECT_CUMULATIVE)
    gpu = download_index_sets(bufs)
    bad = compare_index_sets(gpu, ref)
    assert not bad, "\n".join(bad[:20])
    rows = None if name == "tiny" else synth.sample_rows(wl)
    _check_attention(wl, I, X, spec, bufs, ref, rows, f"{name} cumulative")


@pytest.mark.timeout(600)
@pytest.mark.parametrize("alpha", [(5, 4), (3, 2)])
def test_alpha_variants(alpha):
    """Eq. 4 with the pages' larger multipliers: VS lists bit-exact against the oracle on the
    same (bit-exact) masses; a larger alpha never keeps more blocks."""
    import dataclasses
    wl, I, X, spec, bufs, ref = _case("llama_32k")
    spec_a = dataclasses.replace(spec, alpha=alpha)
    b2 = run_route_select(spec_a, X)
    gpu = download_index_sets(b2)
    base = download_index_sets(bufs)
    pr = ref["proxy"]
    for h in range(wl.hq):
        if not pr["route"][h]:
            continue
        for key, mk in (("vertical", "mass_v"), ("slash", "mass_s")):
            want = oracle.vs_select(pr[mk][h], pr["total"][h], alpha)
            assert np.array_equal(gpu["heads"][h][key], want), (h, key)
            assert set(want.tolist()) <= set(base["heads"][h][key].tolist()), (h, key)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("mode", [crisp.SELECT_NOISE_FLOOR, crisp.SELECT_CUMULATIVE])
def test_gamma_variant(mode):
    """gamma = 97/100, the pages' wider coverage: PE index sets (and, in the cumulative mode,
    the VS lists) bit-exact against the oracle; a larger gamma never keeps fewer blocks."""
    import dataclasses
    wl, I, X, spec, bufs, ref = _case("llama_32k", select_mode=mode)
    spec_g = dataclasses.replace(spec, gamma=(97, 100))
    b2 = run_route_select(spec_g, X)
    gpu = download_index_sets(b2)
    base = download_index_sets(bufs)
    pr = ref["proxy"]
    G = wl.hq // wl.hkv
    assert np.array_equal(gpu["route"], pr["route"])
    checked = 0
    for h in range(wl.hq):
        g, b = gpu["heads"][h], base["heads"][h]
        if pr["route"][h]:
            if mode != crisp.SELECT_CUMULATIVE:
                continue
            for key, mk in (("vertical", "mass_v"), ("slash", "mass_s")):
                want = oracle.cumulative_select(pr[mk][h], pr["total"][h], (97, 100))
                assert np.array_equal(g[key], want), (h, key)
                assert set(b[key].tolist()) <= set(want.tolist()), (h, key)
        else:
            if checked >= 4:  # the oracle's PE index is the slow part; four heads span both KV groups
                continue
            rowptr, cols = oracle.pe_index(I.q[h], I.k[h // G], wl.block, (97, 100))
            assert np.array_equal(g["rowptr"], rowptr), h
            assert np.array_equal(g["cols"], cols), h
            assert g["rowptr"][-1] >= b["rowptr"][-1], h
            checked += 1


@pytest.mark.timeout(120)
def test_binding_checks_tensors():
    """Wrong element type, layout or size is refused before anything is launched."""
    import torch
    wl = EDGE["ragged_bf16"]
    spec = spec_for(wl)
    bufs = crisp.Buffers(spec)
    q = torch.zeros(wl.hq, wl.n, wl.d, dtype=torch.bfloat16, device="cuda")
    k = torch.zeros(wl.hkv, wl.n, wl.d, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(crisp.CrispError, match="expected torch.bfloat16"):
        crisp.route(spec, q.float(), k, bufs)
    with pytest.raises(crisp.CrispError, match="contiguous"):
        crisp.route(spec, q.transpose(1, 2), k, bufs)
    with pytest.raises(crisp.CrispError, match="elements"):
        crisp.select_indices(spec, q.reshape(-1)[:-8], k, bufs)
    with pytest.raises(crisp.CrispError, match="bias_offsets"):
        crisp.route(spec, q, k, bufs, torch.zeros(wl.hq, 2, dtype=torch.int64, device="cuda"),
                    torch.zeros(wl.hq, 2, device="cuda"))
    torch.cuda.synchronize()


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["tiny", "llama_32k"])
def test_graph_replay_matches_eager(name):
    """The whole layer (route, select, sparse attention) captured in a HIP graph: the
    library allocates, clears with memset and synchronises nothing, so every replay,
    with eager work of the program in between, gives the eager bits."""
    import torch
    wl, I, X, spec, bufs, ref = _case(name)
    o_eager = torch.empty_like(X.q)
    crisp.prefill(spec, X.q, X.k, X.v, o_eager, bufs, X.bias_offsets, X.bias_values)
    torch.cuda.synchronize()
    gb = crisp.Buffers(spec)
    o = torch.empty_like(X.q)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # one eager call on the capture stream first
        crisp.prefill(spec, X.q, X.k, X.v, o, gb, X.bias_offsets, X.bias_values)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        crisp.prefill(spec, X.q, X.k, X.v, o, gb, X.bias_offsets, X.bias_values)
    torch.cuda.synchronize()
    od = torch.empty_like(X.q)
    for rep in range(3):
        o.fill_(float("nan"))
        gb.route.fill_(7)
        gb.pe_rowptr.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_eager), f"replay {rep}: output"
        bad = compare_index_sets(download_index_sets(gb), ref)
        assert not bad, f"replay {rep}: " + "\n".join(bad[:5])
        crisp.dense_prefill(spec, X.q, X.k, X.v, od, gb, X.bias_offsets, X.bias_values)  # eager work between
        torch.cuda.synchronize()


@pytest.mark.timeout(600)
def test_two_streams_with_own_workspaces():
    """The library keeps no state: two layers in flight on two streams, each with its
    own workspace and index buffers, give the bits of the same calls run alone."""
    import torch
    wl, I, X, spec, bufs, ref = _case("llama_32k")
    o_ref = torch.empty_like(X.q)
    crisp.prefill(spec, X.q, X.k, X.v, o_ref, bufs, X.bias_offsets, X.bias_values)
    torch.cuda.synchronize()
    b1, b2 = crisp.Buffers(spec), crisp.Buffers(spec)
    o1, o2 = torch.empty_like(X.q), torch.empty_like(X.q)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()  # default priority
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    for _ in range(2):
        crisp.prefill(spec, X.q, X.k, X.v, o1, b1, X.bias_offsets, X.bias_values, stream=s1)
        crisp.prefill(spec, X.q, X.k, X.v, o2, b2, X.bias_offsets, X.bias_values, stream=s2)
    torch.cuda.synchronize()
    assert torch.equal(o1, o_ref) and torch.equal(o2, o_ref)
    for b in (b1, b2):
        bad = compare_index_sets(download_index_sets(b), ref)
        assert not bad, "\n".join(bad[:5])


@pytest.mark.timeout(600)
def test_determinism():
    wl, I, X, spec, bufs, ref = _case("llama_32k")
    import torch
    o1 = run_sparse(spec, X, bufs)
    b2 = run_route_select(spec, X)
    for name in ("route", "cstruct_num", "mass_v", "mass_s", "mass_total", "vs_count", "vs_vertical", "vs_slash",
                 "pe_rowptr"):
        assert torch.equal(getattr(bufs, name), getattr(b2, name)), name
    nnz = int(bufs.pe_rowptr[:, -1].max())
    assert torch.equal(bufs.pe_col[:, :nnz], b2.pe_col[:, :nnz])
    o2 = run_sparse(spec, X, b2)
    assert torch.equal(o1, o2)
    assert torch.equal(run_dense(spec, X), run_dense(spec, X))


EDGE = {
    "ragged_f32": synth.Workload(name="ragged_f32", hq=4, hkv=2, d=64, n=1000, dtype="f32", block=64,
                                 rope_theta=0.0, seed=31, planted_heads=[0, 1], n_vertical=4,
                                 vertical_gain=(3.0, 3.0), fixed_slash=(0, 5)),
    "ragged_bf16": synth.Workload(name="ragged_bf16", hq=4, hkv=1, d=128, n=5000, dtype="bf16", block=128,
                                  rope_theta=5e5, seed=32, planted_heads=[0], n_vertical=8),
    "two_blocks_f32_d128": synth.Workload(name="two_blocks", hq=2, hkv=1, d=128, n=200, dtype="f32", block=128,
                                          rope_theta=0.0, seed=33, planted_heads=[0], n_vertical=0,
                                          fixed_slash=(0,)),
    "one_block_bf16": synth.Workload(name="one_block", hq=2, hkv=2, d=128, n=100, dtype="bf16", block=128,
                                     rope_theta=0.0, seed=34, planted_heads=[1], n_vertical=0, fixed_slash=(3,)),
    "single_token": synth.Workload(name="single_token", hq=1, hkv=1, d=64, n=1, dtype="f32", block=64,
                                   rope_theta=0.0, seed=35, planted_heads=[], n_vertical=0),
    "bf16_b64_d64": synth.Workload(name="bf16_b64_d64", hq=4, hkv=2, d=64, n=3000, dtype="bf16", block=64,
                                   rope_theta=1e4, seed=36, planted_heads=[0, 2], n_vertical=6),
    "batch2_bf16": synth.Workload(name="batch2", hq=4, hkv=2, d=128, n=2100, dtype="bf16", block=128,
                                  rope_theta=5e5, seed=37, planted_heads=[0, 1], n_vertical=5, batch=2),
    "f32_b128_d128": synth.Workload(name="f32_b128_d128", hq=2, hkv=1, d=128, n=1500, dtype="f32", block=128,
                                    rope_theta=0.0, seed=38, planted_heads=[0], n_vertical=3),
    # GQA groups of 8 (four full head pairs per KV head) and of 3 (the second pair
    # of each KV head has one head) on the matrix engine
    "gqa8_bf16": synth.Workload(name="gqa8", hq=8, hkv=1, d=128, n=6000, dtype="bf16", block=128,
                                rope_theta=5e5, seed=44, planted_heads=[0, 3, 4], n_vertical=5),
    "gqa3_bf16": synth.Workload(name="gqa3", hq=6, hkv=2, d=128, n=5200, dtype="bf16", block=128,
                                rope_theta=5e5, seed=45, planted_heads=[2, 3], n_vertical=4),
    # Degenerate inputs.  Q = K = 0: every causal key of a row ties, so all full key
    # blocks carry the same vertical mass (the noise floor keeps only the first and
    # last block), every pooled row is uniform (the PE selection is decided by ties),
    # and attention is the running mean of V.
    "constant_qk_vs_bf16": synth.Workload(name="constant_qk_vs", hq=4, hkv=2, d=128, n=1100, dtype="bf16",
                                          block=128, rope_theta=5e5, seed=42, planted_heads=[], n_vertical=0,
                                          qk_scale=0.0),
    "constant_qk_vs_f32": synth.Workload(name="constant_qk_vs_f32", hq=2, hkv=1, d=64, n=700, dtype="f32",
                                         block=64, rope_theta=0.0, seed=43, planted_heads=[1], n_vertical=0,
                                         fixed_slash=(0, 200), qk_scale=0.0),
    "constant_qk_pe_bf16": synth.Workload(name="constant_qk_pe", hq=4, hkv=2, d=128, n=3000, dtype="bf16",
                                          block=128, rope_theta=5e5, seed=39, planted_heads=[0], n_vertical=4,
                                          qk_scale=0.0),
    # Q and K scaled by 16 (logits by 256): rows dominated by one key, most
    # probabilities below the exp cutoff, the running maximum jumping by
    # thousands of nats between tiles.
    "peaked_bf16": synth.Workload(name="peaked", hq=4, hkv=2, d=128, n=3000, dtype="bf16", block=128,
                                  rope_theta=5e5, seed=40, planted_heads=[0, 1], n_vertical=6, qk_scale=16.0),
    "peaked_f32": synth.Workload(name="peaked_f32", hq=2, hkv=1, d=64, n=1500, dtype="f32", block=64,
                                 rope_theta=0.0, seed=41, planted_heads=[0], n_vertical=3, qk_scale=16.0),
}


@pytest.mark.timeout(300)
@pytest.mark.parametrize("name", list(EDGE))
@pytest.mark.parametrize("mode", [crisp.SELECT_NOISE_FLOOR, crisp.SELECT_KEEP_ALL])
def test_edge_shapes(name, mode):
    wl, I, X, spec, bufs, ref = _case("edge_" + name, EDGE[name], mode)
    gpu = download_index_sets(bufs)
    bad = compare_index_sets(gpu, ref)
    assert not bad, "\n".join(bad[:20])
    if mode == crisp.SELECT_NOISE_FLOOR:
        _check_jsd(wl, I, X, spec, bufs, ref)
    _check_attention(wl, I, X, spec, bufs, ref, None, f"{name} mode {mode}")
    if mode == crisp.SELECT_KEEP_ALL:
        import torch
        assert torch.equal(run_sparse(spec, X, bufs), run_dense(spec, X))


@pytest.mark.timeout(1200)
def test_long_context_1m():
    """Beyond the longest workload: a 1M-token layer through the whole path.  The GPU
    routes and selects every head; the oracle recomputes one planted and one i.i.d.
    head (routing outputs and index sets bit-exact) and 256 sampled rows of both."""
    import torch
    _cache.clear()
    gc.collect()
    wl = synth.WORKLOADS["llama_1m"]
    with Timer("inputs 1m"):
        I = synth.make_inputs(wl)
    X = DeviceInputs(I)
    spec = spec_for(wl)
    with Timer("gpu route+select 1m"):
        bufs = run_route_select(spec, X)
    gpu = download_index_sets(bufs)
    assert gpu["route"].tolist() == [1 if h in wl.planted_heads else 0 for h in range(wl.hq)]
    heads, kvs = [0, 16], [0, 16 // (wl.hq // wl.hkv)]
    with Timer("oracle index sets 1m (2 heads)"):
        ref = oracle.index_sets(I.q[heads], I.k[kvs], wl.block, wl.w_sink, wl.w_local, synth.TAU, synth.ALPHA,
                                synth.GAMMA, I.bias_offsets[heads], I.bias_values[heads])
    sub = {key: gpu[key][heads] for key in ("route", "cnum", "mass_v", "mass_s", "total")}
    sub["heads"] = [gpu["heads"][h] for h in heads]
    bad = compare_index_sets(sub, ref)
    assert not bad, "\n".join(bad[:20])
    rows = synth.sample_rows(wl)
    with Timer("gpu sparse 1m"):
        o = rows_of(run_sparse(spec, X, bufs)[torch.as_tensor(heads, device="cuda")], rows)
    with Timer("oracle attention 1m (2 heads, 256 rows)"):
        r = oracle.attention(I.q[heads], I.k[kvs], I.v[kvs], wl.block, oracle.specs_from_index_sets(ref), rows=rows,
                             bias_offsets=I.bias_offsets[heads], bias_values=I.bias_values[heads], chunk=512)
    err = np.abs(o - r).max()
    log("1m max-abs", err)
    assert np.isfinite(o).all() and err <= TOL["bf16"]
