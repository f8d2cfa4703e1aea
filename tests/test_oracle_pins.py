"""Pins for the CPU oracle against what the pages and mathematics fix.

Every check here compares the oracle with something other than itself: closed
forms, hand-derived cases of Eq. 3 / Eq. 4 (tests/golden), an fp64 softmax,
library routines, brute force on tiny inputs and the invariants the pages state
(CRISP summary page, Methodology and Theoretical Implications).
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
FIX = 2 ** 40


# ------------------------------------------------------------------ exp ----
def test_exp_crisp_exact_at_zero_and_cutoff(oracle_lib):
    assert oracle.exp_crisp(np.float32(0.0)) == np.float32(1.0)
    assert oracle.exp_crisp(np.float32(-80.5)) == 0.0
    assert oracle.exp_crisp(np.float32(-1e30)) == 0.0


def test_exp_crisp_within_2ulp_of_exp(oracle_lib):
    rng = np.random.default_rng(1)
    x = np.concatenate([
        rng.uniform(-80.0, 0.0, 400000),
        -np.arange(0, 116) * np.log(2.0),  # range-reduction boundaries k ln2
        -(np.arange(0, 116) + 0.5) * np.log(2.0),  # half-way points
        -rng.uniform(0, 1e-3, 2000), [-80.0, -0.0, -1e-30],
    ]).astype(np.float32)
    x = x[x >= -80.0]  # the routine returns 0 below -80 by definition
    y = oracle.exp_crisp(x).astype(np.float64)
    ref = np.exp(x.astype(np.float64))
    ulp = np.spacing(ref.astype(np.float32)).astype(np.float64)
    err = np.abs(y - ref) / ulp
    assert err.max() <= 2.0, f"max error {err.max()} ulp at x={x[err.argmax()]}"
    # monotone: exp is non-decreasing in x
    order = np.argsort(x, kind="stable")
    assert np.all(np.diff(y[order]) >= 0)


# --------------------------------------------------------- proxy / Eq. 2 --
def _closed_form_uniform(n, B, w_sink, w_local):
    """Q = 0 makes every proxy score 0: e = 1, L_i = (i+1) 2^40, A[i, j] = fl32(1/(i+1))."""
    nb = (n + B - 1) // B
    q0 = (nb - 1) * B
    mv = np.zeros(nb, np.int64)
    ms = np.zeros(nb, np.int64)
    cn = 0
    L = []
    for i in range(q0, n):
        a = np.float32(1.0) / np.float32(i + 1)
        aq = int(np.rint(np.float64(a) * FIX))
        L.append((i + 1) * FIX)
        for b in range(nb):
            # keys j <= i with j // B == b; offsets o = i - j in [0, i] with o // B == b
            cnt = max(0, min(i, (b + 1) * B - 1) - b * B + 1)
            mv[b] += cnt * aq
            ms[b] += cnt * aq
        sink = min(w_sink, i + 1)
        local = min(w_local, i + 1)
        both = max(0, min(w_sink - 1, i) - max(0, i - w_local + 1) + 1)
        cn += (sink + local - both) * aq
    return mv, ms, cn, np.array(L, np.int64)


@pytest.mark.parametrize("n,B,w", [(1000, 64, 64), (4096, 64, 64), (130, 64, 64), (700, 128, 96), (64, 64, 64),
                                   (1, 64, 64)])
def test_proxy_closed_form_zero_queries(oracle_lib, n, B, w):
    rng = np.random.default_rng(n)
    d = 32
    k = rng.standard_normal((2, n, d)).astype(np.float32)
    q = np.zeros((4, n, d), np.float32)
    pr = oracle.proxy(q, k, B, w, w, (1, 10))
    mv, ms, cn, L = _closed_form_uniform(n, B, w, w)
    qrows = pr["qrows"]
    for h in range(4):
        assert np.all(pr["m"][h] == 0.0)
        np.testing.assert_array_equal(pr["L"][h], L)
        np.testing.assert_array_equal(pr["mass_v"][h], mv)
        np.testing.assert_array_equal(pr["mass_s"][h], ms)
        assert pr["cnum"][h] == cn
        assert pr["total"][h] == mv.sum()
        cstruct = cn / (qrows * FIX)
        assert pr["route"][h] == (1 if cstruct >= 0.1 else 0)
        # every middle block of either direction holds exactly the same mass (B keys per
        # proxy row), which equals the floor mu of Eq. 3, so the strict test of Eq. 4
        # keeps nothing but the first and last block
        nb = len(mv)
        want = list(range(nb)) if nb <= 2 else [0, nb - 1]
        assert oracle.vs_select(pr["mass_v"][h], pr["total"][h]).tolist() == want
        assert oracle.vs_select(pr["mass_s"][h], pr["total"][h]).tolist() == want


def test_proxy_matches_fp64_softmax(oracle_lib):
    """The quantised proxy map equals the exact softmax of the last query block within fp32 error."""
    wl = synth.WORKLOADS["tiny"]
    I = synth.make_inputs(wl)
    pr = oracle.proxy(I.q, I.k, wl.block, wl.w_sink, wl.w_local, synth.TAU, I.bias_offsets, I.bias_values,
                      want_aq=True)
    n, d, B = wl.n, wl.d, wl.block
    q0 = n - pr["qrows"]
    for h in range(wl.hq):
        qh = I.q[h, q0:].astype(np.float64)
        K = I.k[h // (wl.hq // wl.hkv)].astype(np.float64)
        z = qh @ K.T / math.sqrt(d)
        i = np.arange(q0, n)[:, None]
        j = np.arange(n)[None, :]
        for off, val in zip(I.bias_offsets[h], I.bias_values[h]):
            z = z + val * ((i - j) == off)
        z = np.where(j <= i, z, -np.inf)
        P = np.exp(z - z.max(1, keepdims=True))
        P /= P.sum(1, keepdims=True)
        A = pr["A_q"][h] / FIX
        assert np.abs(A - P).max() < 5e-6
        # rows of the quantised map sum to one within rounding
        assert np.abs(pr["A_q"][h].sum(1) - FIX).max() < 1e-6 * FIX


def test_proxy_pooling_recount(oracle_lib):
    """Block masses and anchor mass re-counted from the quantised map with the definitions."""
    rng = np.random.default_rng(5)
    n, d, B, ws, wlc = 1000, 16, 64, 100, 70
    q = (rng.standard_normal((2, n, d)) * 2).astype(np.float32)
    k = rng.standard_normal((1, n, d)).astype(np.float32)
    offs = np.array([[0, 3, 200], [5, -1, -1]], np.int32)
    vals = np.array([[2.0, 1.0, 3.0], [4.0, 0.0, 0.0]], np.float32)
    pr = oracle.proxy(q, k, B, ws, wlc, (1, 10), offs, vals, want_aq=True)
    nb = pr["nb"]
    q0 = n - pr["qrows"]
    for h in range(2):
        mv = np.zeros(nb, np.int64)
        ms = np.zeros(nb, np.int64)
        cn = 0
        for r in range(pr["qrows"]):
            i = q0 + r
            row = pr["A_q"][h, r]
            j = np.arange(i + 1)
            np.add.at(mv, j // B, row[: i + 1])
            np.add.at(ms, (i - j) // B, row[: i + 1])
            cn += int(row[: i + 1][(j < ws) | (i - j < wlc)].sum())
            assert np.all(row[i + 1:] == 0)
        np.testing.assert_array_equal(pr["mass_v"][h], mv)
        np.testing.assert_array_equal(pr["mass_s"][h], ms)
        assert pr["cnum"][h] == cn
        assert pr["mass_v"][h].sum() == pr["mass_s"][h].sum() == pr["total"][h]


@pytest.mark.parametrize("name", ["tiny", "llama_32k", "llama_64k", "llama_128k", "qwen_128k", "llama_256k", "llama_512k"])
def test_routing_planted_vs_high_entropy(oracle_lib, name):
    """Low-entropy (planted) heads route to VS, i.i.d. heads to pooled estimation (Eq. 2 + routing rule)."""
    wl = synth.WORKLOADS[name]
    I = synth.make_inputs(wl, with_v=False, q_last_block_only=True)
    pr = oracle.proxy(I.q, I.k, wl.block, wl.w_sink, wl.w_local, synth.TAU, I.bias_offsets, I.bias_values)
    expect = np.array([1 if h in wl.planted_heads else 0 for h in range(wl.hq)], np.uint8)
    np.testing.assert_array_equal(pr["route"], expect)
    cs = pr["cnum"] / (pr["qrows"] * FIX)
    planted = np.array(wl.planted_heads)
    other = np.setdiff1d(np.arange(wl.hq), planted)
    assert cs[planted].min() > 3 * 0.1 and cs[other].max() < 0.1 / 3  # both margins >= 3x tau
    sink_share = pr["mass_v"][planted, 0] / pr["total"][planted]
    if name == "qwen_128k":
        assert sink_share.min() > 0.90  # "sinks hold >90% of the mass"
        # sink-only collapse of the cumulative rule; the noise floor keeps the signal
        G = wl.hq // wl.hkv
        for h in planted:
            nb = pr["nb"]
            cum = oracle.cumulative_select(pr["mass_v"][h], pr["total"][h], synth.GAMMA)
            np.testing.assert_array_equal(cum, [0, nb - 1])
            crisp = set(oracle.vs_select(pr["mass_v"][h], pr["total"][h], synth.ALPHA).tolist())
            planted_blocks = set((I.verticals[h // G] // wl.block).tolist())
            assert len(crisp & planted_blocks) >= 0.8 * len(planted_blocks)


# ----------------------------------------------------- Eq. 3 / Eq. 4 -----
def _golden():
    with open(os.path.join(GOLDEN, "selection_cases.json")) as f:
        return json.load(f)


@pytest.mark.parametrize("case", _golden()["vs_select"], ids=lambda c: c["name"])
def test_vs_select_golden(oracle_lib, case):
    got = oracle.vs_select(np.array(case["p"], np.int64), case["T"], tuple(case["alpha"]))
    assert got.tolist() == case["expect"], case["why"]


@pytest.mark.parametrize("case", _golden()["cumulative_select"], ids=lambda c: c["name"])
def test_cumulative_select_golden(oracle_lib, case):
    got = oracle.cumulative_select(np.array(case["p"], np.int64), case["T"], tuple(case["gamma"]))
    assert got.tolist() == case["expect"], case["why"]


def test_vs_select_exact_threshold_large_values(oracle_lib):
    """Equality at fixed-point scale near the int64 range: strictly greater is required."""
    nb = 4098
    p = np.zeros(nb, np.int64)
    p[0] = 3 << 45
    mid = (1 << 45) - 4096 * 7
    p[1:nb - 1] = mid // (nb - 2)
    p[1] = p[2] = mid // (nb - 2)  # equal to the floor: not selected
    T = int(p.sum())
    M = T - p[0] - p[-1]
    got = oracle.vs_select(p, T, (1, 1))
    floor_eq = [b for b in range(1, nb - 1) if (nb - 2) * int(p[b]) > M]
    assert got.tolist() == [0] + floor_eq + [nb - 1]
    p2 = p.copy()
    p2[7] += 1  # one unit above the floor mass is selected
    got2 = oracle.vs_select(p2, int(p2.sum()), (1, 1))
    assert 7 in got2.tolist()


def test_cumulative_prefix_is_minimal_bruteforce(oracle_lib):
    rng = np.random.default_rng(3)
    for trial in range(60):
        nb = int(rng.integers(3, 11))
        p = rng.integers(0, 50, nb).astype(np.int64)
        if trial % 3 == 0:
            p[rng.integers(0, nb)] = p.max()  # force ties
        T = int(p.sum())
        g = (int(rng.integers(1, 20)), 20)
        got = set(oracle.cumulative_select(p, T, g).tolist()) - {0, nb - 1}
        # the shortest subset reaching gamma T, by brute force
        kmin = None
        for k in range(0, nb + 1):
            if any(g[1] * sum(p[list(c)]) >= g[0] * T for c in itertools.combinations(range(nb), k)):
                kmin = k
                break
        # the oracle's prefix (before adding first/last) has kmin elements: recover it by size
        full = oracle.cumulative_select(p, T, g)
        order = sorted(range(nb), key=lambda b: (-p[b], b))
        prefix = set(order[:kmin])
        assert set(full.tolist()) == prefix | {0, nb - 1}
        assert got <= prefix


def test_noise_floor_does_not_grow_with_background():
    """Mass-cliff invariant (Theoretical Implications): with the signal fixed, the
    sink-aware rule selects no background block at any length, while the
    cumulative rule's count grows with n."""
    base = synth.Workload(name="sweep", hq=1, hkv=1, d=64, n=2048, dtype="f32", block=64, rope_theta=0.0,
                          seed=77, planted_heads=[0], sink_gain=2.0, vertical_gain=(3.0, 3.0),
                          fixed_verticals=(200, 333, 700, 1000, 1300, 1500, 1700, 1900), fixed_slash=(0,))
    crisp_counts, cum_counts = [], []
    for n in (2048, 4096, 8192, 16384, 32768):
        wl = base.replace(n=n)
        I = synth.make_inputs(wl, with_v=False, q_last_block_only=True)
        pr = oracle.proxy(I.q, I.k, wl.block, wl.w_sink, wl.w_local, synth.TAU, I.bias_offsets, I.bias_values)
        nb = pr["nb"]
        sel = set(oracle.vs_select(pr["mass_v"][0], pr["total"][0], synth.ALPHA).tolist())
        allowed = {0, nb - 2, nb - 1} | set((np.array(base.fixed_verticals) // wl.block).tolist())
        assert sel <= allowed, sorted(sel - allowed)
        crisp_counts.append(len(sel))
        cum_counts.append(len(oracle.cumulative_select(pr["mass_v"][0], pr["total"][0], synth.GAMMA)))
    assert max(crisp_counts) - min(crisp_counts) <= 1
    assert all(b > a for a, b in zip(cum_counts, cum_counts[1:]))
    assert cum_counts[-1] > 8 * cum_counts[0] / 2


def test_sink_only_collapse_tiny(oracle_lib):
    wl = synth.WORKLOADS["tiny"]
    I = synth.make_inputs(wl, with_v=False, q_last_block_only=True)
    pr = oracle.proxy(I.q, I.k, wl.block, wl.w_sink, wl.w_local, synth.TAU, I.bias_offsets, I.bias_values)
    nb = pr["nb"]
    assert pr["mass_v"][0, 0] / pr["total"][0] > 0.95
    cum = oracle.cumulative_select(pr["mass_v"][0], pr["total"][0], synth.GAMMA)
    np.testing.assert_array_equal(cum, [0, nb - 1])
    sel = set(oracle.vs_select(pr["mass_v"][0], pr["total"][0], synth.ALPHA).tolist())
    assert set((I.verticals[0] // wl.block).tolist()) <= sel


# ------------------------------------------------------------- Alg. 4 ----
@pytest.mark.parametrize("n,B", [(1000, 64), (64 * 16, 64), (300, 128), (5, 64)])
def test_pe_index_uniform_closed_form(oracle_lib, n, B):
    """Q = K = 0: every pooled row is uniform, A[qb, kb] = fl32(1/(qb+1)); the
    order is rows ascending (values strictly decrease), kb ascending within a row."""
    d = 16
    q = np.zeros((n, d), np.float32)
    k = np.zeros((n, d), np.float32)
    g = (19, 20)
    rowptr, cols, abar, tbar, taken = oracle.pe_index(q, k, B, g, want_abar=True)
    nb = (n + B - 1) // B
    vals = [int(np.rint(np.float64(np.float32(1.0) / np.float32(qb + 1)) * FIX)) for qb in range(nb)]
    expect_abar = np.concatenate([[vals[qb]] * (qb + 1) for qb in range(nb)])
    np.testing.assert_array_equal(abar, expect_abar)
    T = sum((qb + 1) * vals[qb] for qb in range(nb))
    assert tbar == T
    keep = [[False] * (qb + 1) for qb in range(nb)]
    cum, cnt = 0, 0
    for qb in range(nb):
        for kb in range(qb + 1):
            if g[1] * cum >= g[0] * T:
                break
            cum += vals[qb]
            cnt += 1
            keep[qb][kb] = True
    assert taken == cnt
    for qb in range(nb):
        keep[qb][qb] = True
        assert cols[rowptr[qb]:rowptr[qb + 1]].tolist() == [kb for kb in range(qb + 1) if keep[qb][kb]]


def test_pe_index_matches_fp64_pooled_softmax(oracle_lib):
    rng = np.random.default_rng(11)
    n, d, B = 2000, 32, 64
    q = (rng.standard_normal((n, d)) * 3).astype(np.float32)
    k = (rng.standard_normal((n, d)) * 3).astype(np.float32)
    rowptr, cols, abar, tbar, taken = oracle.pe_index(q, k, B, (19, 20), want_abar=True)
    nb = (n + B - 1) // B
    Qb = np.array([q[b * B:(b + 1) * B].astype(np.float64).mean(0) for b in range(nb)])
    Kb = np.array([k[b * B:(b + 1) * B].astype(np.float64).mean(0) for b in range(nb)])
    z = Qb @ Kb.T / math.sqrt(d)
    z = np.where(np.tri(nb, dtype=bool), z, -np.inf)
    P = np.exp(z - z.max(1, keepdims=True))
    P /= P.sum(1, keepdims=True)
    flat = np.concatenate([P[qb, :qb + 1] for qb in range(nb)])
    assert np.abs(abar / FIX - flat).max() < 2e-6
    assert abs(tbar - nb * FIX) < 1e-6 * nb * FIX  # "flatten and normalise": rows sum to one


def test_pe_index_minimal_prefix_bruteforce(oracle_lib):
    rng = np.random.default_rng(12)
    for trial in range(12):
        B = 8
        nb = int(rng.integers(2, 6))
        n = nb * B - int(rng.integers(0, B))
        q = (rng.standard_normal((n, 8)) * rng.uniform(0.5, 6)).astype(np.float32)
        k = (rng.standard_normal((n, 8)) * rng.uniform(0.5, 6)).astype(np.float32)
        nb = (n + B - 1) // B
        g = (int(rng.integers(10, 20)), 20)
        rowptr, cols, abar, tbar, taken = oracle.pe_index(q, k, B, g, want_abar=True)
        ntri = nb * (nb + 1) // 2
        kmin = None
        for kk in range(ntri + 1):
            if any(g[1] * int(abar[list(c)].sum()) >= g[0] * tbar for c in itertools.combinations(range(ntri), kk)):
                kmin = kk
                break
        assert taken == kmin
        kept = set()
        for qb in range(nb):
            for kb in cols[rowptr[qb]:rowptr[qb + 1]]:
                kept.add(qb * (qb + 1) // 2 + int(kb))
        diag = {qb * (qb + 1) // 2 + qb for qb in range(nb)}
        # every kept off-prefix element is a diagonal; every dropped value <= every prefix value
        assert len(kept) >= taken
        dropped = set(range(ntri)) - kept
        prefix_candidates = kept - (diag - kept)
        if dropped:
            assert max(abar[list(dropped)]) <= max(abar[list(prefix_candidates)])
        assert diag <= kept


# ---------------------------------------------------- masked attention ---
def _rand_qkv(rng, bh, bkv, n, d):
    q = rng.standard_normal((bh, n, d)).astype(np.float32)
    k = rng.standard_normal((bkv, n, d)).astype(np.float32)
    v = rng.standard_normal((bkv, n, d)).astype(np.float32)
    return q, k, v


def test_attention_zero_queries_is_prefix_mean():
    rng = np.random.default_rng(21)
    n, d, B = 300, 16, 64
    _, k, v = _rand_qkv(rng, 1, 1, n, d)
    q = np.zeros((2, n, d), np.float32)
    specs = [dict(kind="dense"), dict(kind="vs", vertical=np.array([0, 2, 4]), slash=np.array([0]))]
    out = oracle.attention(q, k, v, B, specs)
    pm = np.cumsum(v[0].astype(np.float64), 0) / np.arange(1, n + 1)[:, None]
    np.testing.assert_allclose(out[0], pm, rtol=0, atol=1e-12)
    # masked: mean over the allowed keys only
    for i in (0, 70, 150, 299):
        allowed = [j for j in range(i + 1) if (j // B) in (0, 2, 4) or (i - j) // B == 0]
        np.testing.assert_allclose(out[1, i], v[0, allowed].astype(np.float64).mean(0), atol=1e-12)


def test_attention_single_token():
    rng = np.random.default_rng(22)
    q, k, v = _rand_qkv(rng, 1, 1, 1, 8)
    out = oracle.attention(q, k, v, 64, [dict(kind="dense")])
    np.testing.assert_allclose(out[0, 0], v[0, 0], atol=0)


def test_attention_dense_matches_torch_sdpa():
    import torch
    rng = np.random.default_rng(23)
    q, k, v = _rand_qkv(rng, 4, 2, 257, 32)
    out = oracle.attention(q, k, v, 64, [dict(kind="dense")] * 4)
    Q = torch.from_numpy(q).double()[None]
    K = torch.from_numpy(k).double().repeat_interleave(2, 0)[None]
    V = torch.from_numpy(v).double().repeat_interleave(2, 0)[None]
    ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, is_causal=True)[0].numpy()
    np.testing.assert_allclose(out, ref, atol=1e-12, rtol=0)


def test_attention_matches_loop_writing_with_masks_and_bias():
    rng = np.random.default_rng(24)
    n, d, B = 333, 16, 32
    q, k, v = _rand_qkv(rng, 3, 1, n, d)
    offs = np.array([[0, 40, -1], [3, -1, -1], [-1, -1, -1]], np.int32)
    vals = np.array([[2.5, 1.0, 0.0], [3.0, 0.0, 0.0], [0.0, 0.0, 0.0]], np.float32)
    nb = (n + B - 1) // B
    rowptr = [0]
    cols = []
    for qb in range(nb):
        c = sorted(set(rng.choice(qb + 1, size=min(qb + 1, 3), replace=False).tolist()) | {qb})
        cols += c
        rowptr.append(len(cols))
    specs = [dict(kind="vs", vertical=np.array([0, 3, 7]), slash=np.array([0, 2, 5])),
             dict(kind="pe", rowptr=np.array(rowptr), cols=np.array(cols)), dict(kind="dense")]
    rows = np.array([0, 1, 31, 32, 100, 200, 250, 332])
    out = oracle.attention(q, k, v, B, specs, rows=rows, bias_offsets=offs, bias_values=vals)
    for h in range(3):
        for t, i in enumerate(rows):
            j = np.arange(n)
            if specs[h]["kind"] == "vs":
                al = np.isin(j // B, [0, 3, 7]) | np.isin(np.maximum(i - j, 0) // B, [0, 2, 5])
            elif specs[h]["kind"] == "pe":
                al = np.isin(j // B, cols[rowptr[i // B]:rowptr[i // B + 1]])
            else:
                al = np.ones(n, bool)
            ref = oracle.attention_row_loop(i, q[h, i], k[0], v[0], offs[h], vals[h], al & (j <= i))
            np.testing.assert_allclose(out[h, t], ref, atol=1e-12, rtol=0)


def test_mask_bruteforce_enumeration():
    import torch
    n, B = 200, 32
    nb = (n + B - 1) // B
    V, S = [0, 3], [0, 2]
    rp, cl = [0], []
    for qb in range(nb):
        cl += sorted({0, qb, qb // 2})
        rp.append(len(cl))
    rows = torch.arange(n)
    j = torch.arange(n)
    mvs = oracle._allowed(dict(kind="vs", vertical=V, slash=S), rows, j, B, nb).numpy()
    mpe = oracle._allowed(dict(kind="pe", rowptr=rp, cols=cl), rows, j, B, nb).numpy()
    for i in range(n):
        for jj in range(n):
            e_vs = jj <= i and ((jj // B) in V or ((i - jj) // B) in S)
            e_pe = jj <= i and (jj // B) in cl[rp[i // B]:rp[i // B + 1]]
            assert mvs[i, jj] == e_vs and mpe[i, jj] == e_pe


def test_keep_all_equals_dense_bitwise(oracle_lib):
    """Alg. 1 with every block kept is exactly dense causal attention."""
    rng = np.random.default_rng(25)
    n, d, B = 500, 16, 64
    q, k, v = _rand_qkv(rng, 2, 1, n, d)
    offs = np.array([[0, 7], [1, -1]], np.int32)
    vals = np.array([[1.0, 2.0], [0.5, 0.0]], np.float32)
    isets = oracle.index_sets(q, k, B, B, B, keep_all=True, bias_offsets=offs, bias_values=vals)
    specs = oracle.specs_from_index_sets(isets)
    out = oracle.attention(q, k, v, B, specs, bias_offsets=offs, bias_values=vals)
    dense = oracle.attention(q, k, v, B, [dict(kind="dense")] * 2, bias_offsets=offs, bias_values=vals)
    assert np.array_equal(out, dense)


def test_generator_bf16_storage():
    wl = synth.WORKLOADS["llama_32k"].replace(n=1024, hq=4, hkv=1, planted_heads=[0, 1])
    I = synth.make_inputs(wl)
    for a in (I.q, I.k, I.v):
        assert np.all((a.view(np.uint32) & 0xFFFF) == 0)
    bits = synth.to_bf16_bits(I.q)
    assert np.array_equal((bits.astype(np.uint32) << 16).view(np.float32), I.q)


def test_generator_qk_scale():
    """The degenerate-input variants: Q and K scaled exactly (still bf16 values), or zero."""
    wl = synth.WORKLOADS["llama_32k"].replace(n=600, hq=4, hkv=2, planted_heads=[0])
    base = synth.make_inputs(wl)
    big = synth.make_inputs(wl.replace(qk_scale=16.0))
    zero = synth.make_inputs(wl.replace(qk_scale=0.0))
    assert np.array_equal(big.q, base.q * 16) and np.array_equal(big.k, base.k * 16)
    assert np.array_equal(big.v, base.v) and np.array_equal(zero.v, base.v)
    assert not zero.q.any() and not zero.k.any()
    assert np.all((big.q.view(np.uint32) & 0xFFFF) == 0)
    with pytest.raises(AssertionError):
        synth.make_inputs(wl.replace(qk_scale=3.0))


# -------------------------------------------------------- divergence router ----
def test_log_crisp_within_3ulp_of_log(oracle_lib):
    """Measured bound of the reduction + atanh series: 3 ulp where ln x is small against x
    (m just above 1), 2 ulp elsewhere."""
    rng = np.random.default_rng(31)
    x = np.concatenate([
        np.exp(rng.uniform(-690.0, 690.0, 200000)),  # wide exponent range
        rng.uniform(0.5, 2.0, 200000),  # around the reduction boundaries
        1.0 + rng.uniform(-1e-6, 1e-6, 20000),  # near the zero of ln
        np.sqrt(2.0) * (1.0 + np.arange(-50, 51) * 2.0 ** -52),  # the sqrt(2) switch
        2.0 ** np.arange(-1020, 1020, dtype=np.float64), [1.0, 2.0, 0.5, math.e],
    ])
    y = oracle.log_crisp(x)
    ref = np.log(x)
    assert oracle.log_crisp(np.array([1.0]))[0] == 0.0  # exact zero keeps identical distributions at JSD 0
    ulp = np.spacing(np.abs(ref))
    err = np.abs(y - ref)
    # near x = 1 the result is tiny: measure those against the ulp of x - 1 instead
    bound = np.where(np.abs(ref) < 1e-3, np.spacing(np.abs(x - 1.0) + 1e-300) * 4, 3 * ulp)
    assert np.all(err <= bound), (x[err > bound][:5], err[err > bound][:5])


def _rand_fixed(rng, nb, zero_frac=0.0, total=128 * FIX):
    w = rng.gamma(0.3, 1.0, nb)
    w[rng.random(nb) < zero_frac] = 0.0
    if w.sum() == 0:
        w[0] = 1.0
    return np.floor(w / w.sum() * total).astype(np.int64)


def test_jsd_matches_scipy_jensenshannon(oracle_lib):
    from scipy.spatial.distance import jensenshannon
    rng = np.random.default_rng(32)
    for trial in range(60):
        nb = int(rng.integers(2, 3000))
        p = _rand_fixed(rng, nb, zero_frac=0.2 if trial % 3 == 0 else 0.0)
        a = _rand_fixed(rng, nb, zero_frac=0.3 if trial % 4 == 1 else 0.0, total=FIX)
        J = oracle.jsd_fixed(p, p.sum(), a, a.sum())
        ref = jensenshannon(p / p.sum(), a / a.sum()) ** 2  # scipy returns the distance (square root)
        assert abs(J * 2.0 ** -53 - ref) < 1e-12, (trial, J * 2.0 ** -53, ref)


def test_jsd_closed_forms(oracle_lib):
    # identical distributions: zero exactly
    rng = np.random.default_rng(33)
    p = _rand_fixed(rng, 500)
    assert oracle.jsd_fixed(p, p.sum(), p, p.sum()) == 0
    # the same distribution at another scale is still identical
    assert oracle.jsd_fixed(p, p.sum(), 4 * p, 4 * p.sum()) == 0
    # disjoint supports: ln 2
    a = np.zeros_like(p)
    a[p == 0] = 1
    p2 = p.copy()
    p2[:] = 0
    p2[:250] = 3
    a2 = np.zeros_like(p)
    a2[250:] = 7
    J = oracle.jsd_fixed(p2, p2.sum(), a2, a2.sum())
    # each of the N_b terms is rounded to 2^-52 once: JSD moves by at most N_b 2^-54
    assert abs(J * 2.0 ** -53 - math.log(2.0)) <= len(p2) * 2.0 ** -54 + 1e-15
    # two points: P = (x, 1-x), Q = (y, 1-y), written out
    for x, y in ((0.25, 0.75), (0.5, 0.125), (0.9, 0.1), (1e-6, 0.5)):
        P = np.array([x, 1 - x])
        Q = np.array([y, 1 - y])
        M = (P + Q) / 2
        ref = 0.5 * np.sum(P * np.log(P / M)) + 0.5 * np.sum(Q * np.log(Q / M))
        pf = np.array([round(x * FIX), FIX - round(x * FIX)], np.int64)
        qf = np.array([round(y * FIX), FIX - round(y * FIX)], np.int64)
        J = oracle.jsd_fixed(pf, FIX, qf, FIX)
        assert abs(J * 2.0 ** -53 - ref) < 1e-11, (x, y)
    # symmetric, bit for bit
    q = _rand_fixed(rng, 500, total=FIX)
    assert oracle.jsd_fixed(p, p.sum(), q, q.sum()) == oracle.jsd_fixed(q, q.sum(), p, p.sum())


@pytest.mark.parametrize("n,B", [(1000, 64), (4096, 64), (300, 128)])
def test_pooled_row_is_last_row_of_pe_map(oracle_lib, n, B):
    """The divergence router's pooled estimate is Alg. 4's pooled map at the last query block."""
    rng = np.random.default_rng(34)
    d = 32
    q = (rng.standard_normal((n, d)) * 2).astype(np.float32)
    k = (rng.standard_normal((n, d)) * 2).astype(np.float32)
    abar, ta = oracle.pooled_last_row(q, k, B)
    _, _, full, _, _ = oracle.pe_index(q, k, B, (19, 20), want_abar=True)
    nb = (n + B - 1) // B
    assert np.array_equal(abar, full[nb * (nb - 1) // 2:])
    assert ta == abar.sum()
    # Q = 0: every pooled score is 0, so the estimate is uniform: rne(fl(1/N_b) 2^40)
    z, _ = oracle.pooled_last_row(np.zeros_like(q), k, B)
    assert np.all(z == np.int64(np.rint(np.float32(1.0) / np.float32(nb) * np.float64(FIX))))


def test_jsd_route_matches_fp64_writing_and_separates_heads(oracle_lib):
    """The router end to end on the small planted layer against a plain fp64 writing of
    the same definitions; the planted head diverges, the i.i.d. head does not."""
    wl = synth.WORKLOADS["tiny"]
    I = synth.make_inputs(wl)
    B, nb = wl.block, (wl.n + wl.block - 1) // wl.block
    pr = oracle.proxy(I.q, I.k, B, wl.w_sink, wl.w_local, synth.TAU, I.bias_offsets, I.bias_values)
    out = oracle.jsd_route(I.q, I.k, B, pr)
    G = wl.hq // wl.hkv
    for h in range(wl.hq):
        q = I.q[h].astype(np.float64)
        k = I.k[h // G].astype(np.float64)
        qbar = q[(nb - 1) * B:].mean(0)
        kbar = np.stack([k[b * B:(b + 1) * B].mean(0) for b in range(nb)])
        z = kbar @ qbar / math.sqrt(wl.d)
        Q = np.exp(z - z.max())
        Q /= Q.sum()
        P = pr["mass_v"][h] / pr["total"][h]
        M = (P + Q) / 2
        ref = 0.5 * np.sum(P[P > 0] * np.log(P[P > 0] / M[P > 0])) + 0.5 * np.sum(Q * np.log(Q / M))
        got = out["jsd"][h] * 2.0 ** -53
        assert abs(got - ref) < 1e-6 * max(ref, 1e-3), (h, got, ref)
        assert np.abs(out["abar"][h] / out["abar_total"][h] - Q).max() < 1e-6
    assert out["route"].tolist() == [1 if h in wl.planted_heads else 0 for h in range(wl.hq)]
    assert out["route"].tolist() == pr["route"].tolist()

