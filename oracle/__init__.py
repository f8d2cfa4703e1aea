"""CPU oracle for the CRISP sparse-prefill path.  TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package; the GPU library never does, and the two
share no code.

Two parts:

* ``crisp_oracle.c`` (built to ``liboracle.so``): the steps whose results are
  decisions (proxy map, C_struct routing, sink-aware selection, the
  cumulative-gamma baseline, the pooled-estimation index).  They use the
  exactly specified fp32 / int64 fixed-point arithmetic described in that
  file, so the GPU must reproduce them bit for bit.
* attention in fp64 with plain PyTorch CPU operations (matmul, masked softmax),
  the textbook definition: softmax over allowed keys of (q.k)/sqrt(d) + bias,
  times V.  Outputs are compared within a tolerance, so no bit-level contract.

Citations are to the CRISP summary page (picx.dev), "Methodology" section:
Eq. 2 (C_struct), Eq. 3 (noise floor), Eq. 4 (selection rule), and the
algorithm overview (Alg. 1 pipeline, Alg. 2 PatSearch, Alg. 3 VS index,
Alg. 4 PE index).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

FIX = 2 ** 40


def build(force: bool = False) -> str:
    src = os.path.join(_HERE, "crisp_oracle.c")
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(src):
        subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-mfma", "-fopenmp", "-fPIC", "-shared",
                               src, "-o", _LIB_PATH, "-lm"])
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        # CRISP_ORACLE_LIB: another build of the same source (the sanitizer test loads one)
        path = os.environ.get("CRISP_ORACLE_LIB") or _LIB_PATH
        if path == _LIB_PATH and not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(path)
        P, i32, i64, u32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32
        lib.oracle_exp_crisp.argtypes = [ctypes.c_float]
        lib.oracle_exp_crisp.restype = ctypes.c_float
        lib.oracle_exp_crisp_array.argtypes = [P, P, i64]
        lib.oracle_exp_crisp_array.restype = None
        lib.oracle_scale.argtypes = [i32]
        lib.oracle_scale.restype = ctypes.c_float
        lib.oracle_proxy.argtypes = [i32, i32, i64, i32, i32, i32, i32, u32, u32, P, P, i32, P, P, P, P,
                                     P, P, P, P, P, P]
        lib.oracle_proxy.restype = ctypes.c_int
        lib.oracle_vs_select.argtypes = [i64, P, i64, u32, u32, P]
        lib.oracle_vs_select.restype = i32
        lib.oracle_cumulative_select.argtypes = [i64, P, i64, u32, u32, P]
        lib.oracle_cumulative_select.restype = i32
        lib.oracle_pe_index.argtypes = [i64, i32, i32, P, P, u32, u32, P, P, P, P, i32]
        lib.oracle_pe_index.restype = i64
        lib.oracle_attention_row.argtypes = [i64, i32, P, P, P, i32, P, P, P, P]
        lib.oracle_attention_row.restype = None
        lib.oracle_log_crisp.argtypes = [ctypes.c_double]
        lib.oracle_log_crisp.restype = ctypes.c_double
        lib.oracle_log_crisp_array.argtypes = [P, P, i64]
        lib.oracle_log_crisp_array.restype = None
        lib.oracle_jsd_fixed.argtypes = [i64, P, i64, P, i64]
        lib.oracle_jsd_fixed.restype = i64
        lib.oracle_pooled_last_row.argtypes = [i64, i32, i32, P, P, P]
        lib.oracle_pooled_last_row.restype = i64
        _lib = lib
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dt):
    return np.ascontiguousarray(a, dtype=dt)


def exp_crisp(x) -> np.ndarray:
    lib = _load()
    x = _c(x, np.float32)
    y = np.empty_like(x)
    lib.oracle_exp_crisp_array(_p(x), _p(y), x.size)
    return y


def scale(d: int) -> np.float32:
    return np.float32(_load().oracle_scale(d))


def num_blocks(n: int, B: int) -> int:
    return (n + B - 1) // B


def proxy(q, k, B, w_sink, w_local, tau=(1, 10), bias_offsets=None, bias_values=None, want_aq=False):
    """Alg. 2 with Eq. 2 and the block pooling of Alg. 3.

    q [bh, n, d] (or only its last query block, [bh, qrows, d]), k [bkv, n, d]
    float32.  Returns a dict with per-head arrays:
    m, L (proxy row max / fixed-point row sums), mass_v, mass_s [bh, N_b],
    total [bh], cnum [bh] (fixed-point anchor mass), route [bh] (1 = VS) and,
    if want_aq, A_q [bh, qrows, n] (quantised post-softmax proxy map).
    """
    lib = _load()
    k = _c(k, np.float32)
    bkv, n, d = k.shape
    bh = q.shape[0]
    nb = num_blocks(n, B)
    qrows = n - (nb - 1) * B
    q = _c(q[:, q.shape[1] - qrows:, :], np.float32)
    if bias_offsets is None or bias_offsets.size == 0:
        cnt, bo, bv = 0, None, None
    else:
        bo = _c(bias_offsets, np.int32)
        bv = _c(bias_values, np.float32)
        cnt = bo.shape[1]
    out = dict(m=np.zeros((bh, qrows), np.float32), L=np.zeros((bh, qrows), np.int64),
               mass_v=np.zeros((bh, nb), np.int64), mass_s=np.zeros((bh, nb), np.int64),
               total=np.zeros(bh, np.int64), cnum=np.zeros(bh, np.int64), route=np.zeros(bh, np.uint8))
    aq = np.zeros((bh, qrows, n), np.int64) if want_aq else None
    rc = lib.oracle_proxy(bh, bkv, n, d, B, w_sink, w_local, tau[0], tau[1], _p(q), _p(k), cnt, _p(bo),
                          _p(bv), _p(out["m"]), _p(out["L"]), _p(out["mass_v"]), _p(out["mass_s"]),
                          _p(out["total"]), _p(out["cnum"]), _p(out["route"]), _p(aq))
    if rc != 0:
        raise ValueError("oracle_proxy: bad shape")
    if want_aq:
        out["A_q"] = aq
    out["qrows"] = qrows
    out["nb"] = nb
    return out


def vs_select(p, total, alpha=(1, 1)) -> np.ndarray:
    """Eq. 3 and Eq. 4 for one direction (sink-aware noise floor)."""
    lib = _load()
    p = _c(p, np.int64)
    nb = p.shape[0]
    out = np.zeros(max(nb, 1), np.int32)
    c = lib.oracle_vs_select(nb, _p(p), int(total), alpha[0], alpha[1], _p(out))
    return out[:c].copy()


def cumulative_select(p, total, gamma=(19, 20)) -> np.ndarray:
    """The cumulative-coverage rule the pages contrast with Eq. 4 (baseline only)."""
    lib = _load()
    p = _c(p, np.int64)
    nb = p.shape[0]
    out = np.zeros(max(nb, 1), np.int32)
    c = lib.oracle_cumulative_select(nb, _p(p), int(total), gamma[0], gamma[1], _p(out))
    return out[:c].copy()


def pe_index(qh, kh, B, gamma=(19, 20), want_abar=False, threads=0):
    """Alg. 4 (GlobalAdaptive) for one query head.

    Returns (rowptr, cols) or, with want_abar, (rowptr, cols, Abar_q, Tbar, prefix_len)."""
    lib = _load()
    qh = _c(qh, np.float32)
    kh = _c(kh, np.float32)
    n, d = qh.shape
    nb = num_blocks(n, B)
    ntri = nb * (nb + 1) // 2
    rowptr = np.zeros(nb + 1, np.int32)
    cols = np.zeros(ntri, np.int32)
    abar = np.zeros(ntri, np.int64) if want_abar else None
    tbar = np.zeros(2, np.int64)
    nnz = lib.oracle_pe_index(n, d, B, _p(qh), _p(kh), gamma[0], gamma[1], _p(rowptr), _p(cols),
                              _p(abar), _p(tbar), threads)
    cols = cols[:nnz].copy()
    if want_abar:
        return rowptr, cols, abar, int(tbar[0]), int(tbar[1])
    return rowptr, cols


def index_sets(q, k, B, w_sink, w_local, tau=(1, 10), alpha=(1, 1), gamma=(19, 20),
               bias_offsets=None, bias_values=None, keep_all=False, cumulative=False):
    """Alg. 1 up to the sparse attention: route every head, then its index set.

    Returns dict(proxy=<proxy dict>, heads=[...]) with one entry per query head:
    {"route": 1, "vertical": ids, "slash": ids} or {"route": 0, "rowptr", "cols"}.
    keep_all: every head keeps its complete (causal) index set.
    cumulative: VS heads use the cumulative-coverage rule (cumulative_select with
    gamma) instead of the noise floor; PE heads are unchanged.
    """
    pr = proxy(q, k, B, w_sink, w_local, tau, bias_offsets, bias_values)
    bh = q.shape[0]
    G = bh // k.shape[0]
    nb = pr["nb"]
    pe_heads = [h for h in range(bh) if not pr["route"][h]]
    pe_out = {}
    if not keep_all and pe_heads:
        # independent heads in parallel threads (the C routine releases the GIL)
        import concurrent.futures as cf
        workers = max(1, min(len(pe_heads), os.cpu_count() or 1, 16))
        with cf.ThreadPoolExecutor(workers) as ex:
            futs = {h: ex.submit(pe_index, q[h], k[h // G], B, gamma, False, 1 if workers > 1 else 0)
                    for h in pe_heads}
            pe_out = {h: f.result() for h, f in futs.items()}
    heads = []
    for h in range(bh):
        if pr["route"][h]:
            if keep_all:
                vv = np.arange(nb, dtype=np.int32)
                ss = np.arange(nb, dtype=np.int32)
            elif cumulative:
                vv = cumulative_select(pr["mass_v"][h], pr["total"][h], gamma)
                ss = cumulative_select(pr["mass_s"][h], pr["total"][h], gamma)
            else:
                vv = vs_select(pr["mass_v"][h], pr["total"][h], alpha)
                ss = vs_select(pr["mass_s"][h], pr["total"][h], alpha)
            heads.append(dict(route=1, vertical=vv, slash=ss))
        else:
            if keep_all:
                rowptr = np.concatenate([[0], np.cumsum(np.arange(1, nb + 1))]).astype(np.int32)
                cols = np.concatenate([np.arange(qb + 1) for qb in range(nb)]).astype(np.int32)
            else:
                rowptr, cols = pe_out[h]
            heads.append(dict(route=0, rowptr=rowptr, cols=cols))
    return dict(proxy=pr, heads=heads)


# ------------------------------------------------------ divergence router ---
JSD_SHIFT = 52  # per-block divergence terms are summed as rne(t 2^52); JSD = J 2^-53


def log_crisp(x) -> np.ndarray:
    """Natural logarithm (fp64) by 2^e m reduction and the atanh series."""
    lib = _load()
    x = _c(x, np.float64)
    y = np.empty_like(x)
    lib.oracle_log_crisp_array(_p(x), _p(y), x.size)
    return y


def jsd_fixed(p, tp, a, ta) -> int:
    """J = sum_b rne(t_b 2^52) of the Jensen-Shannon divergence of p / tp and a / ta."""
    p = _c(p, np.int64)
    a = _c(a, np.int64)
    assert p.shape == a.shape
    return int(_load().oracle_jsd_fixed(p.shape[0], _p(p), int(tp), _p(a), int(ta)))


def pooled_last_row(qh, kh, B):
    """The pooled (pool-then-softmax) estimate of one head's last query block over
    key blocks, in the fixed point of Alg. 4.  Returns (abar [N_b] int64, total)."""
    qh = _c(qh, np.float32)
    kh = _c(kh, np.float32)
    n, d = kh.shape
    assert qh.shape == (n, d)
    abar = np.zeros(num_blocks(n, B), np.int64)
    t = _load().oracle_pooled_last_row(n, d, B, _p(qh), _p(kh), _p(abar))
    return abar, int(t)


def jsd_route(q, k, B, pr, tau_jsd=(1, 100)):
    """The divergence router on the same proxy: per query head the pooled estimate,
    its divergence from the per-query estimate p^v / T of the proxy dict pr, and
    the routing decision (1 = VS iff tau_den J >= tau_num 2^53)."""
    bh = q.shape[0]
    G = bh // k.shape[0]
    nb = pr["nb"]
    out = dict(jsd=np.zeros(bh, np.int64), route=np.zeros(bh, np.uint8), abar=np.zeros((bh, nb), np.int64),
               abar_total=np.zeros(bh, np.int64))
    for h in range(bh):
        abar, ta = pooled_last_row(q[h], k[h // G], B)
        J = jsd_fixed(pr["mass_v"][h], pr["total"][h], abar, ta)
        out["abar"][h] = abar
        out["abar_total"][h] = ta
        out["jsd"][h] = J
        out["route"][h] = 1 if tau_jsd[1] * J >= tau_jsd[0] * (1 << (JSD_SHIFT + 1)) else 0
    return out


# ------------------------------------------------------------ attention ----
def _allowed(spec, rows, j, B, nb):
    """Alg. 1 mask for one head: which (row, key) pairs the index set covers (causal)."""
    import torch
    o = rows[:, None] - j[None, :]
    causal = o >= 0
    kind = spec["kind"]
    if kind == "dense":
        return causal
    if kind == "vs":
        inv = torch.zeros(nb, dtype=torch.bool)
        inv[torch.as_tensor(spec["vertical"], dtype=torch.long)] = True
        ins = torch.zeros(nb, dtype=torch.bool)
        ins[torch.as_tensor(spec["slash"], dtype=torch.long)] = True
        vert = inv[j // B][None, :]
        sl = ins[torch.div(torch.clamp(o, min=0).to(torch.int32), B, rounding_mode="floor").long()]
        return causal & (vert | sl)
    if kind == "pe":
        keep = spec.get("_keep")
        if keep is None:
            keep = torch.zeros((nb, nb), dtype=torch.bool)
            rp = spec["rowptr"]
            for qb in range(nb):
                keep[qb, torch.as_tensor(spec["cols"][rp[qb]:rp[qb + 1]], dtype=torch.long)] = True
            spec["_keep"] = keep
        return causal & keep[(rows // B)[:, None], (j // B)[None, :]]
    raise ValueError(kind)


def attention(q, k, v, B, specs, rows=None, bias_offsets=None, bias_values=None, chunk=256, heads=None):
    """Masked causal attention in fp64 (plain PyTorch CPU ops).

    q [bh, n, d], k/v [bkv, n, d] (float32 values).  specs: one dict per query
    head, {"kind": "dense"} or {"kind": "vs", "vertical", "slash"} or
    {"kind": "pe", "rowptr", "cols"}.  rows: query rows to evaluate (default
    all); heads: query heads to evaluate (default all).  Returns float64
    [len(heads), len(rows), d].
    """
    import torch
    bh, n, d = q.shape
    G = bh // k.shape[0]
    nb = num_blocks(n, B)
    rows = np.arange(n) if rows is None else np.asarray(rows)
    heads = list(range(bh)) if heads is None else list(heads)
    rows_t = torch.as_tensor(rows, dtype=torch.long)
    out = torch.empty((len(heads), len(rows), d), dtype=torch.float64)
    c = 1.0 / np.sqrt(d)
    kv_cache = {}
    for hi, h in enumerate(heads):
        g = h // G
        if g not in kv_cache:
            kv_cache.clear()
            kv_cache[g] = (torch.from_numpy(np.ascontiguousarray(k[g])).double(),
                           torch.from_numpy(np.ascontiguousarray(v[g])).double())
        K, V = kv_cache[g]
        qh = torch.from_numpy(np.ascontiguousarray(q[h]))
        has_bias = bias_offsets is not None and bias_offsets.size and np.any(bias_values[h] != 0)
        for s in range(0, len(rows), chunk):
            r = rows_t[s:s + chunk]
            jmax = int(r.max()) + 1
            j = torch.arange(jmax)
            S = (qh[r].double() @ K[:jmax].T) * c
            if has_bias:
                # logit(i, j) += value where i - j == offset: one entry per row
                for off, val in zip(bias_offsets[h], bias_values[h]):
                    if val != 0 and off >= 0:
                        jj = r - int(off)
                        ok = (jj >= 0) & (jj < jmax)
                        S[torch.nonzero(ok).ravel(), jj[ok]] += float(val)
            mask = _allowed(specs[h], r, j, B, nb)
            S = S.masked_fill(~mask, float("-inf"))
            P = torch.softmax(S, dim=1)
            out[hi, s:s + chunk] = P @ V[:jmax]
    return out.numpy()


def specs_from_index_sets(isets):
    specs = []
    for hd in isets["heads"]:
        if hd["route"]:
            specs.append(dict(kind="vs", vertical=hd["vertical"], slash=hd["slash"]))
        else:
            specs.append(dict(kind="pe", rowptr=hd["rowptr"], cols=hd["cols"]))
    return specs


def attention_row_loop(i, q_row, k, v, bias_off=None, bias_val=None, allowed=None):
    """Loop-based fp64 attention for one row (C); an independent writing used as a pin."""
    lib = _load()
    n, d = k.shape
    allowed = np.ones(n, np.uint8) if allowed is None else _c(allowed, np.uint8)
    out = np.zeros(d, np.float64)
    if bias_off is None or len(bias_off) == 0:
        cnt, bo, bv = 0, None, None
    else:
        bo, bv, cnt = _c(bias_off, np.int32), _c(bias_val, np.float32), len(bias_off)
    lib.oracle_attention_row(int(i), d, _p(_c(q_row, np.float32)), _p(_c(k, np.float32)),
                             _p(_c(v, np.float32)), cnt, _p(bo), _p(bv), _p(allowed), _p(out))
    return out
