"""Helpers for the GPU parity tests: upload seeded inputs, run the C-ABI path,
download its outputs in the oracle's formats.  Only argument marshalling here."""
from __future__ import annotations

import sys
import time

import numpy as np

import dynamic_sparse_attention_proxy_amd as crisp
import synth


def log(*a):
    print("[gpu]", *a, flush=True)
    sys.stdout.flush()


def spec_for(wl: synth.Workload, select_mode=crisp.SELECT_NOISE_FLOOR, block=None) -> crisp.LayerSpec:
    B = block or wl.block
    return crisp.LayerSpec(batch=wl.batch, n_q_heads=wl.hq, n_kv_heads=wl.hkv, seq_len=wl.n, head_dim=wl.d,
                           dtype=crisp.BF16 if wl.dtype == "bf16" else crisp.F32, block=B, w_sink=B, w_local=B,
                           tau=synth.TAU, alpha=synth.ALPHA, gamma=synth.GAMMA, select_mode=select_mode)


class DeviceInputs:
    def __init__(self, I: synth.Inputs, device="cuda"):
        import torch
        dt = torch.bfloat16 if I.wl.dtype == "bf16" else torch.float32

        def up(a):
            if a is None:
                return None
            t = torch.from_numpy(a).to(device)
            return t.to(dt).contiguous() if dt != torch.float32 else t.contiguous()

        self.q = up(I.q)
        self.k = up(I.k)
        self.v = up(I.v)
        if I.bias_offsets.size:
            self.bias_offsets = torch.from_numpy(I.bias_offsets).to(device).contiguous()
            self.bias_values = torch.from_numpy(I.bias_values).to(device).contiguous()
        else:
            self.bias_offsets = self.bias_values = None
        torch.cuda.synchronize()


def run_route_select(spec, X: DeviceInputs, bufs: crisp.Buffers = None):
    import torch
    bufs = bufs or crisp.Buffers(spec)
    crisp.route(spec, X.q, X.k, bufs, X.bias_offsets, X.bias_values)
    crisp.select_indices(spec, X.q, X.k, bufs)
    torch.cuda.synchronize()
    return bufs


def download_index_sets(bufs: crisp.Buffers):
    """GPU routing outputs and index sets in the oracle's formats."""
    route = bufs.route.cpu().numpy()
    out = dict(route=route, cnum=bufs.cstruct_num.cpu().numpy(), mass_v=bufs.mass_v.cpu().numpy(),
               mass_s=bufs.mass_s.cpu().numpy(), total=bufs.mass_total.cpu().numpy())
    cnt = bufs.vs_count.cpu().numpy()
    vv = bufs.vs_vertical.cpu().numpy()
    ss = bufs.vs_slash.cpu().numpy()
    rp = bufs.pe_rowptr.cpu().numpy()
    heads = []
    nnz = rp[:, -1]
    cols_all = bufs.pe_col[:, : int(nnz.max()) if nnz.size else 0].cpu().numpy()
    for h in range(len(route)):
        if route[h]:
            heads.append(dict(route=1, vertical=vv[h, : cnt[h, 0]], slash=ss[h, : cnt[h, 1]], count=cnt[h]))
        else:
            heads.append(dict(route=0, rowptr=rp[h], cols=cols_all[h, : rp[h, -1]], count=cnt[h]))
    out["heads"] = heads
    return out


def compare_index_sets(gpu, ref):
    """Bit-exact comparison of routing outputs and index sets; returns a list of mismatch strings."""
    bad = []
    pr = ref["proxy"]
    for key, rk in (("route", "route"), ("cnum", "cnum"), ("mass_v", "mass_v"), ("mass_s", "mass_s"),
                    ("total", "total")):
        if not np.array_equal(gpu[key], pr[rk]):
            diff = np.argwhere(np.asarray(gpu[key] != pr[rk]))
            bad.append(f"{key}: {len(diff)} differences, first at {diff[:3].tolist()}")
    for h, (g, r) in enumerate(zip(gpu["heads"], ref["heads"])):
        if g["route"] != r["route"]:
            continue
        if r["route"]:
            if not np.array_equal(g["vertical"], r["vertical"]):
                bad.append(f"head {h} vertical: gpu {g['vertical'][:10]}.. ({len(g['vertical'])}) "
                           f"oracle {r['vertical'][:10]}.. ({len(r['vertical'])})")
            if not np.array_equal(g["slash"], r["slash"]):
                bad.append(f"head {h} slash: gpu {g['slash'][:10]} oracle {r['slash'][:10]}")
        else:
            if not np.array_equal(g["rowptr"], r["rowptr"]):
                d = np.argwhere(g["rowptr"] != r["rowptr"])
                bad.append(f"head {h} rowptr differs at {d[:3].ravel().tolist()} "
                           f"(nnz gpu {g['rowptr'][-1]} oracle {r['rowptr'][-1]})")
            elif not np.array_equal(g["cols"], r["cols"]):
                bad.append(f"head {h} cols differ")
    return bad


def run_sparse(spec, X: DeviceInputs, bufs: crisp.Buffers):
    import torch
    o = torch.empty_like(X.q)
    crisp.sparse_prefill(spec, X.q, X.k, X.v, o, bufs, X.bias_offsets, X.bias_values)
    torch.cuda.synchronize()
    return o


def run_dense(spec, X: DeviceInputs, bufs: crisp.Buffers = None):
    import torch
    o = torch.empty_like(X.q)
    crisp.dense_prefill(spec, X.q, X.k, X.v, o, bufs if bufs is not None else crisp.Buffers(spec), X.bias_offsets,
                        X.bias_values)
    torch.cuda.synchronize()
    return o


def rows_of(o, rows=None):
    import torch
    if rows is None:
        return o.float().cpu().numpy()
    return o[:, torch.as_tensor(rows, device=o.device)].float().cpu().numpy()


class Timer:
    def __init__(self, what):
        self.what = what

    def __enter__(self):
        self.t = time.time()
        log("start", self.what)
        return self

    def __exit__(self, *a):
        log("done", self.what, f"{time.time() - self.t:.1f}s")


def expected_tile_modes(head, nb):
    """Mask mode of every causal key tile (qb, kb) of one head, from its index set:
    3 for a selected vertical block or a PE block, 1 for the lower triangle of tile
    qb - s and 2 for the upper triangle of tile qb - s - 1 of a selected slash block s,
    the diagonal tile cut to its causal (lower) part; 0 where the head does not look."""
    qb = np.arange(nb, dtype=np.int32)[:, None]
    kb = np.arange(nb, dtype=np.int32)[None, :]
    delta = qb - kb
    M = np.zeros((nb, nb), np.uint8)
    if head["route"]:
        col = np.zeros(nb, bool)
        col[np.asarray(head["vertical"], np.int64)] = True
        sl = np.zeros(nb + 1, bool)
        sl[np.asarray(head["slash"], np.int64)] = True
        causal = delta >= 0
        M[causal & col[None, :]] |= 3
        M[causal & sl[np.clip(delta, 0, nb)]] |= 1
        M[(delta >= 1) & sl[np.clip(delta - 1, 0, nb)]] |= 2
    else:
        rp = np.asarray(head["rowptr"], np.int64)
        rows = np.repeat(np.arange(nb), np.diff(rp))
        M[rows, np.asarray(head["cols"], np.int64)] = 3
    d = np.arange(nb)
    M[d, d] &= 1
    return M


def compare_tile_lists(spec, bufs, ref):
    """The key-tile lists crisp_sparse_prefill left in the workspace against lists built
    here from the oracle's index sets (ascending key blocks per query block, mask modes
    per head).  Bit-exact; returns a list of mismatch strings."""
    lay, lists, counts = crisp.tile_lists(spec, bufs)
    nb = spec.num_blocks
    G = spec.n_q_heads // spec.n_kv_heads
    tri_r, tri_c = np.tril_indices(nb)
    bad = []
    if lay["pair_lists"]:
        pairs = (G + 1) // 2
        owners = []
        for kv in range(spec.batch * spec.n_kv_heads):
            b, g = divmod(kv, spec.n_kv_heads)
            for w in range(pairs):
                h0 = b * spec.n_q_heads + g * G + 2 * w
                owners.append((h0, h0 + 1 if 2 * w + 1 < G else None))
    else:
        owners = [(h, None) for h in range(spec.heads)]
    assert len(owners) == lay["n_lists"]
    for li, (h0, h1) in enumerate(owners):
        m0 = expected_tile_modes(ref["heads"][h0], nb)[tri_r, tri_c].astype(np.int32)
        m1 = (expected_tile_modes(ref["heads"][h1], nb)[tri_r, tri_c].astype(np.int32) if h1 is not None
              else np.zeros_like(m0))
        keep = (m0 | m1) != 0
        if lay["pair_lists"]:
            want = (tri_c.astype(np.int32) | (m0 << 24) | (m1 << 26))[keep]
        else:
            want = (tri_c.astype(np.int32) | (m0 << 28))[keep]
        want_cnt = np.bincount(tri_r[keep], minlength=nb)
        got_cnt = counts[li].cpu().numpy()
        if not np.array_equal(got_cnt, want_cnt):
            d = np.argwhere(got_cnt != want_cnt).ravel()
            bad.append(f"list {li} (heads {h0}, {h1}): counts differ at qb {d[:5].tolist()} "
                       f"(gpu {got_cnt[d[:5]].tolist()} expected {want_cnt[d[:5]].tolist()})")
            continue
        got = lists[li].cpu().numpy()[tri_c < got_cnt[tri_r]]
        if not np.array_equal(got, want):
            d = np.argwhere(got != want).ravel()
            bad.append(f"list {li} (heads {h0}, {h1}): {len(d)} entries differ, first {d[:3].tolist()}")
    return bad


def block_indicator_v(wl):
    """Values that mark each key: the first d/2 columns one-hot on the key's block
    (block index mod d/2), the last d/2 one-hot on its column (index mod d/2).  Exact in
    bf16 and fp32."""
    n, d, B = wl.n, wl.d, wl.block
    half = d // 2
    j = np.arange(n)
    v = np.zeros((wl.batch * wl.hkv, n, d), np.float32)
    v[:, j, (j // B) % half] = 1.0
    v[:, j, half + j % half] = 1.0
    return v
