"""Host-side helpers of bench.py: the density figures it reports, against brute force."""
import os
import sys
import types

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


class _T:
    def __init__(self, a):
        self.a = np.asarray(a)

    def cpu(self):
        return self

    def numpy(self):
        return self.a


def _random_sets(seed, B, n, route):
    rng = np.random.default_rng(seed)
    nb, H = n // B, len(route)
    cnt = np.zeros((H, 2), np.int32)
    vv = np.zeros((H, nb), np.int32)
    ss = np.zeros((H, nb), np.int32)
    rp = np.zeros((H, nb + 1), np.int32)
    allowed = []
    for h in range(H):
        if route[h]:
            V = np.sort(rng.choice(nb, 3, replace=False))
            S = np.sort(rng.choice(nb, 3, replace=False))
            cnt[h] = (len(V), len(S))
            vv[h, :len(V)] = V
            ss[h, :len(S)] = S
            allowed.append(lambda i, j, V=set(V.tolist()), S=set(S.tolist()): j // B in V or (i - j) // B in S)
        else:
            rows, ptr = [], [0]
            for qb in range(nb):
                ks = set(rng.choice(qb + 1, min(qb + 1, 2), replace=False).tolist()) | {qb}
                rows.append(ks)
                ptr.append(ptr[-1] + len(ks))
            rp[h] = ptr
            allowed.append(lambda i, j, rows=rows: j // B in rows[i // B])
    bufs = types.SimpleNamespace(route=_T(route), vs_count=_T(cnt), vs_vertical=_T(vv), vs_slash=_T(ss),
                                 pe_rowptr=_T(rp))
    return bufs, allowed


def test_useful_pair_density_bruteforce():
    B, n = 4, 32
    route = np.array([1, 0, 1, 0])
    bufs, allowed = _random_sets(7, B, n, route)
    spec = types.SimpleNamespace(block=B, seq_len=n, num_blocks=n // B)
    truth = sum(allowed[h](i, j) for h in range(len(route)) for i in range(n) for j in range(i + 1))
    got = bench.useful_pair_density(bufs, spec) * len(route) * n * (n + 1) / 2
    assert abs(got - truth) < 1e-6


def test_tile_counts_bruteforce():
    B, n = 4, 32
    nb = n // B
    route = np.array([1, 0, 1])
    bufs, allowed = _random_sets(8, B, n, route)
    spec = types.SimpleNamespace(block=B, seq_len=n, num_blocks=nb)
    got = bench.tile_counts(bufs, spec)
    for h in range(len(route)):
        tiles = sum(any(allowed[h](qb * B + r, kb * B + c) for r in range(B) for c in range(B)
                        if qb * B + r >= kb * B + c)
                    for qb in range(nb) for kb in range(qb + 1))
        assert got[h] == tiles, (h, got[h], tiles)


def test_bench_refuses_more_than_one_gpu():
    """The path runs on one GPU; asking for more exits with a message, before any GPU work."""
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode != 0
    assert "--gpus 1" in r.stderr
    assert not r.stdout.strip()


def test_amd_smi_parse():
    """The clock / power sampler reads amd-smi's text output (format as printed by
    `amd-smi metric --power --clock` on an MI355X machine, trimmed)."""
    import bench
    text = """GPU: 0
    POWER:
        SOCKET_POWER: 1383 W
        GFX_VOLTAGE: N/A
    CLOCK:
        GFX_0:
            CLK: 2047 MHz
            MIN_CLK: 157 MHz
            MAX_CLK: 2400 MHz
        GFX_1:
            CLK: 2101 MHz
            MIN_CLK: 157 MHz
            MAX_CLK: 2400 MHz
        MEM_0:
            CLK: 2000 MHz
"""
    r = bench.parse_amd_smi([text, text.replace("1383", "1371")])
    assert r["gfx_mhz_min"] == 2047 and r["gfx_mhz_max"] == 2101 and r["gfx_mhz_mean"] == 2074.0
    assert r["socket_power_w_median"] == 1377.0 and r["samples"] == 2
    assert bench.parse_amd_smi(["AMDSMI Tool: no GPU"]) is None
