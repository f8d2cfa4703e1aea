"""Seeded synthetic workloads for the CRISP sparse-prefill path.

Inputs only: this module draws Q, K, V and the planted attention structure
(sinks, vertical columns, slash diagonals as a relative-position bias) and
rounds them to the storage precision.  It contains none of the method's
arithmetic; the CPU oracle and the GPU library both consume the bytes it
produces.

The workloads are single attention layers shaped like Llama-3.1-8B and
Qwen2.5-7B (the two model families the CRISP summary page names in its
Overview), with synthetic values standing in for real activations:

* base Q, K, V ~ N(0,1)/sqrt(d), rotary embedding on Q and K (theta per model);
* "VS-planted" heads reproduce the post-softmax mass hierarchy the pages
  describe (sinks holding most of the mass, a few vertical columns and slash
  diagonals, near-uniform background): a per-KV-group direction u is added to
  every query row of the planted query heads (1.5 u) and to the sink rows and
  vertical-column rows of K (gain * u); ||u||^2 = (lambda/1.5) sqrt(d) so that
  gain g adds lambda*g nats to the logit, lambda = 2;
* slash diagonals are a per-head relative-position bias of 6 nats at a few
  offsets;
* "high-entropy" heads are left i.i.d.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libsynth.so")
_lib = None

LAMBDA = 2.0  # logit nats per unit of planted gain
Q_PLANT = 1.5  # query-side multiple of u
SLASH_BIAS = 6.0  # nats added at each planted slash offset

# Method constants fixed for every workload (data, not arithmetic).
TAU = (1, 10)  # routing threshold tau_proxy
ALPHA = (1, 1)  # noise-floor multiplier alpha
GAMMA = (19, 20)  # coverage of the pooled-estimation index (and the cumulative baseline)


def build(force: bool = False) -> str:
    src = os.path.join(_HERE, "synth.c")
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(src):
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", src, "-o", _LIB_PATH, "-lm"])
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        # CRISP_SYNTH_LIB: another build of the same source (the sanitizer test loads one)
        path = os.environ.get("CRISP_SYNTH_LIB") or _LIB_PATH
        if path == _LIB_PATH and not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(path)
        P = ctypes.c_void_p
        lib.synth_fill.argtypes = [P, ctypes.c_int32, ctypes.c_int64, ctypes.c_int64, ctypes.c_int32,
                                   ctypes.c_uint64, ctypes.c_uint32, ctypes.c_double, ctypes.c_double, P, P, P,
                                   ctypes.c_int32]
        lib.synth_fill.restype = None
        lib.synth_to_bf16_bits.argtypes = [P, P, ctypes.c_int64]
        lib.synth_to_bf16_bits.restype = None
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


@dataclass
class Workload:
    name: str
    hq: int
    hkv: int
    d: int
    n: int
    dtype: str  # "f32" or "bf16"
    block: int
    rope_theta: float
    seed: int
    planted_heads: list  # query heads that are VS-planted
    sink_tokens: int = 4
    sink_gain: float = 6.0
    n_vertical: int = 64
    vertical_gain: tuple = (2.0, 4.0)
    n_slash: int = 4
    slash_range: int = 4096
    fixed_slash: tuple = ()  # used instead of random draws when given
    fixed_verticals: tuple = ()  # key positions used instead of random draws when given
    slash_bias: float = SLASH_BIAS  # nats added at each planted slash offset
    batch: int = 1
    qk_scale: float = 1.0  # power of two multiplying Q and K after rounding (0: all-zero Q and K)
    description: str = ""

    @property
    def w_sink(self):
        return self.block

    @property
    def w_local(self):
        return self.block

    def replace(self, **kw) -> "Workload":
        d = dict(self.__dict__)
        d.update(kw)
        return Workload(**d)


WORKLOADS = {
    "tiny": Workload(
        name="tiny", hq=2, hkv=1, d=64, n=4096, dtype="f32", block=64, rope_theta=0.0, seed=1001,
        planted_heads=[0], sink_gain=6.0, n_vertical=8, vertical_gain=(3.0, 3.0), n_slash=3,
        fixed_slash=(0, 1, 64),
        description="tiny fp32 layer: 2 query heads on 1 KV head, d=64, n=4096, block 64"),
    "llama_32k": Workload(
        name="llama_32k", hq=32, hkv=8, d=128, n=32768, dtype="bf16", block=128, rope_theta=5e5,
        seed=1002, planted_heads=list(range(16)),
        description="Llama-3.1-8B-shaped layer: 32 q / 8 kv heads, d=128, n=32768, bf16, causal"),
    "llama_64k": Workload(
        name="llama_64k", hq=32, hkv=8, d=128, n=65536, dtype="bf16", block=128, rope_theta=5e5,
        seed=1006, planted_heads=list(range(16)),
        description="Llama-3.1-8B-shaped layer: 32 q / 8 kv heads, d=128, n=65536, bf16, causal"),
    "llama_128k": Workload(
        name="llama_128k", hq=32, hkv=8, d=128, n=131072, dtype="bf16", block=128, rope_theta=5e5,
        seed=1003, planted_heads=list(range(16)),
        description="Llama-3.1-8B-shaped layer: 32 q / 8 kv heads, d=128, n=131072, bf16, causal"),
    "qwen_128k": Workload(
        name="qwen_128k", hq=28, hkv=4, d=128, n=131072, dtype="bf16", block=128, rope_theta=1e6,
        seed=1004, planted_heads=list(range(14)), sink_gain=8.0,
        description="Qwen2.5-7B-shaped layer: 28 q / 4 kv heads, d=128, n=131072, bf16, causal"),
    "llama_256k": Workload(
        name="llama_256k", hq=32, hkv=8, d=128, n=262144, dtype="bf16", block=128, rope_theta=5e5,
        seed=1007, planted_heads=list(range(16)),
        description="Llama-3.1-8B-shaped layer: 32 q / 8 kv heads, d=128, n=262144, bf16, causal"),
    "llama_512k": Workload(
        name="llama_512k", hq=32, hkv=8, d=128, n=524288, dtype="bf16", block=128, rope_theta=5e5,
        seed=1005, planted_heads=list(range(16)), n_vertical=256, n_slash=8,
        description="Llama-3.1-8B-shaped layer: 32 q / 8 kv heads, d=128, n=524288, bf16, causal"),
    "llama_1m": Workload(
        name="llama_1m", hq=32, hkv=8, d=128, n=1 << 20, dtype="bf16", block=128, rope_theta=5e5,
        seed=1008, planted_heads=list(range(16)), n_vertical=256, n_slash=8,
        description="Llama-3.1-8B-shaped layer: 32 q / 8 kv heads, d=128, n=1048576, bf16, causal"),
}


@dataclass
class Inputs:
    wl: Workload
    q: np.ndarray  # [batch*hq, n, d] float32 (values exactly representable in the storage dtype);
    #               [batch*hq, qrows, d] (last query block only) when drawn with q_last_block_only
    k: np.ndarray  # [batch*hkv, n, d]
    v: np.ndarray  # [batch*hkv, n, d]
    bias_offsets: np.ndarray  # [batch*hq, count] int32 (count may be 0)
    bias_values: np.ndarray  # [batch*hq, count] float32 (0 where a head has no bias)
    verticals: dict = field(default_factory=dict)  # kv head -> sorted column positions
    slashes: dict = field(default_factory=dict)  # q head -> slash offsets
    sinks: int = 0

    @property
    def group(self):
        return self.wl.hq // self.wl.hkv


def plant_metadata(wl: Workload):
    """Planted directions, rows and offsets (small; numpy PCG64 from the seed)."""
    rng = np.random.default_rng([wl.seed, 17])
    d, n, B = wl.d, wl.n, wl.block
    G = wl.hq // wl.hkv
    groups = sorted({h // G for h in wl.planted_heads})
    u = {}
    cols = {}
    gains = {}
    for g in groups:
        w = rng.standard_normal(d)
        u[g] = w / np.linalg.norm(w) * np.sqrt(LAMBDA / Q_PLANT * np.sqrt(d))
        lo, hi = B, n - B
        if wl.fixed_verticals:
            c = np.array(sorted(wl.fixed_verticals), np.int64)
            nv = len(c)
        else:
            nv = min(wl.n_vertical, max(hi - lo, 0))
            c = np.sort(rng.choice(np.arange(lo, hi), size=nv, replace=False)) if nv > 0 else np.zeros(0, np.int64)
        cols[g] = c
        gains[g] = rng.uniform(wl.vertical_gain[0], wl.vertical_gain[1], size=nv)
    slashes = {}
    for h in wl.planted_heads:
        if wl.fixed_slash:
            slashes[h] = np.array(wl.fixed_slash, np.int64)
        else:
            slashes[h] = np.sort(rng.choice(np.arange(0, min(wl.slash_range, n)), size=wl.n_slash, replace=False))
    return u, cols, gains, slashes


def make_inputs(wl: Workload, with_v: bool = True, q_last_block_only: bool = False) -> Inputs:
    """Draw the workload.  q_last_block_only: Q holds only the rows of the last
    query block ([bh, qrows, d]); enough for the proxy map and routing."""
    lib = _load()
    d, n, B = wl.d, wl.n, wl.block
    G = wl.hq // wl.hkv
    bh, bkv = wl.batch * wl.hq, wl.batch * wl.hkv
    u, cols, gains, slashes = plant_metadata(wl)
    scale = 1.0 / np.sqrt(d)
    rb = 1 if wl.dtype == "bf16" else 0

    q_add = np.zeros((bh, d), np.float64)
    for b in range(wl.batch):
        for h in wl.planted_heads:
            q_add[b * wl.hq + h] = Q_PLANT * u[h // G]
    k_gain = np.zeros((bkv, n), np.float64)
    k_dir = np.zeros((bkv, d), np.float64)
    for b in range(wl.batch):
        for g, ug in u.items():
            k_dir[b * wl.hkv + g] = ug
            k_gain[b * wl.hkv + g, : min(wl.sink_tokens, n)] = wl.sink_gain
            k_gain[b * wl.hkv + g, cols[g]] = gains[g]

    q0 = ((n + B - 1) // B - 1) * B if q_last_block_only else 0
    q = np.empty((bh, n - q0, d), np.float32)
    k = np.empty((bkv, n, d), np.float32)
    lib.synth_fill(_ptr(q), bh, n, q0, d, wl.seed, 1, scale, wl.rope_theta, _ptr(q_add), None, None, rb)
    lib.synth_fill(_ptr(k), bkv, n, 0, d, wl.seed, 2, scale, wl.rope_theta, None, _ptr(k_gain), _ptr(k_dir), rb)
    if wl.qk_scale == 0.0:
        q[...] = 0.0
        k[...] = 0.0
    elif wl.qk_scale != 1.0:
        m, _ = np.frexp(wl.qk_scale)
        assert m == 0.5, "qk_scale must be a power of two (exact in both storage types)"
        q *= np.float32(wl.qk_scale)
        k *= np.float32(wl.qk_scale)
    if with_v:
        v = np.empty((bkv, n, d), np.float32)
        lib.synth_fill(_ptr(v), bkv, n, 0, d, wl.seed, 3, scale, 0.0, None, None, None, rb)
    else:
        v = None

    count = max([len(s) for s in slashes.values()], default=0)
    offs = np.zeros((bh, count), np.int32)
    vals = np.zeros((bh, count), np.float32)
    for b in range(wl.batch):
        for h, s in slashes.items():
            offs[b * wl.hq + h, : len(s)] = s
            vals[b * wl.hq + h, : len(s)] = wl.slash_bias
    # heads without a planted slash get offsets that never occur (value 0 anyway)
    for r in range(bh):
        if count and not vals[r].any():
            offs[r, :] = -1
    return Inputs(wl=wl, q=q, k=k, v=v, bias_offsets=offs, bias_values=vals,
                  verticals={g: c for g, c in cols.items()},
                  slashes={h: s for h, s in slashes.items()}, sinks=wl.sink_tokens)


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Bit patterns (uint16) of the bf16 values nearest to float32 array a."""
    lib = _load()
    a = np.ascontiguousarray(a, np.float32)
    out = np.empty(a.shape, np.uint16)
    lib.synth_to_bf16_bits(_ptr(a), _ptr(out), a.size)
    return out


def sample_rows(wl: Workload, count: int = 256) -> np.ndarray:
    """Seeded rows checked at long lengths: 0, n-1, 32 rows of the last query block, the rest uniform."""
    n, B = wl.n, wl.block
    rng = np.random.default_rng(wl.seed + 7919)
    q0 = ((n + B - 1) // B - 1) * B
    last = np.arange(q0, n)
    pick_last = rng.choice(last, size=min(32, len(last)), replace=False)
    rest = rng.choice(np.arange(1, n - 1), size=max(count - 2 - len(pick_last), 0), replace=False)
    rows = np.unique(np.concatenate([[0, n - 1], pick_last, rest]).astype(np.int64))
    return rows
