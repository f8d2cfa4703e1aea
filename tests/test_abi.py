"""C-ABI contract on the CPU: the built library exports every call the header
declares, and argument validation returns its error codes without touching a
GPU (no call here reaches a kernel launch)."""
import ctypes
import os
import re

import pytest

import dynamic_sparse_attention_proxy_amd as crisp

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "crisp.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(crisp.LIB_PATH):
        from dynamic_sparse_attention_proxy_amd import build
        build.build()
    return crisp.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(crisp_[a-z_]+)\s*\(", text)))


def test_header_declares_the_four_calls():
    names = declared_functions()
    for n in ("crisp_route", "crisp_select_indices", "crisp_sparse_prefill", "crisp_dense_prefill",
              "crisp_route_jsd"):
        assert n in names
    assert sorted(crisp.EXPORTS) == names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def _spec(**kw):
    base = dict(batch=1, n_q_heads=4, n_kv_heads=2, seq_len=1000, head_dim=128, dtype=crisp.BF16, block=128,
                w_sink=128, w_local=128)
    base.update(kw)
    return crisp.LayerSpec(**base)


def test_sizes(lib):
    s = _spec()
    nb = 8
    assert crisp.index_capacity(s) == nb * (nb + 1) // 2
    ws = crisp.workspace_size(s)
    assert ws >= 4 * nb * 128 * 128 * 4  # proxy tiles of every head
    assert crisp.workspace_size(_spec(head_dim=96)) == 0
    assert crisp.index_capacity(_spec(n_q_heads=3)) == -1
    # largest accepted sizes
    assert crisp.index_capacity(_spec(seq_len=65535 * 128)) == 65535 * 65536 // 2
    assert crisp.workspace_size(_spec(batch=64, n_q_heads=32, n_kv_heads=8, seq_len=8191 * 128)) > 0


@pytest.mark.parametrize("kw,code", [
    (dict(head_dim=96), -2), (dict(n_q_heads=6, n_kv_heads=4), -2), (dict(seq_len=0), -2),
    (dict(seq_len=(1 << 23) + 1), -2), (dict(dtype=7), -3), (dict(block=32), -4), (dict(w_sink=0), -4),
    (dict(tau=(1, 0)), -4), (dict(alpha=(1, 0)), -4), (dict(gamma=(3, 2)), -4), (dict(select_mode=5), -4),
    # N_b above 65535 (int32 CSR offsets), with either block size
    (dict(seq_len=65535 * 128 + 1), -2), (dict(seq_len=65535 * 64 + 1, block=64, w_sink=64, w_local=64), -2),
    # 2^24 (head, query block) items
    (dict(batch=64, n_q_heads=32, n_kv_heads=8, seq_len=8192 * 128), -2),
])
def test_validation_errors(lib, kw, code):
    s = _spec(**kw)
    fake = ctypes.c_void_p(1 << 20)  # aligned, never dereferenced on the host
    idx = crisp.IndexSets(*([1 << 20] * 10), 1 << 20)
    rc = lib.crisp_route(ctypes.byref(s.shape()), ctypes.byref(s.config()), fake, fake, None, fake, 1 << 40,
                         ctypes.byref(idx), None)
    assert rc == code
    rc = lib.crisp_dense_prefill(ctypes.byref(s.shape()), ctypes.byref(s.config()), fake, fake, fake, None, fake,
                                 1 << 40, fake, None)
    assert rc == code


def test_null_alignment_workspace_capacity(lib):
    s = _spec()
    sh, cf = ctypes.byref(s.shape()), ctypes.byref(s.config())
    fake = ctypes.c_void_p(1 << 20)
    cap = crisp.index_capacity(s)
    ws = crisp.workspace_size(s)
    idx = crisp.IndexSets(*([1 << 20] * 10), cap)
    assert lib.crisp_route(None, cf, fake, fake, None, fake, ws, ctypes.byref(idx), None) == -1
    assert lib.crisp_route(sh, cf, None, fake, None, fake, ws, ctypes.byref(idx), None) == -1
    assert lib.crisp_route(sh, cf, ctypes.c_void_p((1 << 20) + 2), fake, None, fake, ws, ctypes.byref(idx),
                           None) == -8
    assert lib.crisp_route(sh, cf, fake, fake, None, fake, ws - 1, ctypes.byref(idx), None) == -5
    nullidx = crisp.IndexSets(*([1 << 20] * 4), None, *([1 << 20] * 5), cap)
    assert lib.crisp_route(sh, cf, fake, fake, None, fake, ws, ctypes.byref(nullidx), None) == -1
    small = crisp.IndexSets(*([1 << 20] * 10), cap - 1)
    assert lib.crisp_select_indices(sh, cf, fake, fake, fake, ws, ctypes.byref(small), None) == -6
    bad_bias = crisp.RelBias(9, 1 << 20, 1 << 20)
    assert lib.crisp_route(sh, cf, fake, fake, ctypes.byref(bad_bias), fake, ws, ctypes.byref(idx), None) == -4
    nb = crisp.RelBias(2, None, 1 << 20)
    assert lib.crisp_sparse_prefill(sh, cf, fake, fake, fake, ctypes.byref(nb), ctypes.byref(idx), fake, ws, fake,
                                    None) == -1
    assert lib.crisp_dense_prefill(sh, cf, fake, fake, fake, None, fake, ws - 1, fake, None) == -5
    assert lib.crisp_dense_prefill(sh, cf, fake, fake, fake, None, None, ws, fake, None) == -1


def test_route_jsd_validation(lib):
    """The divergence router's argument checks (no launch is reached)."""
    s = _spec()
    sh, cf = ctypes.byref(s.shape()), ctypes.byref(s.config())
    fake = ctypes.c_void_p(1 << 20)
    ws = crisp.workspace_size(s)
    idx = crisp.IndexSets(*([1 << 20] * 10), crisp.index_capacity(s))
    f = lib.crisp_route_jsd
    assert f(sh, cf, 1, 0, fake, fake, ctypes.byref(idx), fake, ws, fake, fake, None, None) == -4
    assert f(sh, cf, 1, 100, fake, fake, None, fake, ws, fake, fake, None, None) == -1
    assert f(sh, cf, 1, 100, fake, fake, ctypes.byref(idx), fake, ws, None, fake, None, None) == -1
    assert f(sh, cf, 1, 100, fake, fake, ctypes.byref(idx), fake, ws, fake, None, None, None) == -1
    assert f(sh, cf, 1, 100, fake, fake, ctypes.byref(idx), fake, ws, fake, ctypes.c_void_p((1 << 20) + 4), None,
             None) == -8
    assert f(sh, cf, 1, 100, fake, fake, ctypes.byref(idx), fake, ws - 1, fake, fake, None, None) == -5
    nomass = crisp.IndexSets(*([1 << 20] * 2), None, *([1 << 20] * 7), crisp.index_capacity(s))
    assert f(sh, cf, 1, 100, fake, fake, ctypes.byref(nomass), fake, ws, fake, fake, None, None) == -1
    bad = _spec(head_dim=96)
    assert f(ctypes.byref(bad.shape()), ctypes.byref(bad.config()), 1, 100, fake, fake, ctypes.byref(idx), fake, ws,
             fake, fake, None, None) == -2


def test_select_modes(lib):
    """Noise floor, keep-all and the cumulative comparison mode validate; others do not."""
    for mode in (crisp.SELECT_NOISE_FLOOR, crisp.SELECT_KEEP_ALL, crisp.SELECT_CUMULATIVE):
        assert crisp.workspace_size(_spec(select_mode=mode)) > 0
    assert crisp.workspace_size(_spec(select_mode=3)) == 0


def test_status_strings(lib):
    for code in range(-9, 1):
        assert lib.crisp_status_string(code)
    assert lib.crisp_status_string(-99) == b"unknown status"


def test_product_path_does_not_use_the_oracle():
    pkg = os.path.join(ROOT, "dynamic_sparse_attention_proxy_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in text and "from oracle" not in text and "liboracle" not in text, f


def test_binding_rejects_host_tensors():
    """The binding hands the C-ABI device pointers only: host tensors are refused
    before any call is made."""
    import torch
    with pytest.raises(crisp.CrispError, match="CUDA"):
        crisp._tensor(torch.zeros(4), 4, torch.float32, "q")
    with pytest.raises(crisp.CrispError, match="CUDA"):
        crisp._qkvo(_spec(), q=torch.zeros(4 * 1000 * 128, dtype=torch.bfloat16))


def test_library_loads_after_torch():
    """libcrisp.so must bind to the HIP runtime torch brings: loading it imports torch
    first, even in a process that has not imported torch yet."""
    import subprocess
    import sys
    code = ("import sys; import dynamic_sparse_attention_proxy_amd as c; assert 'torch' not in sys.modules; "
            "c.load_library(); assert 'torch' in sys.modules; print('ok')")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stderr[-2000:]


def test_tile_layout(lib):
    """Where crisp_sparse_prefill keeps its tile lists: pair lists for the matrix engine
    (bf16, d 128, B 128), per-head lists otherwise, inside the workspace."""
    s = _spec(n_q_heads=6, n_kv_heads=2)  # groups of 3: two pairs per KV head, the second with one head
    lay = crisp.tile_layout(s)
    nb = 8
    assert lay["pair_lists"] == 1 and lay["n_lists"] == 2 * 2 and lay["list_stride"] == nb * (nb + 1) // 2
    ws = crisp.workspace_size(s)
    assert 0 <= lay["list_offset"] and lay["list_offset"] + 4 * lay["n_lists"] * lay["list_stride"] <= ws
    assert lay["count_offset"] >= lay["list_offset"] + 4 * lay["n_lists"] * lay["list_stride"]
    assert lay["count_offset"] + 4 * lay["n_lists"] * nb <= ws
    g = crisp.tile_layout(_spec(dtype=crisp.F32, head_dim=64, block=64))
    assert g["pair_lists"] == 0 and g["n_lists"] == 4 and g["list_stride"] == 16 * 17 // 2
    assert lib.crisp_tile_layout_of(ctypes.byref(s.shape()), ctypes.byref(s.config()), None) == -1
    with pytest.raises(crisp.CrispError, match="SHAPE"):
        crisp.tile_layout(_spec(head_dim=96))


def test_noalloc_validation(lib):
    """The allocation-free entry point: the same argument checks as crisp_sparse_prefill, and a
    problem whose attention scratch exceeds its static array is refused (no launch is reached)."""
    f = lib.crisp_sparse_prefill_noalloc
    s = _spec()
    sh, cf = ctypes.byref(s.shape()), ctypes.byref(s.config())
    fake = ctypes.c_void_p(1 << 20)
    idx = crisp.IndexSets(*([1 << 20] * 10), crisp.index_capacity(s))
    assert f(sh, cf, None, fake, fake, None, ctypes.byref(idx), fake, None) == -1
    assert f(sh, cf, fake, fake, fake, None, None, fake, None) == -1
    assert f(sh, cf, fake, fake, fake, None, ctypes.byref(idx), ctypes.c_void_p((1 << 20) + 2), None) == -8
    small = crisp.IndexSets(*([1 << 20] * 10), crisp.index_capacity(s) - 1)
    assert f(sh, cf, fake, fake, fake, None, ctypes.byref(small), fake, None) == -6
    bad = _spec(head_dim=96)
    assert f(ctypes.byref(bad.shape()), ctypes.byref(bad.config()), fake, fake, fake, None, ctypes.byref(idx), fake,
             None) == -2
    # a Llama-shaped 128K layer: V^T of 8 KV heads alone is 256 MiB
    big = _spec(n_q_heads=32, n_kv_heads=8, seq_len=131072)
    bidx = crisp.IndexSets(*([1 << 20] * 10), crisp.index_capacity(big))
    assert f(ctypes.byref(big.shape()), ctypes.byref(big.config()), fake, fake, fake, None, ctypes.byref(bidx), fake,
             None) == -9
    assert b"128 MiB" in lib.crisp_status_string(-9)
