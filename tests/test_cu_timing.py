"""Timing probes of one compute unit (tests/probes/cu_timing.hip) that the attention
engine's design rests on: a 32x32x16 bf16 matrix instruction every 32 clocks per
SIMD, also as a dependent accumulation chain; how much independent vector work
hides under it with one and two waves per SIMD; LDS read bandwidth per CU.  The
report is printed; the assertions hold the figures the design quotes to loose
bounds."""
import ctypes
import os

import pytest

pytestmark = pytest.mark.gpu

LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "probes", "libcuprobe.so")


@pytest.mark.timeout(300)
def test_cu_timing_probes():
    import torch  # noqa: F401  (the probe binds to the HIP runtime torch brings)
    assert os.path.exists(LIB), "build the probe first: python -c 'import __graft_entry__ as g; g.build()'"
    lib = ctypes.CDLL(LIB)
    lib.crisp_probe_cu_timing.argtypes = [ctypes.c_char_p, ctypes.c_size_t]
    lib.crisp_probe_cu_timing.restype = ctypes.c_int
    buf = ctypes.create_string_buffer(1 << 14)
    assert lib.crisp_probe_cu_timing(buf, len(buf)) == 0
    text = buf.value.decode()
    print(text, flush=True)
    rows = [ln.split() for ln in text.splitlines() if ln.strip()]

    def val(kind, **kw):
        for r in rows:
            if r[0] != kind:
                continue
            d = dict(zip(r[1::2], r[2::2]))
            if all(d.get(k) == str(v) for k, v in kw.items()):
                return float(r[-1])
        raise KeyError((kind, kw))

    assert 28 <= val("issue", waves_per_simd=1, valu_per_mfma=0, mix_exp=0) <= 36
    assert 28 <= val("chain", waves_per_simd=1, chains=1) <= 36  # dependent chains at full rate
    assert val("issue", waves_per_simd=2, valu_per_mfma=4, mix_exp=0) < 40  # 4 FMAs per MFMA mostly hidden
    assert val("lds", waves_per_cu=8) >= 128
