"""The CPU oracle and the input generator under AddressSanitizer and
UndefinedBehaviorSanitizer: both C libraries are rebuilt with
-fsanitize=address,undefined and the oracle's pins are run against those
builds in a child process (CPU only; the HIP library is not involved)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# the pins that drive the C code: scores, fixed-point softmax, block masses,
# routing, both selection rules, the PE index, the logarithm and divergence,
# the pooled row, the loop attention writing, and the generator
PINS = ("exp_crisp or closed_form or fp64_softmax or pooling_recount or golden or exact_threshold or "
        "bruteforce or uniform_closed_form or pe_index_matches or loop_writing or log_crisp or jsd or pooled_row "
        "or generator or sink_only")


def _gcc(src, out):
    cmd = ["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=undefined", "-ffp-contract=off", "-mfma", "-fopenmp", "-fPIC", "-shared", src,
           "-o", out, "-lm"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)


def _runtime(name):
    p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


@pytest.mark.timeout(900)
def test_oracle_and_generator_under_asan_ubsan(tmp_path):
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("gcc sanitizer runtimes not installed")
    ora = str(tmp_path / "liboracle_asan.so")
    syn = str(tmp_path / "libsynth_asan.so")
    _gcc(os.path.join(ROOT, "oracle", "crisp_oracle.c"), ora)
    _gcc(os.path.join(ROOT, "synth", "synth.c"), syn)
    env = dict(os.environ)
    # the sanitizer runtimes first; anything the environment already preloads stays
    env["LD_PRELOAD"] = " ".join(x for x in (asan, ubsan, os.environ.get("LD_PRELOAD", "")) if x)
    env["ASAN_OPTIONS"] = "detect_leaks=0:verify_asan_link_order=0:halt_on_error=1:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["CRISP_ORACLE_LIB"] = ora
    env["CRISP_SYNTH_LIB"] = syn
    env["OMP_NUM_THREADS"] = "4"
    code = ("import sys, oracle, synth; "
            "oracle._load(); synth._load(); "
            "import ctypes; "
            "assert oracle._lib._name == sys.argv[1] and synth._lib._name == sys.argv[2]; "
            "import pytest; sys.exit(pytest.main(['-q', '-x', '-p', 'no:cacheprovider', '-k', sys.argv[3], "
            "'tests/test_oracle_pins.py']))")
    r = subprocess.run([sys.executable, "-c", code, ora, syn, PINS], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=880)
    tail = (r.stdout[-3000:] + "\n" + r.stderr[-3000:])
    assert r.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error:" not in r.stderr, tail
    assert " passed" in r.stdout, tail
