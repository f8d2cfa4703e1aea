"""The allocation-free entry point against crisp_sparse_prefill: same bits, on two
calls in a row (the second with a smaller problem), for the matrix engine and the
vector engine."""
import numpy as np
import pytest

import dynamic_sparse_attention_proxy_amd as crisp
import synth
from gpu_harness import DeviceInputs, Timer, log, run_route_select, run_sparse, spec_for

pytestmark = pytest.mark.gpu

# a Llama-shaped 32K layer (matrix engine, about 67 MB of scratch), then smaller ones:
# 5000 tokens on one KV head (matrix engine, ragged), then the tiny fp32 layer (vector
# engine, split partials in the scratch)
SMALL = synth.Workload(name="noalloc_small", hq=4, hkv=1, d=128, n=5000, dtype="bf16", block=128, rope_theta=5e5,
                       seed=47, planted_heads=[0], n_vertical=8)


@pytest.mark.timeout(600)
def test_noalloc_matches_sparse_prefill():
    import torch
    for wl in (synth.WORKLOADS["llama_32k"], SMALL, synth.WORKLOADS["tiny"]):
        log("noalloc case", wl.name, "n", wl.n, wl.dtype)
        with Timer(f"inputs {wl.name}"):
            X = DeviceInputs(synth.make_inputs(wl))
        spec = spec_for(wl)
        bufs = run_route_select(spec, X)
        want = run_sparse(spec, X, bufs)
        o = torch.full_like(X.q, float("nan"))
        crisp.sparse_prefill_noalloc(spec, X.q, X.k, X.v, o, bufs, X.bias_offsets, X.bias_values)
        torch.cuda.synchronize()
        assert torch.equal(o, want), f"{wl.name}: max-abs {float((o.float() - want.float()).abs().max())}"
        # twice in a row on the same problem: the array's leftovers from the last call do not matter
        o.fill_(float("nan"))
        crisp.sparse_prefill_noalloc(spec, X.q, X.k, X.v, o, bufs, X.bias_offsets, X.bias_values)
        torch.cuda.synchronize()
        assert torch.equal(o, want), wl.name
        del X, bufs, want, o
