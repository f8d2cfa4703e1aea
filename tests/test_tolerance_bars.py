"""The per-element bars of the GPU parity tests, checked on the CPU.

The bf16 bar (_bf16_tolerance) against a float32 / bfloat16 emulation of the rounding
steps it bounds: scores in fp32, probabilities exp2(s c log2e - m) in fp32 rounded to
bf16, their sum and the P V product accumulated in fp32, the normalised output rounded
to bf16.  The emulation must stay within the bar everywhere, and the bar must not be
loose by orders of magnitude.  The fp32 bar of the x 16 inputs (_peaked_f32_tolerance)
against a plain fp32 attention of the same inputs."""
import numpy as np
import pytest

import oracle
import synth


@pytest.mark.parametrize("seed, planted", [(11, [0, 1]), (12, [])])
def test_bf16_bar_covers_the_rounding_steps(seed, planted):
    import torch
    from test_gpu_parity import _bf16_tolerance
    wl = synth.Workload(name="bar", hq=4, hkv=2, d=128, n=1500, dtype="bf16", block=128, rope_theta=5e5,
                        seed=seed, planted_heads=planted, n_vertical=4)
    I = synth.make_inputs(wl)
    ref = oracle.index_sets(I.q, I.k, wl.block, wl.w_sink, wl.w_local, synth.TAU, synth.ALPHA, synth.GAMMA,
                            I.bias_offsets, I.bias_values)
    specs = oracle.specs_from_index_sets(ref)
    heads = list(range(wl.hq))
    want = oracle.attention(I.q, I.k, I.v, wl.block, specs, bias_offsets=I.bias_offsets,
                            bias_values=I.bias_values)
    bar = _bf16_tolerance(wl, I, None, heads, specs)
    n, d = wl.n, wl.d
    nb = oracle.num_blocks(n, wl.block)
    c = np.float32(1.0 / np.sqrt(d))
    ksc = np.float32(c * np.float32(1.4426950408889634))
    rows = torch.arange(n)
    worst = 0.0
    for h in heads:
        g = h // (wl.hq // wl.hkv)
        Q = torch.from_numpy(I.q[h]); K = torch.from_numpy(I.k[g]); V = torch.from_numpy(I.v[g])
        S = (Q @ K.T)  # fp32
        x = S * ksc
        for off, val in zip(I.bias_offsets[h], I.bias_values[h]):
            if val != 0 and off >= 0:
                jj = rows - int(off); ok = jj >= 0
                x[torch.nonzero(ok).ravel(), jj[ok]] += np.float32(val * 1.4426950408889634)
        mask = oracle._allowed(specs[h], rows, rows, wl.block, nb)
        x = x.masked_fill(~mask, float("-inf"))
        m = x.max(dim=1, keepdim=True).values
        P = torch.exp2(x - m).to(torch.bfloat16).float()
        l = P.sum(dim=1, keepdim=True)
        o = (P @ V / l).to(torch.bfloat16).double().numpy()
        err = np.abs(o - want[h])
        assert np.all(err <= bar[h]), (h, float((err / bar[h]).max()))
        worst = max(worst, float((err / bar[h]).max()))
    print(f"emulated rounding: largest error / bar {worst:.3f}")
    assert worst > 0.05  # the bar is of the size of the errors it bounds


def test_peaked_f32_bar_covers_plain_fp32_attention():
    """The per-element bar of the x 16 fp32 inputs (_peaked_f32_tolerance: logits of
    thousands of nats) against a plain fp32 attention of the same inputs, index sets and
    bias: within the bar everywhere."""
    import torch
    from test_gpu_parity import EDGE, _peaked_f32_tolerance
    wl = EDGE["peaked_f32"]
    I = synth.make_inputs(wl)
    ref = oracle.index_sets(I.q, I.k, wl.block, wl.w_sink, wl.w_local, synth.TAU, synth.ALPHA, synth.GAMMA,
                            I.bias_offsets, I.bias_values)
    specs = oracle.specs_from_index_sets(ref)
    heads = list(range(wl.hq))
    n = wl.n
    nb = oracle.num_blocks(n, wl.block)
    want = oracle.attention(I.q, I.k, I.v, wl.block, specs, bias_offsets=I.bias_offsets,
                            bias_values=I.bias_values)
    tol = _peaked_f32_tolerance(wl, I, None, heads, specs)
    rows = torch.arange(n)
    worst = 0.0
    for h in heads:
        g = h // (wl.hq // wl.hkv)
        Q = torch.from_numpy(I.q[h]); K = torch.from_numpy(I.k[g]); V = torch.from_numpy(I.v[g])
        S = (Q @ K.T) * np.float32(1.0 / np.sqrt(wl.d))
        for off, val in zip(I.bias_offsets[h], I.bias_values[h]):
            if val != 0 and off >= 0:
                jj = rows - int(off); ok = jj >= 0
                S[torch.nonzero(ok).ravel(), jj[ok]] += float(val)
        mask = oracle._allowed(specs[h], rows, rows, wl.block, nb)
        got = (torch.softmax(S.masked_fill(~mask, float("-inf")), dim=1) @ V).double().numpy()
        err = np.abs(got - want[h])
        assert np.all(err <= tol[h]), (h, float((err / tol[h]).max()))
        worst = max(worst, float((err / tol[h]).max()))
    print(f"plain fp32 attention: largest error / bar {worst:.3f}")
