"""The allocation-free entry point gptq_act_absmean_noalloc against gptq_act_absmean (the same
kernels with a caller-owned workspace), through the C ABI: two calls in a row, the second on
a smaller input, each checked bit for bit against the workspace call on the same input; the
second call also shows that the scratch keeps nothing of the first that matters.  Nothing is
allocated by the call (torch's allocator is unchanged across it)."""

import ctypes

import numpy as np
import pytest

from post_weight_quantization_24_amd import gptq as G
from post_weight_quantization_24_amd import synth

pytestmark = pytest.mark.gpu


def _torch():
    import torch
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    return torch


def say(*a):
    print("[gpu-case]", *a, flush=True)


def _with_workspace(torch, X, d):
    out = torch.zeros(d, dtype=torch.float64, device=X.device)
    G.act_absmean(out, X)
    return out


def _noalloc(torch, X, d):
    out = torch.zeros(d, dtype=torch.float64, device=X.device)
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    rc = G.lib().gptq_act_absmean_noalloc(
        ctypes.c_void_p(out.data_ptr()), d, ctypes.c_void_p(X.data_ptr()), G._dtype_code(X),
        X.shape[0], X.stride(0), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == G.OK, G.lib().gptq_last_error()
    assert torch.cuda.memory_allocated() == before
    return out


@pytest.mark.parametrize("first,second", [((4096, 65536, "f16"), (1000, 3000, "f32")),
                                          ((11008, 20000, "f16"), (96, 300, "f16"))])
def test_noalloc_equals_workspace_call(first, second):
    torch = _torch()
    for d, n_tok, dtype in (first, second):
        say("act_absmean_noalloc", d, n_tok, dtype)
        X = torch.from_numpy(synth.gen_acts(990, "noalloc%d" % d, n_tok, d, dtype)).to("cuda:0")
        a = _noalloc(torch, X, d)
        b = _with_workspace(torch, X, d)
        torch.cuda.synchronize()
        assert torch.equal(a, b), float((a - b).abs().max())
        # sums of |x| over the tokens in float64 within rounding of the exact sums
        ref = np.abs(X.cpu().numpy().astype(np.float64)).sum(axis=0)
        np.testing.assert_allclose(a.cpu().numpy(), ref, rtol=1e-12)


def test_noalloc_accumulates_across_calls():
    """sx_sum += over two chunks equals one call over both (chunked calibration)."""
    torch = _torch()
    d, n_tok = 2048, 12288
    say("act_absmean_noalloc chunks", d, n_tok)
    X = torch.from_numpy(synth.gen_acts(991, "noalloc_chunks", n_tok, d, "f16")).to("cuda:0")
    acc = torch.zeros(d, dtype=torch.float64, device="cuda:0")
    G.act_absmean_noalloc(acc, X[:8192])
    G.act_absmean_noalloc(acc, X[8192:])
    ref = torch.zeros(d, dtype=torch.float64, device="cuda:0")
    G.act_absmean(ref, X[:8192])
    G.act_absmean(ref, X[8192:])
    torch.cuda.synchronize()
    assert torch.equal(acc, ref)
