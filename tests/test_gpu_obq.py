"""The fixed-order claim on the GPU path: the layer loss of the GPU column solve against the
oracle's greedy-order (OBQ) loss on the same small layers (page "量化", section GPTQ, first
improvement).  The GPU loss must also stay within the 0.5 % parity bar of the oracle's own
fixed-order loss.
"""

import numpy as np
import pytest

import oracle as O
from post_weight_quantization_24_amd import gptq as G
from tests.test_oracle_obq import comparison_layers

pytestmark = pytest.mark.gpu


def test_gpu_fixed_order_against_greedy():
    import torch
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    dev = "cuda:0"
    for label, W, X, bits, sym in comparison_layers():
        print("[gpu-case] fixed order vs greedy", label, flush=True)
        d_row, d_col = W.shape
        W32, X32 = W.astype(np.float32), X.astype(np.float32)
        Wd, Xd = torch.from_numpy(W32).to(dev), torch.from_numpy(X32).to(dev)
        Hd = torch.zeros((d_col, d_col), dtype=torch.float32, device=dev)
        G.hessian_accumulate(Hd, Xd)
        Gd = G.prepare_hinv(Hd, damp_frac=0.01)
        spec = G.Spec.make(bits, 0, sym, min(128, d_col), 0.01)
        qw, sc, ze, _ = G.quantize_layer(Wd, Gd, spec)
        loss, _, _, off = G.dequant_check(qw, sc, ze, Wd, Hd, spec)
        torch.cuda.synchronize()
        assert off.item() == 0
        H = O.hessian(X32)
        Hdmp, _ = O.damp(H, 0.01)
        greedy = O.obq_greedy_quantize(W32, Hdmp, bits, sym)
        fixed = O.gptq_quantize(W32, O.inv_chol_upper(Hdmp), bits, 0, sym)
        lg = O.layer_loss(W32, greedy["w_hat"], H)
        lf = O.layer_loss(W32, fixed["w_hat"], H)
        print("[gpu-case]   gpu %.6g oracle fixed %.6g greedy %.6g  gpu/greedy %.3f"
              % (loss.item(), lf, lg, loss.item() / lg), flush=True)
        assert abs(loss.item() - lf) <= 5e-3 * lf
        assert loss.item() <= 1.05 * lg
