"""Layer-sequential quantization of the MLP of one decoder layer (page "大模型常见的量化方式",
section on the layers of a large model; page "量化", section GPTQ, layer by layer): gate_proj
and up_proj are quantized on the block input X with one shared Hessian, then down_proj is
calibrated on silu(X G^T) * (X U^T) computed from the *quantized* gate_proj and up_proj, so
each quantized sub-layer produces the next one's calibration input.

Every step is a call of the C ABI (gptq.py marshals the arguments); torch only holds device
memory.
"""

from __future__ import annotations

from typing import Dict, Optional

from . import gptq as G


def quantize_mlp_block(W_gate, W_up, W_down, X, spec: "G.Spec", stream=None) -> Dict[str, object]:
    """W_gate, W_up [d_ff x d] and W_down [d x d_ff] (fp16 or fp32, device), X [n_tok x d]
    fp16 (device).  Returns the packed outputs of the three layers (qweight, scales, zeros,
    err_sq_rows as quantize_layer returns them), down_proj's calibration input Y, the two
    Hessians and each layer's loss ||W X - W^ X||^2 on its own input (float64 scalars)."""
    torch = G._torch()
    d_ff, d = W_gate.shape
    assert W_up.shape == (d_ff, d) and W_down.shape == (d, d_ff) and X.shape[1] == d
    dev = X.device
    H_x = torch.zeros((d, d), dtype=torch.float32, device=dev)
    G.hessian_accumulate(H_x, X, stream=stream)
    G_x = G.prepare_hinv(H_x, damp_frac=spec.damp_frac, stream=stream)
    gate = G.quantize_layer(W_gate, G_x, spec, stream=stream)
    up = G.quantize_layer(W_up, G_x, spec, stream=stream)
    del G_x
    Y = G.mlp_forward(X, gate[:3], up[:3], spec.bits, spec.group, stream=stream)
    H_y = torch.zeros((d_ff, d_ff), dtype=torch.float32, device=dev)
    G.hessian_accumulate(H_y, Y, stream=stream)
    G_y = G.prepare_hinv(H_y, damp_frac=spec.damp_frac, stream=stream)
    down = G.quantize_layer(W_down, G_y, spec, stream=stream)
    del G_y
    losses = {}
    for name, W, q, H in (("gate", W_gate, gate, H_x), ("up", W_up, up, H_x),
                          ("down", W_down, down, H_y)):
        losses[name] = G.dequant_check(q[0], q[1], q[2], W, H, spec, stream=stream)[0]
    torch.cuda.synchronize()
    return {"gate": gate, "up": up, "down": down, "Y": Y, "H_x": H_x, "H_y": H_y,
            "loss_gate": losses["gate"].item(), "loss_up": losses["up"].item(),
            "loss_down": losses["down"].item()}
