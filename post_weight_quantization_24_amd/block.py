"""Layer-sequential quantization of one decoder layer (page "大模型常见的量化方式", section on
the layers of a large model: the LLaMA layer, its attention q/k/v/o_proj and MLP
gate/up/down_proj quantized, its two RMSNorms kept in float16; page "量化", section GPTQ, layer
by layer).  Each quantized sub-layer produces the next one's calibration input:
  q/k/v_proj   on n1 = rmsnorm(x) gamma1 (one shared Hessian),
  o_proj       on O  = attention of the quantized q/k/v,
  gate/up_proj on n2 = rmsnorm(h) gamma2, h = x + O W_o^T with the quantized o_proj,
  down_proj    on Y  = silu(n2 G^T) * (n2 U^T) with the quantized gate/up_proj.
quantize_mlp_block runs the MLP half alone on a given input.

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


SUBLAYERS = ("q_proj", "k_proj", "v_proj", "o_proj", "gate_proj", "up_proj", "down_proj")


def quantize_decoder_block(W: Dict[str, object], x, gamma1, gamma2, spec: "G.Spec", seq_len: int,
                           eps: float = 1e-6, stream=None) -> Dict[str, object]:
    """W maps the seven sub-layer names to device weights (q/k/v/o [d x d], gate/up
    [d_ff x d], down [d x d_ff], fp16 or fp32); x [n_tok x d] fp16 is the block input, cut
    into sequences of seq_len tokens; gamma1, gamma2 [d] fp16.  Returns each sub-layer's
    packed output (as quantize_layer returns it), the calibration inputs n1, O, h, n2, Y,
    the four Hessians and each layer's loss on its own input (float64 scalars)."""
    torch = G._torch()
    n_tok, d = x.shape
    r: Dict[str, object] = {}

    def run(names, X):
        H = torch.zeros((X.shape[1], X.shape[1]), dtype=torch.float32, device=X.device)
        G.hessian_accumulate(H, X, stream=stream)
        Gm = G.prepare_hinv(H, damp_frac=spec.damp_frac, stream=stream)
        for nm in names:
            q = G.quantize_layer(W[nm], Gm, spec, stream=stream)
            r[nm] = q
            r["loss_" + nm] = G.dequant_check(q[0], q[1], q[2], W[nm], H, spec, stream=stream)[0]
        del Gm
        return H

    n1 = G.rmsnorm(x, gamma1, eps, stream=stream)
    r["H_n1"] = run(("q_proj", "k_proj", "v_proj"), n1)
    O = G.attention_forward(n1, r["q_proj"][:3], r["k_proj"][:3], r["v_proj"][:3], spec.bits,
                            spec.group, seq_len, stream=stream)
    r["H_o"] = run(("o_proj",), O)
    h = G.residual_linear(O, x, r["o_proj"][:3], spec.bits, spec.group, stream=stream)
    n2 = G.rmsnorm(h, gamma2, eps, stream=stream)
    r["H_n2"] = run(("gate_proj", "up_proj"), n2)
    Y = G.mlp_forward(n2, r["gate_proj"][:3], r["up_proj"][:3], spec.bits, spec.group,
                      stream=stream)
    r["H_y"] = run(("down_proj",), Y)
    torch.cuda.synchronize()
    for nm in SUBLAYERS:
        r["loss_" + nm] = r["loss_" + nm].item()
    r.update(n1=n1, O=O, h=h, n2=n2, Y=Y)
    return r
