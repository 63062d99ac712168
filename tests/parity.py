"""Comparison of the GPU column solve with the oracle.

Codes are decided by rounding, so two correct implementations can differ where the value
being rounded sits next to a rounding boundary, and a flipped code then changes the
compensation of the rest of its row.  The comparison runs the oracle with a tie hook: where
the oracle's own float32 value lies within TIE_TOL (1e-3 of a step) of k + 1/2 and the GPU
chose k or k+1, the oracle keeps the GPU's choice and counts it.  The oracle's arithmetic
never takes values from the GPU; only the choice at those positions is followed, so that
the rest of the row stays comparable.

Pass criteria (from the parity bar for this path):
  * every code and zero point equal to the followed oracle's (a mismatch anywhere else
    means a mismatch that is not within 1e-3 of a boundary);
  * followed ties <= 0.1% of the codes (so >= 99.9% are identical);
  * scales within 1e-5 relative;
  * the layer loss within 0.5% relative of the oracle's own (unfollowed) loss.
"""

from __future__ import annotations

import numpy as np

import oracle as O


def follow_hook(gpu_codes: np.ndarray, gpu_zeros: np.ndarray, g: int):
    log = {"code": 0, "zero": 0}

    def hook(kind, q, rows, own, lo, hi):
        if kind == "code":
            theirs = gpu_codes[rows, q]
        else:
            theirs = gpu_zeros[rows, q // g].astype(np.int64)
        ok = (theirs == lo) | (theirs == hi)
        out = np.where(ok, theirs, own)
        log[kind] += int(np.count_nonzero(out != own))
        return out

    return hook, log


def compare(W, G, spec, gpu_codes, gpu_scales, gpu_zeros, H=None, gpu_loss=None,
            block=None, code_frac=1e-3, scale_rtol=1e-5, loss_rtol=5e-3, unfollowed=None):
    """Returns a dict of statistics; raises AssertionError when a criterion fails."""
    bits, group, sym = spec["bits"], spec["group"], spec["sym"]
    d_col = W.shape[1]
    g = d_col if group == 0 else group
    gpu_codes = np.asarray(gpu_codes, np.int64)
    gpu_zeros = np.asarray(gpu_zeros, np.int64)
    hook, log = follow_hook(gpu_codes, gpu_zeros, g)
    fol = O.gptq_quantize(W, G, bits, group, sym, block=block, tie_hook=hook)
    ref = unfollowed if unfollowed is not None else O.gptq_quantize(W, G, bits, group, sym, block=block)
    n = gpu_codes.size
    stats = {
        "raw_agree": float(np.mean(ref["codes"] == gpu_codes)),
        "follow_agree": float(np.mean(fol["codes"] == gpu_codes)),
        "ties_followed": log["code"] + log["zero"],
        "tie_frac": (log["code"] + log["zero"]) / n,
        "scale_rel": float(np.max(np.abs(gpu_scales.astype(np.float64) - fol["scales"]) /
                                  np.abs(fol["scales"].astype(np.float64)))),
    }
    bad = np.argwhere(fol["codes"] != gpu_codes)
    assert bad.size == 0, "codes differ away from rounding boundaries at %s (gpu %s, oracle %s, v %s)" % (
        bad[:5].tolist(), gpu_codes[tuple(bad[:5].T)], fol["codes"][tuple(bad[:5].T)],
        fol["V"][tuple(bad[:5].T)])
    assert np.array_equal(fol["zeros"], gpu_zeros), "zero points differ"
    assert stats["tie_frac"] <= code_frac, stats
    assert stats["scale_rel"] <= scale_rtol, stats
    if H is not None:
        ref_loss = O.layer_loss(W, ref["w_hat"], H)
        w_hat_gpu = O.dequantize(gpu_codes, gpu_scales, gpu_zeros, g)
        gl = O.layer_loss(W, w_hat_gpu, H)
        stats["loss_oracle"] = ref_loss
        stats["loss_gpu_codes"] = gl
        stats["loss_rel"] = abs(gl - ref_loss) / ref_loss
        assert stats["loss_rel"] <= loss_rtol, stats
        if gpu_loss is not None:
            stats["check_rel"] = abs(gpu_loss - gl) / gl
            assert stats["check_rel"] <= 1e-4, stats
    stats["fol"] = fol
    return stats
