#!/usr/bin/env python3
"""Throughput of GPTQ layer quantization on one MI355X.

One step = the whole hot path for one linear layer with its inputs resident in HBM:
  H = 0; H += 2 X^T X over all calibration tokens   (gptq_hessian_accumulate)
  G = Cholesky((H + lambda I)^-1)^T                  (gptq_prepare_hinv)
  packed codes, scales, zeros                        (gptq_quantize_layer)
Metric: weights quantized per second for the layer (d_row * d_col / step time).

Workload (default): q_proj-shaped layer, W 4096 x 4096 fp16 ~ N(0, 0.02^2), X 262144 tokens
(128 sequences x 2048) fp16 with lognormal channel scales, INT4 symmetric, group 128, B = 128,
damping 1% of mean diag(H).  Synthetic, seeded inputs (post_weight_quantization_24_amd.synth).

Also printed: the roofline of the dominant kernel (its per-launch duration from HIP events
recorded by the library around each launch on the stream it runs on) and the CPU oracle timed
on a bounded sample of the same workload.  After the timed steps, outside the metric: the
weight-only quantized product over packed weights (`w4a16`) and AWQ's activation-aware scale
search on the same layer and tokens (`awq`), with the layer losses of round-to-nearest, of
AWQ's choice and of the GPTQ output; and one LLaMA-7B-shaped decoder layer quantized layer
by layer on the same tokens (`decoder_block`: each sub-layer calibrated on the output of the
quantized sub-layers before it, through RMSNorm, rotary causal attention and the MLP).
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "GPTQ weights quantized/sec per layer (INT4 g128); % MFMA & HBM roofline"
PEAK = {"mfma_f16": 2516.6, "mfma_f32": 157.3, "hbm": 8000.0}   # TFLOP/s, TFLOP/s, GB/s


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=5)
    p.add_argument("--warmup", type=int, default=2)
    p.add_argument("--workload", default="qproj_4096")
    p.add_argument("--layer", default=None)
    p.add_argument("--bits", type=int, default=None)
    p.add_argument("--block", type=int, default=None)
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--no-w4a16", action="store_true",
                   help="skip the weight-only quantized product leg")
    p.add_argument("--no-awq", action="store_true",
                   help="skip the AWQ scale-search leg after the timed steps")
    p.add_argument("--no-block", action="store_true",
                   help="skip the layer-sequential decoder-block leg after the timed steps")
    p.add_argument("--no-configs", action="store_true",
                   help="skip the per-layer runs of the 7B layer, 70B MLP and outlier workloads")
    p.add_argument("--cpu-tokens", type=int, default=16384)
    p.add_argument("--cpu-rows", type=int, default=128)
    p.add_argument("--traffic", default=os.path.join(ROOT, "profiles", "traffic.json"),
                   help="JSON with the HBM bytes per launch of kernel families, from rocprofv3 "
                        "FETCH_SIZE/WRITE_SIZE passes; used only while the kernel source is unchanged")
    p.add_argument("--calib-copy-mib", type=int, default=0,
                   help="before the steps, run one elementwise copy (torch.neg) of this many MiB: "
                        "the reference dispatch for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE")
    return p.parse_args()


# Kernel families of the inverse factor.  Its blocked schedule runs trailing updates and tree
# products inside the launches that carry a leaf, so the work is not split between these
# families: they are timed one by one, and the roofline is taken for the phase as a whole.
PREP_FAMILIES = ("prep_damp", "prep_leaf", "prep_gemm")


def family_work(fam, d_row, d_col, n_tok, bits, block, x_dtype):
    """Algorithmic work of one step for a kernel family: (amount, unit, peak, bound)."""
    f32, f16, hbm = PEAK["mfma_f32"], PEAK["mfma_f16"], PEAK["hbm"]
    if fam == "prepare":           # the factor H_d = U U^T and its inverse: d^3 / 3 flops each
        return 2 * d_col ** 3 // 3, "TFLOP/s", f32, "mfma"
    if fam == "hessian_mfma":      # the d (d + 1) / 2 distinct entries, 2 flops per token each
        return n_tok * d_col * (d_col + 1), "TFLOP/s", f16 if x_dtype == "f16" else f32, "mfma"
    if fam == "lazy_gemm":         # sum over blocks of 2 d_row B (d_col - j - B)
        return d_row * d_col * (d_col - block), "TFLOP/s", f32, "mfma"
    if fam == "quant_block":       # read W, write E and codes, read the G blocks
        return d_row * d_col * (8 + bits / 8) + d_col * block * 4, "GB/s", hbm, "hbm"
    if fam == "quant_convert":
        return d_row * d_col * 6, "GB/s", hbm, "hbm"
    if fam == "quant_group_params":  # each group's columns read once, scales and zeros written
        return d_row * d_col * 4, "GB/s", hbm, "hbm"
    if fam == "hessian_reduce":    # H read and written (the partial tiles are extra)
        return d_col * d_col * 8, "GB/s", hbm, "hbm"
    return d_col * d_col * 8, "GB/s", hbm, "hbm"


KERNEL_SOURCE = {   # kernel family -> the source file its counters were taken from
    "hessian_mfma": "hessian.hip", "hessian_reduce": "hessian.hip", "lazy_gemm": "gemm.hip",
    "quant_block": "quant.hip",
}


def source_sha256(name):
    import hashlib
    path = os.path.join(ROOT, "post_weight_quantization_24_amd", "csrc", name)
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def kernel_traffic(path, family, **cfg):
    """HBM bytes per launch of `family` measured with rocprofv3 counters (profiles/), or None
    when there is no measurement for this workload or the kernel source has changed since."""
    if not path or not os.path.exists(path) or family not in KERNEL_SOURCE:
        return None
    with open(path) as f:
        table = json.load(f)
    for e in table.get("entries", []):
        if e.get("kernel") != family or any(e.get(k) != v for k, v in cfg.items()):
            continue
        if e.get("source_sha256") != source_sha256(KERNEL_SOURCE[family]):
            return None
        return e["hbm_bytes_per_launch"]
    return None


def w4a16_leg(G, torch, dev, layers, reps=100):
    """The weight-only quantized product over packed weights (one fp16 activation row): average
    launch time from HIP events on the launch stream, against the HBM roofline.  Algorithmic
    bytes per launch: the packed codes, the scales and zeros, x and y."""
    out = []
    for name, qw, sc, ze, bits, group in layers:
        d_row, d_col = qw.shape[0], qw.shape[1] * 32 // bits
        g = d_col if group == 0 else group
        x = torch.randn((1, d_col), device=dev).to(torch.float16)
        y = torch.empty((1, d_row), dtype=torch.float32, device=dev)
        for _ in range(3):
            G.dequant_matvec(qw, sc, ze, x, bits, group, d_col, y=y)
        torch.cuda.synchronize()
        G.profile_reset()
        G.profile_only("dequant_matvec")
        G.profile_enable(True)
        for _ in range(reps):
            G.dequant_matvec(qw, sc, ze, x, bits, group, d_col, y=y)
        torch.cuda.synchronize()
        G.profile_enable(False)
        G.profile_only(None)
        n, ms = G.profile_read("dequant_matvec")
        avg_s = ms / n / 1e3
        nbytes = d_row * d_col * bits // 8 + d_row * (d_col // g) * 5 + d_col * 2 + d_row * 4
        ach = nbytes / avg_s / 1e9
        out.append({"layer": name, "d_row": d_row, "d_col": d_col, "bits": bits, "group": group,
                    "n": 1, "avg_launch_us": avg_s * 1e6, "bytes_per_launch": nbytes,
                    "achieved": ach, "peak": PEAK["hbm"], "unit": "GB/s", "frac": ach / PEAK["hbm"]})
    return out


def awq_leg(G, torch, Wd, Xd, H, gptq_out, spec, n_grid=20):
    """AWQ's scale search on the same layer and tokens (gptq_act_absmean over all tokens, then
    gptq_awq_search over n_grid exponents against the undamped H of the timed steps): wall time
    of the whole search from events on the launch stream, the loss product against the fp32
    MFMA roofline (D times the upper triangle of H: d_row d_col (d_col + 1) flops per grid
    point), the magnitude pass against HBM, and
    the layer loss of round-to-nearest (alpha = 0), of the search's choice and of this bench's
    GPTQ output on the same H."""
    d_row, d_col = Wd.shape
    n_tok = Xd.shape[0]
    dev = Wd.device
    sx = torch.zeros(d_col, dtype=torch.float64, device=dev)
    ws_a = torch.empty(max(G.lib().gptq_act_absmean_workspace_size(d_col, n_tok), 256),
                       dtype=torch.uint8, device=dev)
    ws_s = torch.empty(G.lib().gptq_awq_workspace_size(d_row, d_col), dtype=torch.uint8,
                       device=dev)

    def run():
        sx.zero_()
        G.act_absmean(sx, Xd, ws=ws_a)
        return G.awq_search(Wd, H, sx, n_tok, spec, n_grid, ws=ws_s)

    run()
    torch.cuda.synchronize()
    G.profile_reset()
    G.profile_only(None)
    G.profile_enable(True)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    qw, sc, ze, s, losses, best = run()
    e1.record()
    torch.cuda.synchronize()
    G.profile_enable(False)
    ms = e0.elapsed_time(e1)
    n_g, ms_g = G.profile_read("awq_gemm")
    n_a, ms_a = G.profile_read("absmean")
    n_r, ms_r = G.profile_read("awq_scale_rtn")
    gemm_tf = float(d_row) * d_col * (d_col + 1) / (ms_g / n_g / 1e3) / 1e12
    am_gbs = n_tok * d_col * Xd.element_size() / (ms_a / n_a / 1e3) / 1e9
    loss_gptq = G.dequant_check(gptq_out[0], gptq_out[1], gptq_out[2], Wd, H, spec)[0].item()
    lo = losses.cpu().numpy()
    b = int(best.item())
    return {"n_grid": n_grid, "ms": ms, "weights_per_s": d_row * d_col / (ms / 1e3),
            "alpha": b / (n_grid - 1), "loss_rtn": float(lo[0]), "loss_awq": float(lo[b]),
            "loss_gptq": loss_gptq,
            "loss_gemm": {"launches": n_g, "avg_launch_ms": ms_g / n_g, "achieved": gemm_tf,
                          "peak": PEAK["mfma_f32"], "unit": "TFLOP/s",
                          "frac": gemm_tf / PEAK["mfma_f32"]},
            "scale_rtn_ms": ms_r,
            "absmean": {"ms": ms_a / n_a, "achieved": am_gbs, "peak": PEAK["hbm"],
                        "unit": "GB/s", "frac": am_gbs / PEAK["hbm"]}}


def block_leg(G, torch, dev, bits, seq_len=2048):
    """Layer-sequential quantization of one LLaMA-7B-shaped decoder layer
    (block.quantize_decoder_block: q/k/v_proj on rmsnorm(x), o_proj on the attention output of
    the quantized q/k/v, gate/up_proj on rmsnorm of the residual, down_proj on the MLP product
    of the quantized gate/up) on the 7B-layer workload's seeded inputs: its sub-layer weights,
    its 131072 calibration tokens (64 sequences of 2048) as the layer input, norm weights
    exp(0.2 N(0, 1)); asymmetric g128, B = 128.  Wall time from events on the launch stream,
    the time of each kernel family, and the attention kernel against the fp32 MFMA peak
    (2 * 128 * l (l + 1) flops per head and sequence of l tokens: q.k and p.v over the causal
    pairs) and the forward products (fp16 activations times the codes as fp16 integers,
    2 n_tok d (4 d + 2 d_ff) flops) against the fp16 MFMA peak."""
    from post_weight_quantization_24_amd import block as BLK
    from post_weight_quantization_24_amd import synth
    wl = synth.WORKLOADS["llama7b_layer"]
    d, d_ff = wl.layer("q_proj").d_col, wl.layer("gate_proj").d_row
    n_tok = wl.n_tok
    Xd = torch.empty((n_tok, d), dtype=torch.float16, device=dev)
    for t in range(0, n_tok, 32768):
        part = synth.layer_acts(wl, "attn_in", n_tok=min(32768, n_tok - t), tok_start=t)
        Xd[t:t + part.shape[0]].copy_(torch.from_numpy(part))
    shapes = {l.name: (l.d_row, l.d_col) for l in wl.layers}
    W = {k: torch.from_numpy(synth.layer_weight(wl, k)).to(dev) for k in shapes}
    g1, g2 = (torch.from_numpy(synth.gen_norm_weight(wl.wid, nm, d)).to(dev)
              for nm in ("input_layernorm", "post_attention_layernorm"))
    spec = G.Spec.make(bits, wl.group, wl.sym, 128, wl.damp)
    BLK.quantize_decoder_block(W, Xd, g1, g2, spec, seq_len)          # warm-up
    torch.cuda.synchronize()
    G.profile_reset()
    G.profile_only(None)
    G.profile_enable(True)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    r = BLK.quantize_decoder_block(W, Xd, g1, g2, spec, seq_len)
    e1.record()
    torch.cuda.synchronize()
    G.profile_enable(False)
    ms = e0.elapsed_time(e1)
    fams = {}
    for f in ("hessian_mfma", "hessian_reduce", "prep_gemm", "prep_leaf", "prep_damp", "quant_block",
              "lazy_gemm", "quant_group_params", "quant_convert", "check", "check_gemm",
              "attention", "block_gemm", "mlp_gemm", "block_elementwise", "mlp_elementwise"):
        n, t = G.profile_read(f)
        if n:
            fams[f] = {"launches": n, "ms": t}
    n_seq_full, tail = divmod(n_tok, seq_len)
    pairs = n_seq_full * seq_len * (seq_len + 1) + tail * (tail + 1)
    attn_flops = 2.0 * 128 * pairs * (d // 128)
    n_a, ms_a = G.profile_read("attention")
    attn_tf = attn_flops / (ms_a / 1e3) / 1e12
    fwd_flops = 2.0 * n_tok * d * (4 * d + 2 * d_ff)
    ms_f = sum(G.profile_read(f)[1] for f in ("block_gemm", "mlp_gemm"))
    fwd_tf = fwd_flops / (ms_f / 1e3) / 1e12
    weights = sum(a * b for a, b in shapes.values())
    out = {"config": {"workload": wl.name, "d": d, "d_ff": d_ff, "heads": d // 128,
                      "seq_len": seq_len, "n_tok": n_tok, "bits": spec.bits, "group": spec.group,
                      "sym": bool(spec.sym), "block": spec.block},
           "ms": ms, "weights": weights, "weights_per_s": weights / (ms / 1e3),
           "families_ms": fams,
           "attention": {"launches": n_a, "ms": ms_a, "achieved": attn_tf, "peak": PEAK["mfma_f32"],
                         "unit": "TFLOP/s", "bound": "mfma", "frac": attn_tf / PEAK["mfma_f32"]},
           "forward_gemm": {"ms": ms_f, "achieved": fwd_tf, "peak": PEAK["mfma_f16"],
                            "unit": "TFLOP/s", "frac": fwd_tf / PEAK["mfma_f16"]},
           "losses": {k: r["loss_" + k] for k in shapes}}
    del r, W, Xd
    return out


# Per-layer runs of the larger workloads: (workload, input, [(layer, k)], bit widths, blocks).
# k = the number of sub-layers of a real model that share the layer's Hessian and G (q/k/v:
# 3, gate/up: 2, every other layer 1); t_layer = t_hessian / k + t_prepare / k + t_quantize.
CONFIG_RUNS = [
    ("llama7b_layer", "attn_in", [("q_proj", 3), ("k_proj", 3), ("v_proj", 3), ("gate_proj", 2),
                                  ("up_proj", 2)], (4, 3), (128,)),
    ("llama7b_layer", "o_in", [("o_proj", 1)], (4, 3), (128,)),
    ("llama7b_layer", "down_in", [("down_proj", 1)], (4, 3), (128,)),
    ("llama70b_mlp", "mlp_in", [("gate_proj", 2), ("up_proj", 2)], (4,), (128,)),
    ("llama70b_mlp", "down_in", [("down_proj", 1)], (4,), (128,)),
    ("outlier_8192", "x", [("w", 1)], (2, 3), (32, 64, 128, 256)),
]


def progress(msg):
    print("bench: " + msg, file=sys.stderr, flush=True)


def configs_leg(G, torch, dev, reps=3):
    """Every layer, bit width and block size of the four larger workloads at full size, on
    their seeded inputs: the Hessian and the inverse factor once per calibration input, the
    column solve once per layer, bit width and block size.  Wall times are medians of `reps`
    runs between HIP events on the launch stream (after one warm-up); one more run with
    every kernel family timed gives each phase's fraction of its roofline."""
    import ctypes
    from post_weight_quantization_24_amd import synth
    out = []

    def timed(fn):
        fn()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return sorted(ts)[len(ts) // 2]

    def families(fn, fams):
        G.profile_reset()
        G.profile_only(None)
        G.profile_enable(True)
        fn()
        torch.cuda.synchronize()
        G.profile_enable(False)
        return {f: G.profile_read(f) for f in fams}

    for wl_name, xname, layers, bit_list, blocks in CONFIG_RUNS:
        wl = synth.WORKLOADS[wl_name]
        d, n_tok = wl.x_dim(xname), wl.n_tok
        Xd = torch.empty((n_tok, d), dtype=torch.float16, device=dev)
        for t in range(0, n_tok, 32768):
            part = synth.layer_acts(wl, xname, n_tok=min(32768, n_tok - t), tok_start=t)
            Xd[t:t + part.shape[0]].copy_(torch.from_numpy(part))
        H = torch.empty((d, d), dtype=torch.float32, device=dev)
        Gm = torch.empty_like(H)
        L = G.lib()
        ws_h = torch.empty(max(L.gptq_hessian_workspace_size(d, n_tok, d, 0), 256),
                           dtype=torch.uint8, device=dev)
        ws_p = torch.empty(L.gptq_prepare_workspace_size(d), dtype=torch.uint8, device=dev)

        def run_h():
            H.zero_()
            G.hessian_accumulate(H, Xd, ws=ws_h)

        def run_p():
            G.prepare_hinv(H, G=Gm, damp_frac=wl.damp, ws=ws_p, check=False)

        t_h = timed(run_h)
        f_h = families(run_h, ("hessian_mfma", "hessian_reduce"))
        t_p = timed(run_p)
        G.prepare_hinv(H, G=Gm, damp_frac=wl.damp, ws=ws_p, check=True)   # pivots checked once
        f_p = families(run_p, ("prep_damp", "prep_leaf", "prep_gemm"))
        del Xd, ws_h
        for layer_name, k in layers:
            layer = wl.layer(layer_name)
            d_row = layer.d_row
            Wd = torch.from_numpy(synth.layer_weight(wl, layer_name)).to(dev)
            for bits in bit_list:
                for block in blocks:
                    spec = G.Spec.make(bits, wl.group, wl.sym, block, wl.damp)
                    g = d if wl.group == 0 else wl.group
                    qw = torch.empty((d_row, d * bits // 32), dtype=torch.int32, device=dev)
                    sc = torch.empty((d_row, d // g), dtype=torch.float32, device=dev)
                    ze = torch.empty((d_row, d // g), dtype=torch.uint8, device=dev)
                    esq = torch.empty(d_row, dtype=torch.float64, device=dev)
                    ws_q = torch.empty(L.gptq_quantize_workspace_size(d_row, d, ctypes.byref(spec)),
                                       dtype=torch.uint8, device=dev)

                    def run_q():
                        G.quantize_layer(Wd, Gm, spec, qweight=qw, scales=sc, zeros=ze,
                                         err_sq=esq, ws=ws_q)

                    t_q = timed(run_q)
                    f_q = families(run_q, ("quant_convert", "quant_group_params", "quant_block",
                                           "lazy_gemm"))
                    phases = {}
                    for fam, (n, ms) in list(f_h.items()) + list(f_p.items()) + list(f_q.items()):
                        if not n:
                            continue
                        if fam in PREP_FAMILIES:      # timed alone; the roofline is "prepare"'s
                            phases[fam] = {"ms": ms, "launches": n}
                            continue
                        work, unit, peak, bound = family_work(fam, d_row, d, n_tok, bits, block,
                                                              "f16")
                        ach = work / (ms / 1e3) / (1e12 if unit == "TFLOP/s" else 1e9)
                        phases[fam] = {"ms": ms, "launches": n, "bound": bound, "achieved": ach,
                                       "unit": unit, "frac": ach / peak}
                    work, unit, peak, bound = family_work("prepare", d_row, d, n_tok, bits, block,
                                                          "f16")
                    ach = work / (t_p / 1e3) / 1e12   # t_p: the whole call, between HIP events
                    phases["prepare"] = {"ms": t_p, "bound": bound, "achieved": ach, "unit": unit,
                                         "frac": ach / peak}
                    t_layer = t_h / k + t_p / k + t_q
                    out.append({
                        "workload": wl_name, "layer": layer_name, "d_row": d_row, "d_col": d,
                        "n_tok": n_tok, "bits": bits, "group": wl.group, "sym": bool(wl.sym),
                        "block": block, "k_shared": k, "hessian_ms": t_h, "prepare_ms": t_p,
                        "quantize_ms": t_q, "t_layer_ms": t_layer,
                        "weights_per_s": d_row * d / (t_layer / 1e3),
                        "quantize_only_weights_per_s": d_row * d / (t_q / 1e3),
                        "phases": phases})
                    del qw, sc, ze, esq, ws_q
                    progress("%s %s INT%d B=%d: %.2f ms per layer" % (wl_name, layer_name, bits,
                                                                      block, t_layer))
            del Wd
        del H, Gm, ws_p
        torch.cuda.empty_cache()
    return out


def host_description():
    """os.cpu_count(), the CPU model from /proc/cpuinfo and the threads of the host BLAS
    libraries the oracle uses (numpy's and torch's)."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.lower().startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = {}
    try:
        from threadpoolctl import threadpool_info
        for i in threadpool_info():
            blas["%s:%s" % (i.get("user_api"), i.get("internal_api"))] = i.get("num_threads")
    except Exception:  # pragma: no cover
        pass
    import torch
    blas["torch"] = torch.get_num_threads()
    return {"cpu_count": os.cpu_count(), "cpu_model": model, "blas_threads": blas}


def cpu_baseline(W, X_sample, n_tok_full, spec, rows):
    """The oracle as it stands on a bounded sample: Hessian on X_sample (scaled to all tokens),
    the inverse factor at full size, the column loop on `rows` rows (scaled to all rows).
    `value` is the rate projected to the whole layer from the measured sample times."""
    import oracle as O
    host = host_description()
    d_row, d_col = W.shape
    t0 = time.perf_counter()
    H = O.hessian(X_sample)
    t_h = time.perf_counter() - t0
    H *= n_tok_full / X_sample.shape[0]
    t0 = time.perf_counter()
    Gm = O.prepare_g(H, spec["damp"])
    t_p = time.perf_counter() - t0
    t0 = time.perf_counter()
    O.gptq_quantize(W[:rows], Gm, spec["bits"], spec["group"], spec["sym"], block=spec["block"])
    t_q = time.perf_counter() - t0
    t_layer = t_h * (n_tok_full / X_sample.shape[0]) + t_p + t_q * (d_row / rows)
    threads = max([v for v in host["blas_threads"].values() if v] + [1])
    return {
        "value": d_row * d_col / t_layer,
        "unit": "weights/s",
        "cores": threads,
        "kind": "oracle",
        "projected": True,
        "sample": "Hessian on %d of %d tokens (x%.0f), inverse factor at full size, column loop "
                  "on %d of %d rows (x%.0f); measured %.1f s, projected %.1f s per layer"
                  % (X_sample.shape[0], n_tok_full, n_tok_full / X_sample.shape[0], rows, d_row,
                     d_row / rows, t_h + t_p + t_q, t_layer),
        "measured_s": {"hessian": t_h, "prepare": t_p, "column_loop": t_q},
        "host": host,
    }


def main():
    a = parse()
    if a.gpus != 1:
        print("bench.py: measures one GPU; --gpus %d is not supported (across GPUs the layer "
              "would shard by output rows and by token ranges)" % a.gpus, file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from post_weight_quantization_24_amd import gptq as G
    from post_weight_quantization_24_amd import synth

    wl = synth.WORKLOADS[a.workload]
    layer = wl.layer(a.layer) if a.layer else wl.layers[0]
    bits = a.bits or wl.bits[0]
    block = a.block or wl.blocks[0]
    d_row, d_col, n_tok = layer.d_row, layer.d_col, wl.n_tok
    spec_d = dict(bits=bits, group=wl.group, sym=bool(wl.sym), block=block, damp=wl.damp)
    spec = G.Spec.make(bits, wl.group, wl.sym, block, wl.damp)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    # ---- inputs resident in HBM
    t0 = time.perf_counter()
    W = synth.layer_weight(wl, layer.name)
    Wd = torch.from_numpy(W).to(dev)
    Xd = torch.empty((n_tok, d_col), dtype=torch.float16 if wl.dtype == "f16" else torch.float32,
                     device=dev)
    chunk = 32768
    X_sample = None
    for t in range(0, n_tok, chunk):
        part = synth.layer_acts(wl, layer.x, n_tok=min(chunk, n_tok - t), tok_start=t)
        if X_sample is None:
            X_sample = part[:min(a.cpu_tokens, part.shape[0])].copy()
        Xd[t:t + part.shape[0]].copy_(torch.from_numpy(part))
    torch.cuda.synchronize()
    gen_s = time.perf_counter() - t0

    H = torch.empty((d_col, d_col), dtype=torch.float32, device=dev)
    Gm = torch.empty_like(H)
    L = G.lib()
    ws_h = torch.empty(max(L.gptq_hessian_workspace_size(d_col, n_tok, d_col, G._dtype_code(Xd)), 256),
                       dtype=torch.uint8, device=dev)
    ws_p = torch.empty(L.gptq_prepare_workspace_size(d_col), dtype=torch.uint8, device=dev)
    import ctypes
    ws_q = torch.empty(L.gptq_quantize_workspace_size(d_row, d_col, ctypes.byref(spec)),
                       dtype=torch.uint8, device=dev)
    g = d_col if wl.group == 0 else wl.group
    qweight = torch.empty((d_row, d_col * bits // 32), dtype=torch.int32, device=dev)
    scales = torch.empty((d_row, d_col // g), dtype=torch.float32, device=dev)
    zeros = torch.empty((d_row, d_col // g), dtype=torch.uint8, device=dev)
    esq = torch.empty(d_row, dtype=torch.float64, device=dev)

    def step(check):
        H.zero_()
        G.hessian_accumulate(H, Xd, ws=ws_h)
        G.prepare_hinv(H, G=Gm, damp_frac=wl.damp, ws=ws_p, check=check)
        G.quantize_layer(Wd, Gm, spec, qweight=qweight, scales=scales, zeros=zeros, err_sq=esq,
                         ws=ws_q)

    if a.calib_copy_mib:
        src = torch.ones(a.calib_copy_mib << 18, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.neg(src, out=dst)          # reads and writes calib_copy_mib MiB each
        torch.cuda.synchronize()
        del src, dst

    for _ in range(a.warmup):
        step(True)
    torch.cuda.synchronize()

    fams = ["hessian_mfma", "hessian_reduce", "prep_damp", "prep_leaf", "prep_gemm",
            "quant_convert", "quant_group_params", "quant_block", "lazy_gemm"]

    def read_phases(steps):
        out = {}
        for f in fams:
            n, ms = G.profile_read(f)
            if n:
                out[f] = {"launches_per_step": n / steps, "ms_per_step": ms / steps,
                          "avg_launch_ms": ms / n}
        return out

    progress("inputs resident, warm-up done")
    # ---- one untimed step with every kernel family timed: the phase table
    G.profile_reset()
    G.profile_only(None)
    G.profile_enable(True)
    step(False)
    torch.cuda.synchronize()
    G.profile_enable(False)
    phases = read_phases(1)
    dom = max((f for f in phases if f not in PREP_FAMILIES), key=lambda k: phases[k]["ms_per_step"])
    for f, ph in phases.items():     # each family against its own roofline (this one step)
        if f in PREP_FAMILIES:
            continue
        work, unit, peak, bound = family_work(f, d_row, d_col, n_tok, bits, block, wl.dtype)
        ach = work / (ph["ms_per_step"] / 1e3) / (1e12 if unit == "TFLOP/s" else 1e9)
        ph.update({"bound": bound, "achieved": ach, "peak": peak, "unit": unit,
                   "frac": ach / peak})
    prep = [phases[f] for f in PREP_FAMILIES if f in phases]
    if prep:                         # the inverse factor as one phase (event overhead included)
        work, unit, peak, bound = family_work("prepare", d_row, d_col, n_tok, bits, block,
                                              wl.dtype)
        ms_p = sum(ph["ms_per_step"] for ph in prep)
        ach = work / (ms_p / 1e3) / 1e12
        phases["prepare"] = {"launches_per_step": sum(ph["launches_per_step"] for ph in prep),
                             "ms_per_step": ms_p, "bound": bound, "achieved": ach, "peak": peak,
                             "unit": unit, "frac": ach / peak}
    quant_ms = sum(phases[f]["ms_per_step"] for f in
                   ("quant_convert", "quant_group_params", "quant_block", "lazy_gemm")
                   if f in phases)

    # ---- timed region: K steps; HIP events around the dominant kernel's launches only
    G.profile_reset()
    G.profile_only(dom)
    G.profile_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(a.steps):
        step(False)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    G.profile_enable(False)
    G.profile_only(None)
    ms_per_step = elapsed * 1e3 / a.steps
    progress("timed steps: %.3f ms per step" % ms_per_step)
    timed = read_phases(a.steps)[dom]
    avg_s = timed["avg_launch_ms"] / 1e3
    launches_per_step = timed["launches_per_step"]
    work, unit, peak, bound = family_work(dom, d_row, d_col, n_tok, bits, block, wl.dtype)
    achieved = work / launches_per_step / avg_s / (1e12 if unit == "TFLOP/s" else 1e9)
    traffic = kernel_traffic(a.traffic, dom, workload=wl.name, layer=layer.name, bits=bits,
                             block=block)
    roofline = {"bound": bound, "achieved": achieved, "peak": peak, "unit": unit,
                "frac": achieved / peak, "traffic": traffic, "kernel": dom,
                "work_per_launch": work / launches_per_step}

    # ---- the weight-only quantized product over packed weights: this layer's GPTQ output and
    # a 70B-shaped gate_proj (28672 x 8192 INT4 g128, random packed codes)
    w4 = None
    if not a.no_w4a16:
        big_rows, big_cols = 28672, 8192
        bq = torch.randint(-2 ** 31, 2 ** 31 - 1, (big_rows, big_cols * 4 // 32), dtype=torch.int32,
                           device=dev)
        bs = torch.rand((big_rows, big_cols // 128), device=dev) * 0.02 + 0.002
        bz = torch.randint(0, 16, (big_rows, big_cols // 128), dtype=torch.uint8, device=dev)
        layers = [("%s %dx%d (GPTQ output of this bench)" % (layer.name, d_row, d_col), qweight,
                   scales, zeros, bits, wl.group),
                  ("gate_proj 28672x8192 INT4 g128 (random codes)", bq, bs, bz, 4, 128)]
        own_ok = wl.group % 32 == 0 and d_col <= 32768      # the call's shape limits
        w4 = w4a16_leg(G, torch, dev, layers if own_ok else layers[1:])
        # context: the same product with fp16 weights through the library GEMM (torch), the
        # unquantized alternative whose 4x larger weight read the packed format avoids
        w16 = torch.randn((big_rows, big_cols), device=dev).to(torch.float16)
        xb = torch.randn((1, big_cols), device=dev).to(torch.float16)
        for _ in range(3):
            torch.matmul(xb, w16.t())
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(50):
            torch.matmul(xb, w16.t())
        e1.record()
        torch.cuda.synchronize()
        ref_us = e0.elapsed_time(e1) / 50 * 1e3
        w4[-1]["fp16_library_us"] = ref_us
        w4[-1]["speedup_vs_fp16"] = ref_us / w4[-1]["avg_launch_us"]
        # the batched regime: 2048 activation rows through the matrix-core path
        # (gptq_dequant_matmul), against the library fp16 GEMM on the dense weights
        nb = 2048
        xm = torch.randn((nb, big_cols), device=dev).to(torch.float16)
        ym = torch.empty((nb, big_rows), dtype=torch.float32, device=dev)
        wsm = torch.empty(max(G.lib().gptq_dequant_matmul_workspace_size(big_rows, big_cols, 4, 128),
                              256), dtype=torch.uint8, device=dev)
        for _ in range(2):
            G.dequant_matmul(bq, bs, bz, xm, 4, 128, big_cols, y=ym, ws=wsm)
        torch.cuda.synchronize()
        G.profile_reset()
        G.profile_enable(True)
        for _ in range(10):
            G.dequant_matmul(bq, bs, bz, xm, 4, 128, big_cols, y=ym, ws=wsm)
        torch.cuda.synchronize()
        G.profile_enable(False)
        n_m, ms_m = G.profile_read("dequant_matmul")
        n_e, ms_e = G.profile_read("dequant_expand")
        flops = 2.0 * nb * big_rows * big_cols
        for _ in range(3):
            torch.matmul(xm, w16.t())
        e0.record()
        for _ in range(10):
            torch.matmul(xm, w16.t())
        e1.record()
        torch.cuda.synchronize()
        lib_ms = e0.elapsed_time(e1) / 10
        tf = flops / (ms_m / n_m / 1e3) / 1e12
        w4[-1]["batched"] = {"n": nb, "product_ms": ms_m / n_m,
                             "expand_ms": ms_e / n_e if n_e else 0.0,
                             "workspace_bytes": G.lib().gptq_dequant_matmul_workspace_size(
                                 big_rows, big_cols, 4, 128),
                             "achieved": tf, "peak": PEAK["mfma_f16"], "unit": "TFLOP/s",
                             "frac": tf / PEAK["mfma_f16"], "fp16_library_ms": lib_ms}
        del w16, xb, xm, ym, wsm, bq, bs, bz

    # ---- AWQ's activation-aware scale search on the same layer, tokens and H
    awq = None
    if not a.no_awq:
        awq = awq_leg(G, torch, Wd, Xd, H, (qweight, scales, zeros), spec)
        progress("awq leg done")

    # ---- one decoder layer quantized layer by layer on the same tokens (7B shapes)
    blk = None
    if not a.no_block:
        blk = []
        for b in (4, 3):
            blk.append(block_leg(G, torch, dev, b))
            progress("decoder block INT%d: %.1f ms" % (b, blk[-1]["ms"]))

    # ---- every layer, bit width and block size of the larger workloads
    cfgs = None
    if not a.no_configs:
        del Xd
        torch.cuda.empty_cache()
        cfgs = configs_leg(G, torch, dev)

    cpu = None
    if not a.no_cpu:
        cpu = cpu_baseline(W, X_sample, n_tok, spec_d, min(a.cpu_rows, d_row))
        progress("cpu baseline done")

    out = {
        "metric": METRIC,
        "value": d_row * d_col / (ms_per_step / 1e3),
        "unit": "weights/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": wl.name, "layer": layer.name, "d_row": d_row, "d_col": d_col,
                   "n_tok": n_tok, "bits": bits, "group": wl.group, "sym": bool(wl.sym),
                   "block": block, "damp": wl.damp, "x_dtype": wl.dtype,
                   "accumulate": "f32"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "phases": phases,
        # the column solve alone (G given), from the same profiled step as the phase table
        "quantize_only": {"value": d_row * d_col / (quant_ms / 1e3), "unit": "weights/s"},
        "w4a16": w4,
        "awq": awq,
        "decoder_block": blk,
        "configs": cfgs,
        "step": "H = 0; H += 2 X^T X over all tokens; G = Cholesky((H + lambda I)^-1)^T; "
                "column solve with packing.  The positive-pivot check of G (one wait of the host "
                "on the stream) runs in the warm-up steps, not in the timed ones.",
        "input_gen_s": gen_s,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
