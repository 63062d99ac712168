"""Seeded synthetic inputs for GPTQ layer quantization, and the workload registry.

This module only draws random numbers and describes workload shapes; it holds
none of the quantization method's arithmetic.  Both the GPU path and the CPU
oracle are fed from here, so the two consume bit-identical weights and
calibration activations.

Recipe (stands in for the LLaMA sub-layers listed on the page "大模型常见的量化方式"
(psvmc.cn), section on the layered structure of large models, calibrated on the
128 C4 segments named on the page "量化" (dingiv.github.io), section GPTQ; neither
the weights nor the text corpus exist here):

* weights  W[r, c] ~ N(0, sigma_w^2), cast to the layer dtype;
* channel scales sigma_c = exp(N(0, 0.5^2)) per input channel; optionally a
  seed-chosen fraction of channels is multiplied by a constant (outliers);
* activations X[t, c] = sigma_c * N(0, 1), token-major [n_tok, d], cast to the
  layer dtype, drawn in chunks of 4096 tokens, each chunk from its own stream;
* for small comparison layers only, correlated activations: the same channel
  scales times a rank-r Gaussian mixture plus independent noise (gen_acts_lowrank).

Every stream is numpy PCG64 seeded by SeedSequence(seed, spawn_key=(workload id,
crc32(tensor name), chunk)), so any chunk can be regenerated on its own.
"""

from __future__ import annotations

import dataclasses
import os
import zlib
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, List, Optional, Sequence

import numpy as np

CHUNK_TOKENS = 4096
_SIGMA_STREAM = 0x7FFF0001
_OUTLIER_STREAM = 0x7FFF0002


def _stream(seed: int, wid: int, name: str, sub: int) -> np.random.Generator:
    key = (int(wid), zlib.crc32(name.encode()) & 0x7FFFFFFF, int(sub))
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=key)))


def _np_dtype(dtype: str):
    return {"f16": np.float16, "f32": np.float32}[dtype]


def gen_weight(wid: int, name: str, d_row: int, d_col: int, sigma: float,
               dtype: str = "f16", seed: int = 0) -> np.ndarray:
    """W [d_row, d_col] ~ N(0, sigma^2) in the given storage dtype."""
    rng = _stream(seed, wid, "W:" + name, 0)
    w = rng.standard_normal((d_row, d_col)) * sigma
    return w.astype(_np_dtype(dtype))


def gen_norm_weight(wid: int, name: str, d: int, dtype: str = "f16", seed: int = 0) -> np.ndarray:
    """A normalization weight gamma [d] = exp(0.2 N(0, 1)) in the given storage dtype."""
    rng = _stream(seed, wid, "N:" + name, 0)
    return np.exp(0.2 * rng.standard_normal(d)).astype(_np_dtype(dtype))


def channel_sigma(wid: int, xname: str, d: int, seed: int = 0,
                  outlier_frac: float = 0.0, outlier_scale: float = 100.0) -> np.ndarray:
    """Per-input-channel scale sigma_c (float64): lognormal(0, 0.5), outliers scaled."""
    sig = np.exp(0.5 * _stream(seed, wid, "X:" + xname, _SIGMA_STREAM).standard_normal(d))
    n_out = int(round(outlier_frac * d))
    if n_out:
        idx = _stream(seed, wid, "X:" + xname, _OUTLIER_STREAM).choice(d, n_out, replace=False)
        sig[idx] *= outlier_scale
    return sig


def outlier_channels(wid: int, xname: str, d: int, seed: int = 0,
                     outlier_frac: float = 0.0) -> np.ndarray:
    n_out = int(round(outlier_frac * d))
    if not n_out:
        return np.zeros(0, np.int64)
    return np.sort(_stream(seed, wid, "X:" + xname, _OUTLIER_STREAM).choice(d, n_out, replace=False))


def gen_act_chunk(wid: int, xname: str, d: int, chunk: int, rows: int, sigma: np.ndarray,
                  dtype: str = "f16", seed: int = 0) -> np.ndarray:
    """Token rows [chunk*4096, chunk*4096 + rows) of X, shape [rows, d]."""
    z = _stream(seed, wid, "X:" + xname, chunk).standard_normal((rows, d))
    z *= sigma[None, :]
    return z.astype(_np_dtype(dtype))


def gen_acts(wid: int, xname: str, n_tok: int, d: int, dtype: str = "f16", seed: int = 0,
             outlier_frac: float = 0.0, outlier_scale: float = 100.0,
             out: Optional[np.ndarray] = None, tok_start: int = 0,
             threads: Optional[int] = None) -> np.ndarray:
    """X token-major [n_tok, d] starting at token tok_start (a multiple of 4096).

    Chunks are drawn in parallel; the result does not depend on the thread count.
    """
    if tok_start % CHUNK_TOKENS:
        raise ValueError("tok_start must be a multiple of 4096")
    sig = channel_sigma(wid, xname, d, seed, outlier_frac, outlier_scale)
    if out is None:
        out = np.empty((n_tok, d), _np_dtype(dtype))
    c0 = tok_start // CHUNK_TOKENS
    n_chunks = (n_tok + CHUNK_TOKENS - 1) // CHUNK_TOKENS

    def fill(i):
        t0 = i * CHUNK_TOKENS
        rows = min(CHUNK_TOKENS, n_tok - t0)
        out[t0:t0 + rows] = gen_act_chunk(wid, xname, d, c0 + i, rows, sig, dtype, seed)

    nthr = threads or min(16, os.cpu_count() or 1)
    if n_chunks == 1 or nthr == 1:
        for i in range(n_chunks):
            fill(i)
    else:
        with ThreadPoolExecutor(nthr) as ex:
            list(ex.map(fill, range(n_chunks)))
    return out


def gen_acts_lowrank(wid: int, xname: str, n_tok: int, d: int, rank: int,
                     noise: float = 0.3, dtype: str = "f32", seed: int = 0) -> np.ndarray:
    """Correlated calibration activations for small comparison layers: X[t, :] =
    sigma_c * (z_t M + noise * n_t), z_t ~ N(0, I_rank), M [rank, d] and n_t ~ N(0, 1),
    with the same lognormal channel scales as gen_acts.  Token-major [n_tok, d]; one
    stream, so only for small n_tok."""
    sig = channel_sigma(wid, xname, d, seed, 0.0, 1.0)
    rng = _stream(seed, wid, "LR:" + xname, 0)
    M = rng.standard_normal((rank, d))
    x = rng.standard_normal((n_tok, rank)) @ M + noise * rng.standard_normal((n_tok, d))
    return (x * sig).astype(_np_dtype(dtype))


# ----------------------------------------------------------------------------------
# Workload registry: the five synthetic workloads the throughput and parity runs use.
# ----------------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class Layer:
    name: str
    d_row: int
    d_col: int
    x: str               # name of the calibration activation tensor feeding this layer


@dataclasses.dataclass(frozen=True)
class Workload:
    wid: int
    name: str
    layers: Sequence[Layer]
    n_tok: int
    w_sigma: float
    dtype: str                       # storage dtype of W and X
    bits: Sequence[int]
    group: int                       # 0 = one group per output row
    sym: bool
    blocks: Sequence[int]
    damp: float = 0.01
    outlier_frac: float = 0.0
    outlier_scale: float = 100.0

    def layer(self, name: str) -> Layer:
        for l in self.layers:
            if l.name == name:
                return l
        raise KeyError(name)

    def x_dim(self, xname: str) -> int:
        for l in self.layers:
            if l.x == xname:
                return l.d_col
        raise KeyError(xname)


WORKLOADS: Dict[str, Workload] = {
    "single_256": Workload(
        0, "single_256", [Layer("w", 256, 256, "x")], n_tok=1024, w_sigma=0.02, dtype="f32",
        bits=(4,), group=0, sym=False, blocks=(128,)),
    "qproj_4096": Workload(
        1, "qproj_4096", [Layer("q_proj", 4096, 4096, "x")], n_tok=262144, w_sigma=0.02,
        dtype="f16", bits=(4,), group=128, sym=True, blocks=(128,)),
    "llama7b_layer": Workload(
        2, "llama7b_layer",
        [Layer("q_proj", 4096, 4096, "attn_in"), Layer("k_proj", 4096, 4096, "attn_in"),
         Layer("v_proj", 4096, 4096, "attn_in"), Layer("o_proj", 4096, 4096, "o_in"),
         Layer("gate_proj", 11008, 4096, "attn_in"), Layer("up_proj", 11008, 4096, "attn_in"),
         Layer("down_proj", 4096, 11008, "down_in")],
        n_tok=131072, w_sigma=0.02, dtype="f16", bits=(4, 3), group=128, sym=False,
        blocks=(128,)),
    "llama70b_mlp": Workload(
        3, "llama70b_mlp",
        [Layer("gate_proj", 28672, 8192, "mlp_in"), Layer("up_proj", 28672, 8192, "mlp_in"),
         Layer("down_proj", 8192, 28672, "down_in")],
        n_tok=65536, w_sigma=0.015, dtype="f16", bits=(4,), group=128, sym=False,
        blocks=(128,)),
    "outlier_8192": Workload(
        4, "outlier_8192", [Layer("w", 8192, 8192, "x")], n_tok=131072, w_sigma=0.02,
        dtype="f16", bits=(2, 3), group=0, sym=False, blocks=(32, 64, 128, 256),
        outlier_frac=0.01),
}

WORKLOAD_ORDER: List[str] = ["single_256", "qproj_4096", "llama7b_layer", "llama70b_mlp",
                             "outlier_8192"]


def layer_weight(wl: Workload, layer: str, seed: int = 0, d_row: Optional[int] = None) -> np.ndarray:
    """The layer's weight; d_row < full takes the first rows of the same draw."""
    l = wl.layer(layer)
    w = gen_weight(wl.wid, l.name, l.d_row, l.d_col, wl.w_sigma, wl.dtype, seed)
    return w if d_row is None else w[:d_row]


def layer_acts(wl: Workload, xname: str, n_tok: Optional[int] = None, seed: int = 0,
               out: Optional[np.ndarray] = None, tok_start: int = 0) -> np.ndarray:
    d = wl.x_dim(xname)
    n = wl.n_tok if n_tok is None else n_tok
    return gen_acts(wl.wid, xname, n, d, wl.dtype, seed, wl.outlier_frac, wl.outlier_scale,
                    out=out, tok_start=tok_start)
