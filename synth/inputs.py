"""Seeded generator for one round's inputs.

Every tensor is drawn from numpy's PCG64 seeded by
``SeedSequence([seed, cfg_id, tensor_id, request, chunk])`` so the values do
not depend on thread count or machine.  Large tensors are drawn in fixed
chunks on a thread pool.

Distributions (stated per workload):
  * matrices ~ N(0, 1/fan_in) in fp32, fan_in = input width of the layer
    (W_lm: d, W1: d+s, W2: r, W_ih: e, W_hh: s);
  * the embedding table is a lookup (one-hot input), so fan_in = 1: N(0, 1);
  * GRU biases b_ih ~ N(0, 1/e), b_hh ~ N(0, 1/s);
  * H ~ N(0, 1) fp32 per request; root tokens uniform on [0, V);
  * a Zipf-like unigram bias bias[v] = -1.1 * ln(1 + pi(v)) with pi a seeded
    permutation of the vocabulary, so frequent tokens are scattered over ids.
bf16 weights are the fp32 draws rounded to nearest-even by torch's cast and
returned as raw uint16 bit patterns; fp32 weights are returned as float32.
"""
from concurrent.futures import ThreadPoolExecutor
import os

import numpy as np

from .configs import Config

T_WLM, T_EMB, T_WIH, T_WHH, T_W1, T_W2, T_PERM, T_H, T_ROOT, T_BIH, T_BHH = range(11)
_CHUNK = 1 << 23


def _rng(seed, cfg_id, tid, req=0, chunk=0):
    return np.random.Generator(np.random.PCG64(
        np.random.SeedSequence([int(seed), int(cfg_id), tid, req, chunk])))


def _normal(shape, scale, seed, cfg_id, tid, req=0):
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    nch = (n + _CHUNK - 1) // _CHUNK

    def fill(c):
        lo, hi = c * _CHUNK, min(n, (c + 1) * _CHUNK)
        x = _rng(seed, cfg_id, tid, req, c).standard_normal(hi - lo, dtype=np.float32)
        x *= np.float32(scale)
        out[lo:hi] = x

    if nch == 1:
        fill(0)
    else:
        workers = min(nch, max(1, min(16, os.cpu_count() or 1)))
        with ThreadPoolExecutor(workers) as ex:
            list(ex.map(fill, range(nch)))
    return out.reshape(shape)


def _to_bf16_bits(x32: np.ndarray) -> np.ndarray:
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def _weight(shape, fan_in, cfg, seed, tid):
    x = _normal(shape, 1.0 / np.sqrt(fan_in), seed, cfg.cfg_id, tid)
    return _to_bf16_bits(x) if cfg.wtype == "bf16" else x


def make_inputs(cfg: Config, seed: int = 0) -> dict:
    """Draw one round's weights, hidden states and root tokens."""
    d, V, e, s, r = cfg.d, cfg.V, cfg.e, cfg.s, cfg.r
    w = {
        "W_lm": _weight((V, d), d, cfg, seed, T_WLM),
        "Emb": _weight((V, e), 1, cfg, seed, T_EMB),
        "W_ih": _weight((3 * s, e), e, cfg, seed, T_WIH),
        "W_hh": _weight((3 * s, s), s, cfg, seed, T_WHH),
        "W1": _weight((r, d + s), d + s, cfg, seed, T_W1),
        "W2": _weight((V, r), r, cfg, seed, T_W2),
        "b_ih": _normal((3 * s,), 1.0 / np.sqrt(e), seed, cfg.cfg_id, T_BIH),
        "b_hh": _normal((3 * s,), 1.0 / np.sqrt(s), seed, cfg.cfg_id, T_BHH),
    }
    perm = _rng(seed, cfg.cfg_id, T_PERM).permutation(V)
    w["bias"] = (-1.1 * np.log1p(perm.astype(np.float64))).astype(np.float32)
    H = np.stack([_normal((cfg.D, d), 1.0, seed, cfg.cfg_id, T_H, q)
                  for q in range(cfg.batch)])
    root = np.array([_rng(seed, cfg.cfg_id, T_ROOT, q).integers(0, V)
                     for q in range(cfg.batch)], dtype=np.int32)
    return {"weights": w, "H": H, "root": root, "wtype": cfg.wtype}


def custom_config(**kw) -> Config:
    """A small workload for tests; cfg_id 1000+ keeps its seeds apart."""
    base = dict(name="custom", cfg_id=1000, d=64, V=512, e=32, s=32, r=16,
                D=4, M=8, K=2, W=4, B=16, beta=-0.1, batch=1, wtype="f32")
    base.update(kw)
    return Config(**base)
