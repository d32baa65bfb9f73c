"""Seeded synthetic inputs: fp16 weights and prompt token ids.

This module is shared by the HIP path and the oracle's tests and holds none of
the method's arithmetic: it only draws numbers.

Recipe (the pages have no weights or prompts; the model they measure is a
trained 2.3B coding model which is not available, so shapes stand in for it):
  * every matrix is N(0, 0.02) drawn in float32 with numpy's PCG64 and rounded
    to float16 (round-to-nearest-even by numpy's astype);
  * RMSNorm gains are exactly 1 (not drawn);
  * a tensor is drawn in chunks of CHUNK_ELEMS elements; chunk c of tensor t
    uses SeedSequence([seed_index, 0, t, c]), so the result does not depend on
    how many threads draw it;
  * tensor order t: embed; per layer attn_norm, wq, wk, wv, wo, mlp_norm,
    w_gate, w_up, w_down; then final_norm, lm_head;
  * prompt ids are uniform in [0, vocab) from SeedSequence([seed_index, 1]).
Weight layout follows the [out, in] Linear convention: wq [H*hd, d],
wk/wv [Hkv*hd, d], wo [d, H*hd], w_gate/w_up [F, d], w_down [d, F],
embed/lm_head [V, d].
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, List, Tuple

import numpy as np

from .config import ModelConfig

STD = 0.02
CHUNK_ELEMS = 1 << 23
LAYER_TENSORS = ("attn_norm", "wq", "wk", "wv", "wo", "mlp_norm", "w_gate", "w_up", "w_down")


def tensor_shapes(cfg: ModelConfig) -> List[Tuple[str, Tuple[int, ...]]]:
    d, F = cfg.d_model, cfg.ffn_dim
    out = [("embed", (cfg.vocab, d))]
    for l in range(cfg.n_layers):
        shp = {
            "attn_norm": (d,), "wq": (cfg.q_dim, d), "wk": (cfg.kv_dim, d),
            "wv": (cfg.kv_dim, d), "wo": (d, cfg.q_dim), "mlp_norm": (d,),
            "w_gate": (F, d), "w_up": (F, d), "w_down": (d, F),
        }
        out += [(f"layers.{l}.{n}", shp[n]) for n in LAYER_TENSORS]
    out += [("final_norm", (d,)), ("lm_head", (cfg.vocab, d))]
    return out


def _fill_chunk(job):
    seed_index, t, c, flat, lo, hi, std = job
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed_index, 0, t, c])))
    tmp = g.standard_normal(hi - lo, dtype=np.float32)
    tmp *= np.float32(std)
    flat[lo:hi] = tmp.astype(np.float16)


def gen_weights(cfg: ModelConfig, seed_index: int | None = None, std: float = STD,
                threads: int | None = None,
                overrides: Dict[str, float] | None = None) -> Dict[str, np.ndarray]:
    """Return {name: float16 array}.  ``overrides`` maps a tensor-name suffix
    (e.g. "wq") to a different std, used only by test variants."""
    seed = cfg.seed_index if seed_index is None else seed_index
    threads = threads or min(16, os.cpu_count() or 1)
    out: Dict[str, np.ndarray] = {}
    jobs = []
    for t, (name, shape) in enumerate(tensor_shapes(cfg)):
        if name.endswith("norm"):
            out[name] = np.ones(shape, dtype=np.float16)
            continue
        s = std
        if overrides:
            for suf, v in overrides.items():
                if name.endswith(suf):
                    s = v
        arr = np.empty(shape, dtype=np.float16)
        out[name] = arr
        flat = arr.reshape(-1)
        n = flat.size
        for c, lo in enumerate(range(0, n, CHUNK_ELEMS)):
            jobs.append((seed, t, c, flat, lo, min(n, lo + CHUNK_ELEMS), s))
    if threads <= 1:
        for j in jobs:
            _fill_chunk(j)
    else:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(_fill_chunk, jobs))
    return out


def gen_prompt(cfg: ModelConfig, n: int | None = None, seed_index: int | None = None) -> np.ndarray:
    seed = cfg.seed_index if seed_index is None else seed_index
    n = cfg.prompt_len if n is None else n
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 1])))
    return g.integers(0, cfg.vocab, size=n, dtype=np.int64).astype(np.int32)


def layer(weights: Dict[str, np.ndarray], l: int, name: str) -> np.ndarray:
    return weights[f"layers.{l}.{name}"]
