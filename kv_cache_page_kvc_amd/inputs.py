"""Seeded synthetic KV-cache inputs shaped like the pages' workloads.

This module holds no codec arithmetic: it only draws random numbers, lays
them out in the engine layouts and picks page ids.  Both the GPU tests/bench
and the CPU oracle checks take their inputs from here.

Distributions (stand-ins for the pages' models; no model weights or
datasets are used):
  K: N(0,1) times a lognormal(0,1) scale per (layer, head, channel);
  K (outlier variant): N(0,1) with Bernoulli(0.02) outlier channels per
     (layer, head, channel) scaled by 20;
  V: N(0,1).
Each (layer, component) tensor is drawn from its own generator seeded with
hash-free arithmetic on (seed, layer, component), so any subset of layers
can be regenerated independently.
"""
from __future__ import annotations

import numpy as np
import torch

SPECIAL_BF16 = {          # bit patterns injected into stress segments
    "nan": 0x7FC0, "+inf": 0x7F80, "-inf": 0xFF80,
    "+450": 0x43E1, "-450": 0xC3E1, "+1000": 0x447A, "-1000": 0xC47A,
}
EDGE_448 = (0x43E0, 0xC3E0)   # +-448 exactly: in range for FP8


def _gen(device, seed, layer, comp):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) * 1_000_003 + layer * 7919 + comp * 104_729 + 17)
    return g


def _k_scale(gen, device, heads, dim, kind):
    if kind == "lognormal":
        return torch.exp(torch.randn((heads, dim), generator=gen, device=device))
    if kind == "outliers":
        m = torch.rand((heads, dim), generator=gen, device=device) < 0.02
        return torch.where(m, torch.full_like(m, 20.0, dtype=torch.float32),
                           torch.ones_like(m, dtype=torch.float32))
    return torch.ones((heads, dim), device=device)


def separate_kv(layers, num_blocks, tokens, heads, dim, dtype=torch.bfloat16, seed=0,
                device="cuda", k_kind="lognormal"):
    """Per-layer K and V tensors [num_blocks, tokens, heads, dim] (NHD)."""
    ks, vs = [], []
    for l in range(layers):
        g = _gen(device, seed, l, 0)
        sc = _k_scale(g, device, heads, dim, k_kind)
        k = torch.randn((num_blocks, tokens, heads, dim), generator=g, device=device)
        k.mul_(sc)
        ks.append(k.to(dtype))
        del k
        g = _gen(device, seed, l, 1)
        vs.append(torch.randn((num_blocks, tokens, heads, dim), generator=g, device=device).to(dtype))
    return ks, vs


def packed_kv(layers, num_blocks, heads, tokens, dim, dtype=torch.float16, seed=0, device="cuda",
              k_kind="lognormal"):
    """Per-layer vLLM packed tensors [num_blocks, heads, tokens, 2*dim] (K then V)."""
    out = []
    for l in range(layers):
        t = torch.empty((num_blocks, heads, tokens, 2 * dim), dtype=dtype, device=device)
        g = _gen(device, seed, l, 0)
        sc = _k_scale(g, device, heads, dim, k_kind)
        k = torch.randn((num_blocks, heads, tokens, dim), generator=g, device=device)
        k.mul_(sc[None, :, None, :])
        t[..., :dim] = k.to(dtype)
        del k
        g = _gen(device, seed, l, 1)
        t[..., dim:] = torch.randn((num_blocks, heads, tokens, dim), generator=g, device=device).to(dtype)
        out.append(t)
    return out


def random_page_ids(pool, n, seed=0):
    """n distinct block ids out of [0, pool), sampled without replacement."""
    rng = np.random.default_rng(seed)
    return rng.choice(pool, size=n, replace=False).astype(np.int32)


def permutation(n, seed=0):
    return np.random.default_rng(seed + 1).permutation(n).astype(np.int32)


def inject_specials(k_layers, v_layers, page_ids, frac=0.01, seed=0, controls=64):
    """Plant one special value (NaN, +-Inf, +-450, +-1000) in a `frac` share
    of the (layer, page, component) segments, and +-448 exactly in `controls`
    other segments.  Returns (injected, control) as sets of (layer, page
    index, component) and the kind injected per segment."""
    rng = np.random.default_rng(seed + 2)
    layers = len(k_layers)
    n_pages = len(page_ids)
    nseg = layers * n_pages * 2
    count = max(1, int(round(frac * nseg)))
    picks = rng.choice(nseg, size=count + controls, replace=False)
    kinds = list(SPECIAL_BF16)
    injected, control, kind_of = set(), set(), {}
    t0 = k_layers[0]
    _, T, H, D = t0.shape
    for n, s in enumerate(picks):
        l, rem = divmod(int(s), 2 * n_pages)
        i, c = divmod(rem, 2)
        tensor = (k_layers if c == 0 else v_layers)[l]
        t, h, d = int(rng.integers(T)), int(rng.integers(H)), int(rng.integers(D))
        if n < count:
            kind = kinds[int(rng.integers(len(kinds)))]
            bits = SPECIAL_BF16[kind]
            injected.add((l, i, c))
            kind_of[(l, i, c)] = kind
        else:
            bits = EDGE_448[int(rng.integers(2))]
            control.add((l, i, c))
        tensor.view(torch.int16)[int(page_ids[i]), t, h, d] = bits - 65536 if bits >= 32768 else bits
    return injected, control, kind_of


# ------------------------------------------------------------------ workloads
CONFIGS = {
    "fp8_dynamic_small": dict(layers=2, heads=8, dim=128, dtype="bf16", layout="separate", tokens=16,
                              pool=64, pages=64, k="FP8_DYNAMIC", v="FP8_DYNAMIC"),
    "k16v8_packed": dict(layers=36, heads=8, dim=128, dtype="fp16", layout="packed", tokens=16,
                         pool=2048, pages=2048, k="RAW", v="FP8_FIXED"),
    "tq4_u4_llama3": dict(layers=32, heads=8, dim=128, dtype="bf16", layout="separate", tokens=16,
                          pool=8192, pages=4096, k="TQ4", v="UNIFORM4", protected=(0, 1, 30, 31),
                          random_pages=True),
    "tq3_u3_dsweep": dict(layers=28, heads=4, dims=(32, 64, 256), dtype="bf16", layout="separate",
                          tokens=16, pool=2048, pages=2048, k="TQ3", v="UNIFORM3", k_kind="outliers"),
    "int8_fp8_stress": dict(layers=32, heads=8, dim=128, dtype="bf16", layout="separate", tokens=16,
                            pool=8192, pages=8192, k="INT8", v="INT8", inject=0.01),
    # the INT8 host-pool record on the Qwen3-8B shape: 3392 pages = 54,272
    # tokens, about the 54,254 BF16 tokens an 8 GB host budget holds
    "int8_records_qwen3": dict(layers=36, heads=8, dim=128, dtype="bf16", layout="separate", tokens=16,
                               pool=4096, pages=3392, k="INT8_ROWS", v="INT8_ROWS", random_pages=True),
    # one tensor-parallel shard (8-way) of tq4_u4_llama3: one KV head per GPU,
    # 4 KiB segments
    "tq4_u4_llama3_tp8": dict(layers=32, heads=1, dim=128, dtype="bf16", layout="separate", tokens=16,
                              pool=8192, pages=4096, k="TQ4", v="UNIFORM4", protected=(0, 1, 30, 31),
                              random_pages=True),
    # the lossless entropy stage on the Llama-3-8B shape
    "ans16_llama3": dict(layers=32, heads=8, dim=128, dtype="bf16", layout="separate", tokens=16,
                         pool=8192, pages=4096, k="ANS16", v="ANS16", random_pages=True),
    # K8/V8 with per-token/head scales on the vLLM packed Qwen3-8B layout
    "k8v8_packed": dict(layers=36, heads=8, dim=128, dtype="fp16", layout="packed", tokens=16,
                        pool=2048, pages=2048, k="FP8_DYNAMIC", v="FP8_DYNAMIC"),
}


def torch_dtype(name):
    return torch.bfloat16 if name == "bf16" else torch.float16
