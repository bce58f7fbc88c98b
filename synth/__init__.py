"""Seeded synthetic inputs for per-head causal local-window attention.

This module is shared by the fp64 oracle's tests and by the HIP path's tests
and benchmark.  It draws random numbers and assembles window vectors; it holds
none of the attention arithmetic (no scores, masks, softmax or products).

Workloads follow the pages' 4096-token bf16 setting (Asymmetric Attention
Heads, Table 2: precision bf16, batch size 1, context 4096, candidate windows
[512, 1024, 2048, 4096]).  The pages train on an unnamed dataset with trained
weights; N(0, 1) activations stand in for the projected Q/K/V.  The
streaming-head workload follows "Autonomy-of-Heads" (section 5: retrieval
heads keep full attention, streaming heads keep sink + recent-window caches;
section 6.1: 128 sinks and a recent window of 256; section 6.4: sparsity
around 0.5) on the same 1B-scale layer shape.  The grouped-query workload has
32 query heads over 8 key/value heads (the Qwen3 grouping "Autonomy-of-Heads"
section 6.1 lists; AAH appendix A.3 transfers the method to a pretrained Qwen3
model at context 4096 in bf16), head dimension 128, and per-query-head windows
drawn like the 1B-scale groups.

Recipe (fixed, so every consumer sees identical bits):
  * ``numpy.random.default_rng(seed)``; fp32 standard normals drawn in the
    order Q, K, V, dO (dO is drawn for every bf16 workload so the window draw
    that follows is the same with or without a backward pass), then windows.
  * bf16 workloads round each fp32 draw once to bf16, round-to-nearest-even.
    The returned float32 arrays hold exactly the bf16 values; ``*_bits`` hold
    the raw uint16 patterns handed to the device.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional

import numpy as np

CANDIDATE_WINDOWS = (512, 1024, 2048, 4096)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (round-to-nearest-even) and return uint16 bit patterns.

    Inputs here are finite normals; NaN/inf handling is not needed."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = (u + 0x7FFF + lsb) >> 16
    return r.astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


@dataclasses.dataclass
class Workload:
    name: str
    B: int
    H: int
    T: int
    d: int
    dtype: str                      # "bf16" or "f32"
    windows: np.ndarray             # int32 [H]
    scale: float
    q: np.ndarray                   # float32 [B,H,T,d] (bf16-exact when dtype == "bf16")
    k: np.ndarray
    v: np.ndarray
    do: Optional[np.ndarray] = None
    bits: Dict[str, np.ndarray] = dataclasses.field(default_factory=dict)  # uint16 for bf16
    backward: bool = False
    meta: Dict[str, object] = dataclasses.field(default_factory=dict)
    sinks: Optional[np.ndarray] = None  # int32 [H] sink sizes, or None


def _draw(rng: np.random.Generator, shape, dtype: str):
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if dtype == "bf16":
        b = bf16_bits(x)
        return bf16_to_f32(b), b
    return x, None


def random_workload(B: int, H: int, T: int, d: int, windows, dtype: str = "bf16",
                    seed: int = 0, backward: bool = True, name: str = "random",
                    value_scale: float = 1.0, sinks=None, H_kv: Optional[int] = None) -> Workload:
    """Q, K, V (and dO) ~ N(0, 1) * value_scale for an arbitrary shape and window vector;
    K and V have H_kv heads (default H)."""
    rng = np.random.default_rng(seed)
    H_kv = H if H_kv is None else H_kv
    out = {}
    bits = {}
    for key in ("q", "k", "v", "do"):
        shape = (B, H_kv if key in ("k", "v") else H, T, d)
        x = rng.standard_normal(size=shape, dtype=np.float32)
        if value_scale != 1.0:
            x = (x * np.float32(value_scale)).astype(np.float32)
        if dtype == "bf16":
            b = bf16_bits(x)
            bits[key] = b
            x = bf16_to_f32(b)
        out[key] = x
    return Workload(name=name, B=B, H=H, T=T, d=d, dtype=dtype,
                    windows=np.asarray(windows, dtype=np.int32), scale=1.0 / np.sqrt(d),
                    q=out["q"], k=out["k"], v=out["v"], do=out["do"] if backward else None,
                    bits=bits, backward=backward,
                    sinks=None if sinks is None else np.asarray(sinks, dtype=np.int32))


def _hierarchy_from_groups(group_windows: np.ndarray) -> List[List[int]]:
    """Binary hierarchy over level-0 groups whose parent window is the larger of
    its two children, so every child window is <= its parent's (the pages'
    parent constraint, Asymmetric Attention Heads section 5.7)."""
    levels = [list(int(x) for x in group_windows)]
    while len(levels[-1]) > 1:
        cur = levels[-1]
        levels.append([max(cur[2 * i], cur[2 * i + 1]) for i in range(len(cur) // 2)])
    return levels


# Workload catalogue.  Index 0 is the small fp32 case the oracle finishes at once;
# 1 and 2 are the single-layer and 1B-scale forward workloads; 3 is workload 2 with
# a backward pass; "4a"/"4b"/"4c" are the coverage controls.
DESCRIPTIONS = {
    0: "tiny fp32 check: B=1 H=4 T=256 d=32, windows [16,32,64,256]",
    1: "single layer fwd: B=1 H=16 T=4096 d=64 bf16, windows uniform over {512..4096}",
    2: "1B-scale layer fwd: B=4 H=32 T=4096 d=64 bf16, 8 groups x 4 heads, P=(.5,.25,.125,.125)",
    3: "1B-scale layer fwd+bwd: workload 2 shapes and windows with dO",
    "4a": "coverage control fwd+bwd: B=4 H=32 T=4096 d=64 bf16, all windows 4096",
    "4b": "coverage control fwd+bwd: B=4 H=32 T=4096 d=64 bf16, all windows 512",
    "4c": "coverage control fwd+bwd: B=4 H=32 T=4096 d=64 bf16, even heads 512, odd heads 4096",
    5: "streaming heads fwd+bwd: B=4 H=32 T=4096 d=64 bf16, heads 0-15 full causal (4096), "
       "heads 16-31 sink 128 + recent window 256",
    6: "grouped-query layer fwd+bwd: B=4 H=32 H_kv=8 T=4096 d=128 bf16, "
       "per-query-head windows from {512..4096}, P=(.5,.25,.125,.125)",
    "5s": "the streaming-head layer of workload 5 for one sequence (B=1): its full-causal heads' long items "
          "exceed a workgroup's share of each launch, so the launches split",
    "6s": "the grouped-query layer for one sequence (B=1) with workload 6's windows: its dK/dV kernel has 256 "
          "grouped work items for 512 resident workgroups and takes its split launch",
}

# Workload 6's per-query-head windows (its seed-0 draw, which follows the draw of its tensors).
GQA_WINDOWS = (512, 2048, 512, 512, 1024, 4096, 1024, 512, 1024, 512, 2048, 512, 2048, 4096, 1024, 512,
               1024, 512, 2048, 1024, 1024, 2048, 512, 512, 512, 512, 4096, 1024, 4096, 1024, 512, 512)


def make_workload(idx, seed: int = 0) -> Workload:
    """Build one catalogued workload (see DESCRIPTIONS)."""
    if idx == 0:
        rng = np.random.default_rng(seed)
        shape = (1, 4, 256, 32)
        q = rng.standard_normal(size=shape, dtype=np.float32)
        k = rng.standard_normal(size=shape, dtype=np.float32)
        v = rng.standard_normal(size=shape, dtype=np.float32)
        return Workload(name="tiny-fp32", B=1, H=4, T=256, d=32, dtype="f32",
                        windows=np.array([16, 32, 64, 256], dtype=np.int32),
                        scale=1.0 / np.sqrt(32), q=q, k=k, v=v, backward=False)

    if idx in (1, 2, 3, "4a", "4b", "4c", 5, "5s"):
        if idx == 1:
            B, H = 1, 16
        elif idx == "5s":
            B, H = 1, 32
        else:
            B, H = 4, 32
        T, d = 4096, 64
        rng = np.random.default_rng(seed)
        shape = (B, H, T, d)
        arrs, bits = {}, {}
        for key in ("q", "k", "v", "do"):
            arrs[key], bits[key] = _draw(rng, shape, "bf16")
        meta: Dict[str, object] = {}
        if idx == 1:
            windows = rng.choice(np.array(CANDIDATE_WINDOWS), size=H).astype(np.int32)
            name = "single-layer-B1-H16-T4096-d64"
        elif idx in (2, 3):
            groups = rng.choice(np.array(CANDIDATE_WINDOWS), size=8,
                                p=[0.5, 0.25, 0.125, 0.125]).astype(np.int32)
            meta["group_windows"] = groups.tolist()
            meta["hierarchy"] = _hierarchy_from_groups(groups)
            windows = np.repeat(groups, H // 8).astype(np.int32)   # head h -> group h // 4
            name = "1b-layer-B4-H32-T4096-d64" + ("-fwdbwd" if idx == 3 else "")
        elif idx == "4a":
            windows = np.full(H, 4096, dtype=np.int32)
            name = "control-all4096"
        elif idx == "4b":
            windows = np.full(H, 512, dtype=np.int32)
            name = "control-all512"
        elif idx == "4c":
            windows = np.where(np.arange(H) % 2 == 0, 512, 4096).astype(np.int32)
            name = "control-interleaved-512-4096"
        else:
            # Retrieval heads first, then streaming heads (the reordered layout of
            # "Autonomy-of-Heads" section 5), half of each at sparsity 0.5 (section 6.4).
            windows = np.where(np.arange(H) < H // 2, T, 256).astype(np.int32)
            meta["sinks"] = np.where(np.arange(H) < H // 2, 0, 128).astype(np.int32)
            name = f"streaming-B{B}-H32-T4096-d64-sink128-recent256"
        backward = idx != 1 and idx != 2
        sinks = meta.pop("sinks", None)
        return Workload(name=name, B=B, H=H, T=T, d=d, dtype="bf16", windows=windows,
                        scale=1.0 / np.sqrt(d), q=arrs["q"], k=arrs["k"], v=arrs["v"],
                        do=arrs["do"] if backward else None, bits=bits, backward=backward,
                        meta=meta, sinks=sinks)
    if idx == 6:
        B, H, H_kv, T, d = 4, 32, 8, 4096, 128
        rng = np.random.default_rng(seed)
        arrs, bits = {}, {}
        for key in ("q", "k", "v", "do"):
            arrs[key], bits[key] = _draw(rng, (B, H_kv if key in ("k", "v") else H, T, d), "bf16")
        windows = rng.choice(np.array(CANDIDATE_WINDOWS), size=H, p=[0.5, 0.25, 0.125, 0.125]).astype(np.int32)
        return Workload(name="gqa-B4-H32-Hkv8-T4096-d128-fwdbwd", B=B, H=H, T=T, d=d, dtype="bf16",
                        windows=windows, scale=1.0 / np.sqrt(d), q=arrs["q"], k=arrs["k"], v=arrs["v"],
                        do=arrs["do"], bits=bits, backward=True, meta={"H_kv": H_kv})
    if idx == "6s":
        B, H, H_kv, T, d = 1, 32, 8, 4096, 128
        rng = np.random.default_rng(seed)
        arrs, bits = {}, {}
        for key in ("q", "k", "v", "do"):
            arrs[key], bits[key] = _draw(rng, (B, H_kv if key in ("k", "v") else H, T, d), "bf16")
        return Workload(name="gqa-B1-H32-Hkv8-T4096-d128-fwdbwd", B=B, H=H, T=T, d=d, dtype="bf16",
                        windows=np.array(GQA_WINDOWS, dtype=np.int32), scale=1.0 / np.sqrt(d), q=arrs["q"],
                        k=arrs["k"], v=arrs["v"], do=arrs["do"], bits=bits, backward=True, meta={"H_kv": H_kv})
    raise KeyError(f"unknown workload {idx!r}")
