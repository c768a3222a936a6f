"""Seeded synthetic inputs and the named workloads.

This module only draws random numbers and describes shapes; it holds none of
the attention or mask-compilation arithmetic.  Both the GPU path's tests and
the CPU oracle receive their inputs from here, so the two sides see the same
bits.

Recipe: numpy.random.default_rng(seed); draw q, then k, then v as float32
standard normals of shapes [B, Hq, Sq, D], [B, Hkv, Skv, D], [B, Hkv, Skv, Dv];
round once to bfloat16 (round-to-nearest-even, via torch) unless the workload
is float32.  A dense random mask is drawn after v as rng.random((Sq, Skv)) <
p_keep, with the diagonal then forced on, shared by all heads (Hm = 1).
"""
from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch


@dataclass(frozen=True)
class MaskSpec:
    kind: str                       # "causal" | "local" | "chunked" | "dense"
    left: Optional[int] = None      # local: left window (None = unbounded)
    right: Optional[int] = None     # local: right window (None = unbounded)
    chunk: Optional[int] = None     # chunked: chunk length
    dense_p: Optional[float] = None  # dense random: probability of keep
    dense_heads: int = 1            # dense random: Hm
    empty_every: Optional[int] = None   # dense random: every n-th query row allows no key


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    Sq: int
    Skv: int
    D: int
    Dv: int
    dtype: str                      # "bf16" | "f32"
    mask: MaskSpec
    soft_cap: Optional[float] = None
    block: int = 128
    seed: int = 0
    growing: Optional[float] = None   # see make_inputs: logits growing along the keys

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32


# The five workloads the method is measured on (block 128 x 128 everywhere).
WORKLOADS = {
    "tiny_causal_f32": Workload("tiny_causal_f32", 1, 2, 2, 512, 512, 64, 64, "f32",
                                MaskSpec("causal"), seed=1),
    "causal_mha_8k": Workload("causal_mha_8k", 1, 16, 16, 8192, 8192, 128, 128, "bf16",
                              MaskSpec("causal"), seed=2),
    "local_gqa_8k": Workload("local_gqa_8k", 1, 32, 8, 8192, 8192, 128, 128, "bf16",
                             MaskSpec("local", left=1024, right=0), seed=3),
    "chunked_gqa_16k_cap": Workload("chunked_gqa_16k_cap", 2, 16, 4, 16384, 16384, 128, 128, "bf16",
                                    MaskSpec("chunked", chunk=2048), soft_cap=30.0, seed=4),
    "random_dense_2k": Workload("random_dense_2k", 1, 8, 8, 2048, 2048, 128, 128, "bf16",
                                MaskSpec("dense", dense_p=0.1), seed=5),
}
WORKLOAD_ORDER = ["tiny_causal_f32", "causal_mha_8k", "local_gqa_8k",
                  "chunked_gqa_16k_cap", "random_dense_2k"]

# A stress input for the kernel's softmax rather than a measured workload:
# the causal 8k shape with every row's logits growing along the keys (from
# about 0 to about 74 at the diagonal), so an exponent base fixed early in a
# row falls far below the row's final max.
WORKLOADS["causal_growing_8k"] = Workload("causal_growing_8k", 1, 16, 16, 8192, 8192, 128, 128, "bf16",
                                          MaskSpec("causal"), seed=7, growing=29.0)

# The random dense workload with every 16th query row allowing no key (as
# padding or document masks produce): such rows must cost nothing extra.
WORKLOADS["dense_empty_rows_2k"] = Workload("dense_empty_rows_2k", 1, 8, 8, 2048, 2048, 128, 128, "bf16",
                                            MaskSpec("dense", dense_p=0.1, empty_every=16), seed=8)

# The causal 8k shape at head dims the forward runs zero-padded (D = Dv = 96
# inside the 128-column kernel): what a head dim off the kernel's own costs.
WORKLOADS["causal_d96_8k"] = Workload("causal_d96_8k", 1, 16, 16, 8192, 8192, 96, 96, "bf16",
                                      MaskSpec("causal"), seed=9)


# Decode (one query per head against a key/value cache, every key allowed):
# a GQA serving shape, measured against HBM bandwidth.
DECODE_WORKLOADS = {
    "decode_gqa_32k": Workload("decode_gqa_32k", 8, 32, 8, 1, 32768, 128, 128, "bf16",
                               MaskSpec("dense"), seed=6),
    # the same cache at a head dim the decode runs zero-padded (96 of 128 columns)
    "decode_gqa_32k_d96": Workload("decode_gqa_32k_d96", 8, 32, 8, 1, 32768, 96, 96, "bf16",
                                   MaskSpec("dense"), seed=10),
}


def random_dense_mask(rng, heads, q_len, kv_len, p_keep, force_diagonal=True):
    """Bernoulli(p_keep) bool mask [heads, q_len, kv_len]; diagonal forced on."""
    m = rng.random((heads, q_len, kv_len)) < p_keep
    if force_diagonal:
        n = min(q_len, kv_len)
        m[:, np.arange(n), np.arange(n)] = True
    return m


def make_inputs(w: Workload):
    """q, k, v as CPU torch tensors in the workload dtype, plus the dense mask
    ([Hm, Sq, Skv] bool numpy array) for dense workloads, else None."""
    rng = np.random.default_rng(w.seed)
    q = rng.standard_normal((w.B, w.Hq, w.Sq, w.D), dtype=np.float32)
    k = rng.standard_normal((w.B, w.Hkv, w.Skv, w.D), dtype=np.float32)
    v = rng.standard_normal((w.B, w.Hkv, w.Skv, w.Dv), dtype=np.float32)
    dense = None
    if w.mask.kind == "dense":
        if w.mask.dense_heads == 1:
            m = rng.random((w.Sq, w.Skv)) < w.mask.dense_p
            n = min(w.Sq, w.Skv)
            m[np.arange(n), np.arange(n)] = True
            if w.mask.empty_every:
                m[::w.mask.empty_every] = False
            dense = m[None]
        else:
            dense = random_dense_mask(rng, w.mask.dense_heads, w.Sq, w.Skv, w.mask.dense_p)
    if w.growing is not None:
        # q_i = a e0 + 0.05 noise, k_j = a (j / Skv) e0 + 0.05 noise: logits
        # of row i grow along the keys up to about a^2 i / Skv / sqrt(D)
        t = (np.arange(w.Skv, dtype=np.float32) / w.Skv)[:, None]
        q = 0.05 * q
        k = 0.05 * k
        q[..., 0] += w.growing
        k[..., 0] += w.growing * t[:, 0]
    td = w.torch_dtype
    return (torch.from_numpy(q).to(td), torch.from_numpy(k).to(td),
            torch.from_numpy(v).to(td), dense)


def make_qkv(seed, B, Hq, Hkv, Sq, Skv, D, Dv, dtype=torch.bfloat16, scale=1.0):
    """Generic seeded q, k, v (CPU torch tensors) for parity cases."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, Sq, D), dtype=np.float32) * scale
    k = rng.standard_normal((B, Hkv, Skv, D), dtype=np.float32) * scale
    v = rng.standard_normal((B, Hkv, Skv, Dv), dtype=np.float32)
    return (torch.from_numpy(q).to(dtype), torch.from_numpy(k).to(dtype),
            torch.from_numpy(v).to(dtype))
