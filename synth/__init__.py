"""Seeded synthetic inputs for the beam-search decode step.

This module is shared test and benchmark infrastructure. It draws random
numbers and lays them out as the workloads' logits, proposals and KV-cache
contents; it holds none of the beam step's own arithmetic (no softmax, no
selection, no argmax, no length penalty).

Random numbers come from one counter-based generator so that any element can
be produced on its own, in any order:

* SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
  generators", OOPSLA 2014; the 64-bit finaliser constants as published by
  Vigna) mixes a 64-bit counter into a 64-bit word.
* A row's base word chains the mix over (seed, stream, step, row); element
  ``col`` then takes two words ``mix(base ^ 2*col)`` and ``mix(base ^ 2*col+1)``
  and turns them into two 53-bit uniforms.
* Box and Muller ("A note on the generation of random normal deviates",
  Ann. Math. Stat. 1958) turns the pair into one standard normal, in double.

Logits are formed in double (``sigma * z + bias``) and rounded to fp32 with
round-to-nearest-even; bf16 logits are that fp32 value rounded again to bf16
with round-to-nearest-even, stored as raw uint16 bit patterns.

The Zipf token bias of exponent ``s`` is the log of an unnormalised Zipf pmf
with rank ``v + 1``: ``bias_v = -s * ln(v + 1)``. A constant normaliser would
cancel in any per-row log-softmax, so it is left out.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

_M64 = np.uint64(0xFFFFFFFFFFFFFFFF)
_GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_C1 = np.uint64(0xBF58476D1CE4E5B9)
_C2 = np.uint64(0x94D049BB133111EB)

# stream tags keep the draws for different purposes independent
STREAM_LOGITS = 1
STREAM_PROPOSAL = 2
STREAM_PLANT = 3
STREAM_PREFIX = 4


def splitmix64(x):
    """SplitMix64 finaliser on uint64 scalars or arrays (wrapping arithmetic)."""
    x = np.asarray(x, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = x + _GOLDEN
        z = (z ^ (z >> np.uint64(30))) * _C1
        z = (z ^ (z >> np.uint64(27))) * _C2
        z = z ^ (z >> np.uint64(31))
    return z


def row_base(seed: int, stream: int, step: int, row: int) -> np.uint64:
    h = splitmix64(np.uint64(seed & 0xFFFFFFFFFFFFFFFF))
    h = splitmix64(h ^ np.uint64(stream))
    h = splitmix64(h ^ np.uint64(step & 0xFFFFFFFFFFFFFFFF))
    h = splitmix64(h ^ np.uint64(row & 0xFFFFFFFFFFFFFFFF))
    return h


def uniforms(base: np.uint64, cols: np.ndarray):
    """Two uniforms per column: u1 in (0, 1], u2 in [0, 1)."""
    c = np.asarray(cols, dtype=np.uint64) * np.uint64(2)
    a = splitmix64(np.uint64(base) ^ c)
    b = splitmix64(np.uint64(base) ^ (c + np.uint64(1)))
    scale = 1.0 / 9007199254740992.0  # 2**-53
    u1 = ((a >> np.uint64(11)).astype(np.float64) + 1.0) * scale
    u2 = (b >> np.uint64(11)).astype(np.float64) * scale
    return u1, u2


def normals(seed: int, stream: int, step: int, row: int, n: int,
            col0: int = 0) -> np.ndarray:
    """n standard normals (float64) for columns col0 .. col0+n-1 of one row."""
    u1, u2 = uniforms(row_base(seed, stream, step, row),
                      np.arange(col0, col0 + n, dtype=np.uint64))
    return np.sqrt(-2.0 * np.log(u1)) * np.cos(2.0 * math.pi * u2)


def uniform01(seed: int, stream: int, step: int, row: int, n: int) -> np.ndarray:
    """n uniforms in [0, 1) (float64) for one row."""
    _, u2 = uniforms(row_base(seed, stream, step, row),
                     np.arange(n, dtype=np.uint64))
    return u2


def f32_to_bf16_bits(x32: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (round to nearest, ties to even); raw uint16 bits.

    Infinities pass through; NaN is not produced by this module.
    """
    b = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32)
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    with np.errstate(over="ignore"):
        r = (b + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    inf_mask = (b & np.uint32(0x7FFFFFFF)) == np.uint32(0x7F800000)
    r = np.where(inf_mask, b >> np.uint32(16), r)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32)
            << np.uint32(16)).view(np.float32)


# ---------------------------------------------------------------------------
# workloads
# ---------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic beam-search workload (shapes, distributions, KV layout)."""
    name: str
    batch: int
    beam: int
    vocab: int
    max_steps: int
    eos_id: int            # < 0: no EOS token
    pad_id: int
    dtype: str             # "f32" | "bf16"
    sigma: float
    zipf_s: float          # 0: no Zipf bias
    eos_ramp: float        # EOS bias reaches this value at step ramp_steps (0: none)
    ramp_steps: int
    eos_start: float       # EOS bias at step 0 when it ramps
    eos_in_zipf: bool      # whether the EOS id also carries the Zipf term
    lp: str                # "none" | "gnmt" | "pow"
    alpha: float
    stop: str              # "true" | "heuristic" | "never"
    num_return: int
    layers: int
    kv_heads: int
    head_dim: int
    kv_dtype: str          # "f32" | "bf16"
    prompt_len: int        # shared prompt positions (never reordered)
    seed: int
    pool: int              # distinct logit buffers the benchmark rotates through

    @property
    def rows(self) -> int:
        return self.batch * self.beam

    @property
    def elem_bytes(self) -> int:
        return 2 if self.dtype == "bf16" else 4

    @property
    def kv_elem_bytes(self) -> int:
        return 2 if self.kv_dtype == "bf16" else 4

    @property
    def kv_bytes_per_pos(self) -> int:
        """Bytes of one position of one (layer, K|V) plane of one row."""
        return self.kv_heads * self.head_dim * self.kv_elem_bytes

    @property
    def kv_bytes_per_token(self) -> int:
        """K and V bytes of one token of one row over all layers."""
        return 2 * self.layers * self.kv_bytes_per_pos

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    # toy: B=3, W=2, V=6, EOS 5, fp32 N(0,1) per step, 10 steps, GNMT 0.6
    "toy": Workload("toy", 3, 2, 6, 10, 5, -1, "f32", 1.0, 0.0, 0.0, 1, 0.0, True,
                    "gnmt", 0.6, "heuristic", 1, 1, 2, 4, "f32", 0, 1001, 1),
    # Transformer-base MT shape
    "tbase": Workload("tbase", 32, 4, 32000, 128, 1, -1, "f32", 2.0, 1.1, 6.0,
                      100, -8.0, False, "gnmt", 0.6, "heuristic", 1, 6, 8, 64, "f32",
                      0, 1002, 128),
    # Llama-3-8B shape: bf16 logits, EOS = V-1 under the Zipf term
    "llama3_8b": Workload("llama3_8b", 8, 4, 128256, 200, 128255, -1, "bf16",
                          3.0, 1.0, 0.0, 1, 0.0, True, "pow", 1.0, "true", 1, 32,
                          8, 128, "bf16", 1000, 1003, 64),
    # wide-beam stress
    "wide": Workload("wide", 16, 16, 250000, 256, 249999, -1, "f32", 2.0, 1.2,
                     0.0, 1, 0.0, True, "gnmt", 0.7, "heuristic", 1, 6, 16, 64,
                     "f32", 0, 1005, 3),
}

# blockwise-parallel verify: B=64, k=8, V=32000, fp32 N(0,2), ~0.6 per position
VERIFY = dict(batch=64, k=8, vocab=32000, sigma=2.0, accept_p=0.6, plant=12.0,
              seed=1004, pool=8)


def token_bias(wl: Workload, step: int) -> np.ndarray:
    """Per-token additive bias (float64) of one step."""
    v = np.arange(wl.vocab, dtype=np.float64)
    bias = -wl.zipf_s * np.log1p(v) if wl.zipf_s else np.zeros(wl.vocab)
    if wl.eos_id >= 0 and not wl.eos_in_zipf:
        bias[wl.eos_id] = 0.0
    if wl.eos_id >= 0 and wl.eos_ramp:
        f = min(step, wl.ramp_steps) / wl.ramp_steps
        bias[wl.eos_id] += wl.eos_start + (wl.eos_ramp - wl.eos_start) * f
    return bias


def logits_f64(wl: Workload, step: int, rows: Optional[range] = None,
               seed: Optional[int] = None) -> np.ndarray:
    """Logits of one decode step (1-based) as float64 [rows, V]."""
    seed = wl.seed if seed is None else seed
    rows = range(wl.rows) if rows is None else rows
    bias = token_bias(wl, step)
    out = np.empty((len(rows), wl.vocab), dtype=np.float64)
    for i, r in enumerate(rows):
        out[i] = wl.sigma * normals(seed, STREAM_LOGITS, step, r, wl.vocab) + bias
    return out


def logits(wl: Workload, step: int, rows: Optional[range] = None,
           seed: Optional[int] = None) -> np.ndarray:
    """Logits of one step in the workload's storage type.

    fp32 workloads return float32 [rows, V]; bf16 workloads return the raw
    uint16 bit patterns [rows, V].
    """
    x32 = logits_f64(wl, step, rows, seed).astype(np.float32)
    if wl.dtype == "bf16":
        return f32_to_bf16_bits(x32)
    return x32


def widen(wl_dtype: str, arr: np.ndarray) -> np.ndarray:
    """Exact fp32 view of logits stored as fp32 or bf16 bits."""
    if wl_dtype == "bf16":
        return bf16_bits_to_f32(arr)
    return np.asarray(arr, dtype=np.float32)


def prefix_logits(seed: int, prefix, vocab: int, sigma: float = 1.0) -> np.ndarray:
    """fp32 logits of a toy "model" whose next-token scores depend only on the
    token prefix (used for exhaustive-search checks on tiny vocabularies)."""
    h = np.uint64(0x243F6A8885A308D3)
    for tok in prefix:
        h = splitmix64(h ^ np.uint64(int(tok) + 1))
    z = normals(seed, STREAM_PREFIX, 0, int(h), vocab)
    return (sigma * z).astype(np.float32)


def verify_inputs(batch: int, k: int, vocab: int, seed: int, sigma: float = 2.0,
                  accept_p: float = 0.6, plant: float = 12.0, call: int = 0):
    """Logits [B, k, V] fp32 and proposals [B, k] int32 for the verify step.

    Every proposal is a uniform random token. Position 0, and each later
    position with probability ``accept_p``, gets its proposal's logit set to
    ``plant`` (6 sigma above the noise at the default sigma), so that the base
    model's greedy choice there is, with overwhelming probability, the
    proposal. No argmax is taken here.
    """
    lg = np.empty((batch, k, vocab), dtype=np.float32)
    prop = np.empty((batch, k), dtype=np.int32)
    for b in range(batch):
        toks = uniform01(seed, STREAM_PROPOSAL, call, b, k)
        coin = uniform01(seed, STREAM_PLANT, call, b, k)
        for i in range(k):
            row = b * k + i
            lg[b, i] = (sigma * normals(seed, STREAM_LOGITS, call, row, vocab)
                        ).astype(np.float32)
            p = min(int(toks[i] * vocab), vocab - 1)
            prop[b, i] = p
            if i == 0 or coin[i] < accept_p:
                lg[b, i, p] = np.float32(plant)
    return lg, prop


def kv_fill_values(b: int, slot: int, pos: int, lk: int, n_words: int) -> np.ndarray:
    """Distinct 32-bit words for one (item, slot, position, layer*2+kv) KV
    vector, so that reordered rows can be told apart bit for bit."""
    base = row_base(0x4B56, (b << 16) | slot, pos, lk)
    return (splitmix64(base ^ np.arange(n_words, dtype=np.uint64))
            & np.uint64(0xFFFFFFFF)).astype(np.uint32)
