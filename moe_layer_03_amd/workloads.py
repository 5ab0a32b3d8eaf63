"""Named workloads and the seeded synthetic input generator.

This module draws random numbers and rounds them to the storage dtype; it
holds none of the layer's arithmetic (no routing, no expert FFN, no combine),
so both the HIP path and the oracle may be fed from it.

Workloads follow the shape of the layer in "Hosting Qwen on Blackwell"
(Perplexity): 128 experts, 8 routed experts per token, about 6000-token
prefill inputs (section "Pre-remplisseurs"), expert-parallel ranks that own a
contiguous range of experts (section "Expert Parallel"), decode shards of a
16-way expert split (section "MoE GEMM").  Hidden size 4096, expert
intermediate size 1536 and SwiGLU experts are the Qwen3-235B shapes this
library targets; the pages do not print them.

Recipe (all draws are float32 standard normals from numpy's PCG64):

* stream ``[seed, 0]``   -> x [T, H]                    (std 1)
* stream ``[seed, 1]``   -> router weight [H, E]        (std 0.02)
* stream ``[seed, 2]``   -> permutation of the E experts (skewed workload only)
* stream ``[seed, 100+e]`` -> expert e: gate [H, I], up [H, I], down [I, H],
  drawn in that order (std 0.02).

A draw is multiplied by its std in float32, then rounded to bfloat16 with
round-to-nearest-even (the tiny workload keeps float32).  Because every
expert has its own stream, expert e is the same tensor in every workload that
shares (H, I, seed): the four 32-expert shards of the whole layer see exactly
the whole layer's experts.

The skewed workload adds a per-expert router bias ``b[e] = -s * ln(r_e)``
(computed in float64, stored float32), where ``r_e`` is one plus the position
of e in the seeded permutation: the logarithm of a Zipf(s) law over a random
ranking of the experts, without its normalising constant (a constant shift of
all logits changes neither the selection nor the weights).
"""
from __future__ import annotations

import dataclasses
import math
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, Optional, Sequence, Tuple

import numpy as np

STD_X = np.float32(1.0)
STD_W = np.float32(0.02)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int              # tokens
    H: int              # hidden size
    E: int              # experts in the layer
    K: int              # routed experts per token
    I: int              # expert intermediate size
    e_begin: int        # first local expert
    e_end: int          # one past the last local expert
    dtype: str          # storage dtype of x and of every weight: "f32" or "bf16"
    zipf_s: Optional[float] = None   # router-bias skew (None: no bias)
    seed: int = 0

    @property
    def E_loc(self) -> int:
        return self.e_end - self.e_begin

    @property
    def cap(self) -> int:
        """Upper bound on routed (token, slot) pairs that can land locally."""
        return self.T * min(self.K, self.E_loc)

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    def describe(self) -> Dict:
        d = dataclasses.asdict(self)
        d["workload"] = d.pop("name")
        return d


WORKLOADS: Dict[str, Workload] = {
    # T=64, hidden 256, 8 experts, top-2, intermediate 128, all experts local, float32.
    "tiny": Workload("tiny", T=64, H=256, E=8, K=2, I=128, e_begin=0, e_end=8, dtype="f32"),
    # One rank of a 4-way expert split during prefill: experts 0..31 of 128.
    "prefill_ep4_shard": Workload("prefill_ep4_shard", T=6000, H=4096, E=128, K=8, I=1536,
                                  e_begin=0, e_end=32, dtype="bf16"),
    # One rank of a 16-way expert split during decode: experts 0..7 of 128.
    "decode_ep16_shard": Workload("decode_ep16_shard", T=128, H=4096, E=128, K=8, I=1536,
                                  e_begin=0, e_end=8, dtype="bf16"),
    # Prefill with Zipf(1.1)-skewed router logits, experts 0..31 local.
    "skewed_prefill": Workload("skewed_prefill", T=16384, H=4096, E=128, K=8, I=1536,
                               e_begin=0, e_end=32, dtype="bf16", zipf_s=1.1),
    # The whole layer on one device: all 128 experts local.
    "whole_layer": Workload("whole_layer", T=6000, H=4096, E=128, K=8, I=1536,
                            e_begin=0, e_end=128, dtype="bf16"),
}

# Order in which the workloads are listed (tiny first; the 6000-token shard is
# the headline throughput workload).
WORKLOAD_ORDER = ["tiny", "prefill_ep4_shard", "decode_ep16_shard", "skewed_prefill", "whole_layer"]


# ---------------------------------------------------------------------------
# bfloat16 storage helpers (storage conversion only)
# ---------------------------------------------------------------------------

def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return the raw uint16 bits.

    Inputs are finite by construction (normal draws), so NaN handling is not needed."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    rounding = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + rounding) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen raw bfloat16 bits to float32 (exact)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _store(a32: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.ascontiguousarray(a32, dtype=np.float32)
    if dtype == "bf16":
        return f32_to_bf16_bits(a32)
    raise ValueError(f"unknown dtype {dtype!r}")


def as_f32(a: np.ndarray) -> np.ndarray:
    """Float32 view of a stored tensor (bf16 bits are widened exactly)."""
    if a.dtype == np.uint16:
        return bf16_bits_to_f32(a)
    return np.asarray(a, dtype=np.float32)


def _normal(seed: int, stream: int, shape: Tuple[int, ...], std: np.float32) -> np.ndarray:
    rng = np.random.default_rng([seed, stream])
    a = rng.standard_normal(shape, dtype=np.float32)
    if std != np.float32(1.0):
        a *= std
    return a


def _threads() -> int:
    n = os.cpu_count() or 1
    try:
        n = min(n, int(os.environ.get("OMP_NUM_THREADS", n)))
    except ValueError:
        pass
    return max(1, min(16, n))


# ---------------------------------------------------------------------------
# generators
# ---------------------------------------------------------------------------

def gen_x(wl: Workload) -> np.ndarray:
    """Activations [T, H] in the workload's storage dtype."""
    return _store(_normal(wl.seed, 0, (wl.T, wl.H), STD_X), wl.dtype)


def gen_router(wl: Workload) -> np.ndarray:
    """Router weight [H, E] in the workload's storage dtype (logits = x @ W)."""
    return _store(_normal(wl.seed, 1, (wl.H, wl.E), STD_W), wl.dtype)


def zipf_ranks(wl: Workload) -> np.ndarray:
    """r_e = 1 + position of expert e in the seeded permutation (int64 [E])."""
    perm = np.random.default_rng([wl.seed, 2]).permutation(wl.E)
    ranks = np.empty(wl.E, dtype=np.int64)
    ranks[perm] = np.arange(1, wl.E + 1, dtype=np.int64)
    return ranks


def gen_bias(wl: Workload) -> Optional[np.ndarray]:
    """Router bias [E] float32, or None for workloads without skew."""
    if wl.zipf_s is None:
        return None
    r = zipf_ranks(wl)
    return np.array([-wl.zipf_s * math.log(float(v)) for v in r], dtype=np.float64).astype(np.float32)


def gen_expert(wl: Workload, e: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """(gate [H, I], up [H, I], down [I, H]) of expert e, storage dtype."""
    rng = np.random.default_rng([wl.seed, 100 + e])
    out = []
    for shape in ((wl.H, wl.I), (wl.H, wl.I), (wl.I, wl.H)):
        a = rng.standard_normal(shape, dtype=np.float32)
        a *= STD_W
        out.append(_store(a, wl.dtype))
    return out[0], out[1], out[2]


def gen_experts(wl: Workload, experts: Optional[Sequence[int]] = None):
    """Stacked (gate [n,H,I], up [n,H,I], down [n,I,H]) for the given experts
    (default: the local range), generated in parallel threads."""
    if experts is None:
        experts = range(wl.e_begin, wl.e_end)
    experts = list(experts)
    np_dtype = np.float32 if wl.dtype == "f32" else np.uint16
    n = len(experts)
    g = np.empty((n, wl.H, wl.I), dtype=np_dtype)
    u = np.empty((n, wl.H, wl.I), dtype=np_dtype)
    d = np.empty((n, wl.I, wl.H), dtype=np_dtype)

    def fill(i):
        g[i], u[i], d[i] = gen_expert(wl, experts[i])

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(fill, range(n)))
    return g, u, d


@dataclasses.dataclass
class Inputs:
    wl: Workload
    x: np.ndarray                 # [T, H] storage dtype
    w_router: np.ndarray          # [H, E] storage dtype
    bias: Optional[np.ndarray]    # [E] float32 or None
    w_gate: np.ndarray            # [E_loc, H, I] storage dtype
    w_up: np.ndarray              # [E_loc, H, I] storage dtype
    w_down: np.ndarray            # [E_loc, I, H] storage dtype


def make_inputs(wl: Workload) -> Inputs:
    g, u, d = gen_experts(wl)
    return Inputs(wl, gen_x(wl), gen_router(wl), gen_bias(wl), g, u, d)


def flops_per_pair(wl: Workload) -> int:
    """Multiply-add FLOPs of one expert FFN evaluation (gate/up + down)."""
    return 2 * wl.H * 2 * wl.I + 2 * wl.I * wl.H


def router_flops(wl: Workload) -> int:
    return 2 * wl.T * wl.H * wl.E


def expert_weight_bytes(wl: Workload) -> int:
    """Bytes of one expert's three matrices in the storage dtype."""
    return (2 if wl.dtype == "bf16" else 4) * 3 * wl.H * wl.I
