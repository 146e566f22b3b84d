"""Seeded synthetic workloads for the expert load-balancing path.

This module only draws inputs.  It holds none of the balancing arithmetic, so
both the HIP path and the CPU oracle may consume what it produces.

The pages measure on production training traces (UltraEP technical article,
section on Qwen3-235B results) and on MMLU/GPQA/GSM8K prompt pools (Waterfill
and LPLB blog, experiments section).  None of those is available, so routing is
drawn from a per-layer Zipf popularity over experts:

* a seeded permutation pi of the experts gives each expert a popularity rank;
* p_e is proportional to (pi(e) + 1) ** (-s);
* each token picks K distinct experts without replacement with probabilities
  proportional to p_e.  This is done with exponential races: the K experts with
  the smallest Exp(1) / p_e win, which is the same law as drawing one expert at
  a time without replacement (equivalently the Gumbel-top-K trick).

Seeds come from ``numpy.random.SeedSequence([config_id, layer, stream])``.
"""

from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

# stream ids inside a (config, layer) seed sequence
_STREAM_SKEW = 0
_STREAM_ROUTING = 1
_STREAM_PLACEMENT = 2
_STREAM_TENSORS = 3


@dataclasses.dataclass(frozen=True)
class Workload:
    """Geometry of one synthetic MoE layer (or a sweep of layers)."""

    name: str
    config_id: int
    R: int          # virtual EP ranks
    E: int          # logical routed experts
    S: int          # redundant slots per rank (UltraEP)
    T: int          # tokens per rank
    K: int          # routed experts per token
    H: int          # hidden size (bf16 activations)
    q_min: int      # minimum quota of a new replica
    zipf_s: Optional[float]  # fixed Zipf exponent, or None for the per-layer draw
    layers: int = 1
    ffn_shape: tuple = (3, 4096, 1536)   # expert weight block (bf16)
    n_static_replicas: int = 0            # LPLB: static redundant replicas
    shared_expert: bool = False           # Waterfill: one shared slot per token

    @property
    def E_loc(self) -> int:
        return self.E // self.R

    @property
    def N(self) -> int:
        return self.R * self.T

    @property
    def P(self) -> int:
        return self.R * self.T * self.K

    @property
    def expert_elems(self) -> int:
        return int(np.prod(self.ffn_shape))


TINY = Workload("tiny", 0, R=4, E=8, S=1, T=512, K=2, H=256, q_min=32, zipf_s=1.2,
                ffn_shape=(3, 64, 32))
QWEN_LAYER = Workload("qwen3_235b_layer", 1, R=32, E=128, S=1, T=8192, K=8, H=4096,
                      q_min=1024, zipf_s=None)
QWEN_SWEEP = Workload("qwen3_235b_94layer_sweep", 2, R=32, E=128, S=1, T=8192, K=8,
                      H=4096, q_min=1024, zipf_s=None, layers=94)
DSV3_WATERFILL = Workload("dsv3_waterfill", 3, R=64, E=256, S=0, T=4096, K=8, H=7168,
                          q_min=0, zipf_s=1.2, shared_expert=True)
LPLB_LAYER = Workload("lplb_layer", 4, R=64, E=256, S=1, T=16384, K=8, H=7168, q_min=0,
                      zipf_s=1.2, n_static_replicas=32)

ALL = {w.name: w for w in (TINY, QWEN_LAYER, QWEN_SWEEP, DSV3_WATERFILL, LPLB_LAYER)}


def scaled(w: Workload, **changes) -> Workload:
    """A copy of ``w`` with some fields changed (smaller parity cases)."""
    return dataclasses.replace(w, **changes)


def _seq(w: Workload, layer: int, stream: int) -> np.random.SeedSequence:
    return np.random.SeedSequence([w.config_id, layer, stream])


def zipf_exponent(w: Workload, layer: int) -> float:
    """Fixed exponent, or s = 0.8 + 0.6 * U for the per-layer skew."""
    if w.zipf_s is not None:
        return float(w.zipf_s)
    u = np.random.default_rng(_seq(w, layer, _STREAM_SKEW)).random()
    return 0.8 + 0.6 * float(u)


def expert_popularity(w: Workload, layer: int) -> np.ndarray:
    """p_e proportional to (pi(e)+1)^-s for a seeded permutation pi (float64, sums to 1)."""
    rng = np.random.default_rng(_seq(w, layer, _STREAM_SKEW))
    rng.random()  # the draw used by zipf_exponent
    pi = rng.permutation(w.E)
    s = zipf_exponent(w, layer)
    p = (pi.astype(np.float64) + 1.0) ** (-s)
    return p / p.sum()


def routing(w: Workload, layer: int = 0, chunk_tokens: int = 1 << 15) -> np.ndarray:
    """top-k expert ids, int32 [R][T][K], K distinct ids per token."""
    p = expert_popularity(w, layer).astype(np.float32)
    rng = np.random.default_rng(_seq(w, layer, _STREAM_ROUTING))
    n = w.R * w.T
    out = np.empty((n, w.K), dtype=np.int32)
    inv_p = (1.0 / p).astype(np.float32)
    for a in range(0, n, chunk_tokens):
        b = min(n, a + chunk_tokens)
        race = rng.standard_exponential((b - a, w.E), dtype=np.float32) * inv_p
        part = np.argpartition(race, w.K - 1, axis=1)[:, : w.K]
        key = np.take_along_axis(race, part, axis=1)
        order = np.argsort(key, axis=1, kind="stable")
        out[a:b] = np.take_along_axis(part, order, axis=1)
    return out.reshape(w.R, w.T, w.K)


def static_replica_placement(w: Workload, layer: int = 0) -> np.ndarray:
    """Static redundant-replica placement for the LPLB layer.

    Returns ``inst_expert`` int32 [R * (E_loc + 1)]: instance j < E_loc of rank r is the
    main of expert r*E_loc + j; instance E_loc of rank r holds a replica or -1.
    The n_static_replicas most popular experts (ties: lowest id) are replicated once,
    walked in descending popularity; each goes to the first rank of a seeded
    permutation of the ranks that is not its home rank and not yet used.
    """
    assert w.n_static_replicas <= w.R
    p = expert_popularity(w, layer)
    order = np.lexsort((np.arange(w.E), -p))  # popularity desc, id asc
    hot = order[: w.n_static_replicas]
    perm = np.random.default_rng(_seq(w, layer, _STREAM_PLACEMENT)).permutation(w.R)
    ipr = w.E_loc + 1
    inst = np.full(w.R * ipr, -1, dtype=np.int32)
    for r in range(w.R):
        inst[r * ipr: r * ipr + w.E_loc] = np.arange(r * w.E_loc, (r + 1) * w.E_loc)
    used = set()
    for e in hot:
        home = int(e) // w.E_loc
        for r in perm:
            r = int(r)
            if r != home and r not in used:
                used.add(r)
                inst[r * ipr + w.E_loc] = int(e)
                break
        else:
            raise ValueError("no free rank for a static replica")
    return inst


def tensor_seed(w: Workload, layer: int, what: int) -> int:
    """An integer seed for a torch generator drawing activations / weights / grads."""
    return int(_seq(w, layer, _STREAM_TENSORS).spawn(what + 1)[what].generate_state(1, np.uint64)[0]
               & 0x7FFF_FFFF_FFFF_FFFF)


def waterfill_seed(w: Workload) -> int:
    return int(np.random.SeedSequence([w.config_id, 0xA7E5]).generate_state(1, np.uint64)[0])


def imbalance(rank_load: np.ndarray) -> float:
    """max / mean rank load (1.0 for an empty layer)."""
    m = float(np.mean(rank_load))
    return float(np.max(rank_load)) / m if m > 0 else 1.0


def bf16_bytes(n_elems: int) -> int:
    return 2 * n_elems


def fmt_bytes(n: int) -> str:
    for unit in ("B", "KiB", "MiB", "GiB"):
        if n < 1024 or unit == "GiB":
            return f"{n:.2f} {unit}" if unit != "B" else f"{n} B"
        n /= 1024.0
    return str(n)


__all__ = [
    "Workload", "TINY", "QWEN_LAYER", "QWEN_SWEEP", "DSV3_WATERFILL", "LPLB_LAYER", "ALL",
    "scaled", "zipf_exponent", "expert_popularity", "routing", "static_replica_placement",
    "tensor_seed", "waterfill_seed", "imbalance",
]
