"""Oracle: redundant-slot weight staging and backward gradient reduction.

UltraEP article:
* section "共享冗余 slot 管理动态专家副本" (shared redundant slots): every rank keeps a
  fixed number of redundant slots; the weights of the experts the current layer needs
  are written into them; slots hold weights and a gradient buffer but no optimizer
  state; one set of slots is reused by every MoE layer (for Qwen3-235B-A22B: 36 MB of
  weights plus 72 MB of gradients per rank, 108 MB, instead of 9.9 GB per rank for
  per-layer slots);
* section "复用前向方案，完成权重恢复与梯度归约" (backward replay): backward does not
  solve again, it reuses the forward plan, writes the replica weights into the slots
  again, reduces the replicas' gradients into the main expert's gradient buffer and
  clears the redundant gradient buffer for the next layer.

Readings: weights are bf16 bits copied verbatim; gradients are fp32 (72 MB = 2 x 36 MB);
the reduction adds the replicas in ascending rank order to the main's gradient, in fp32
with round-to-nearest-even, one add at a time; cleared means +0.0.

Pins: bitwise copy; sums checked against fp64 within the fp32 bound and exactly on
integer-valued data; the article's memory arithmetic (tests/golden/slot_memory.json).
"""

import numpy as np


def stage_forward(slot_expert: np.ndarray, main_w: np.ndarray, slot_w: np.ndarray,
                  r_begin: int = 0, r_end: int = None) -> None:
    """slot_w[r][s] = main_w[slot_expert[r][s]] for used slots of ranks [r_begin, r_end)."""
    R, S = slot_expert.shape
    r_end = R if r_end is None else r_end
    for r in range(r_begin, r_end):
        for s in range(S):
            e = int(slot_expert[r, s])
            if e >= 0:
                slot_w[r, s] = main_w[e]


def grad_reduce(slot_expert: np.ndarray, main_grad: np.ndarray, slot_grad: np.ndarray,
                E_loc: int, r_begin: int = 0, r_end: int = None) -> None:
    """main_grad[e] += replica grads in ascending rank (fp32, one add at a time); zero them.

    Only experts whose home rank e // E_loc lies in [r_begin, r_end) are reduced.
    """
    R, S = slot_expert.shape
    r_end = R if r_end is None else r_end
    assert main_grad.dtype == np.float32 and slot_grad.dtype == np.float32
    replicated = sorted(set(int(e) for e in slot_expert.reshape(-1) if e >= 0))
    for e in replicated:
        if not (r_begin <= e // E_loc < r_end):
            continue
        acc = main_grad[e].copy()
        for r in range(R):
            for s in range(S):
                if int(slot_expert[r, s]) == e:
                    acc = (acc + slot_grad[r, s]).astype(np.float32)
                    slot_grad[r, s] = np.float32(0.0)
        main_grad[e] = acc
