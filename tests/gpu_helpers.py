"""Shared helpers of the GPU parity tests: run the HIP path through the C-ABI binding
on seeded inputs and compare with the oracle on the same inputs."""

import numpy as np
import torch

DEV = "cuda:0"


def to_dev(a, dtype=torch.int32):
    return torch.from_numpy(np.ascontiguousarray(a)).to(device=DEV, dtype=dtype)


def host(t):
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def err_word():
    return torch.zeros(1, dtype=torch.int32, device=DEV)


def say(*a):
    print(*a, flush=True)


def plan_on_gpu(U, ids_d, E, S, q_min, r_begin=0, r_end=None):
    """load matrix -> quota solve -> reroute/assign on the device; returns device tensors."""
    err = err_word()
    counts, bp = U.load_matrix(ids_d, E, err=err)
    plan = U.solve_quota(counts, S, q_min)
    xfer, ioff, dinst, drow = U.reroute_assign(counts, ids_d, bp, plan["inst_per_rank"],
                                               plan["inst_expert"], plan["inst_quota"],
                                               r_begin=r_begin, r_end=r_end, err=err)
    return dict(counts=counts, bucket_pos=bp, plan=plan, xfer=xfer, inst_offset=ioff,
                dest_inst=dinst, dest_row=drow, err=err)


def random_routing(rng, R, T, K, E, p=None, empty_frac=0.0):
    p = rng.dirichlet(np.full(E, 0.3)) if p is None else p
    ids = np.zeros((R, T, K), dtype=np.int32)
    for r in range(R):
        for t in range(T):
            ids[r, t] = rng.choice(E, K, replace=False, p=p)
    if empty_frac:
        ids[rng.random(ids.shape) < empty_frac] = -1
    return ids
