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


def compare_dispatch_rows(x, out, dest_row_oracle, chunk_rows=1 << 18):
    """Every row of a dispatch buffer against the oracle's definition of the permute:
    row d holds x[row_src[d] // K] bit for bit, row_src being the oracle's inverse of its
    own dest_row (oracle.row_sources).  The expected rows are gathered from x on the
    device chunk by chunk (so buffers of 100+ GiB are compared whole) and compared
    element by element with torch.equal.  Rows no pair targets must be all zero bits
    (callers pass a zeroed buffer when such rows exist).  Returns the oracle's row_src."""
    import oracle as O
    P, H = out.shape
    K = dest_row_oracle.shape[-1]
    src = O.row_sources(dest_row_oracle, P)
    xf = x.reshape(-1, H).view(torch.int16)
    of = out.view(torch.int16)
    for a in range(0, P, chunk_rows):
        b = min(P, a + chunk_rows)
        s = src[a:b]
        live = s >= 0
        if live.all():
            exp = xf.index_select(0, torch.from_numpy(s // K).to(DEV))
            assert torch.equal(of[a:b], exp), f"dispatch rows [{a}, {b}) differ"
        else:
            idx = np.nonzero(live)[0]
            if idx.size:
                exp = xf.index_select(0, torch.from_numpy(s[idx] // K).to(DEV))
                got = of[a:b].index_select(0, torch.from_numpy(idx).to(DEV))
                assert torch.equal(got, exp), f"dispatch rows in [{a}, {b}) differ"
            dead = np.nonzero(~live)[0]
            got0 = of[a:b].index_select(0, torch.from_numpy(dead).to(DEV))
            assert int(torch.count_nonzero(got0)) == 0, f"untargeted rows in [{a}, {b}) written"
    return src
