"""Thin Python binding of libuep.so (the C-ABI in include/uep.h).

Argument marshalling only: torch supplies device memory and the HIP stream; every
step of the balancing path runs in the library's HIP kernels.  Output tensors the
caller does not pass are allocated with torch on the input's device.  A non-zero
status raises UEPError.  Importing this module fails loudly when the library is
not built: there is no fallback path.
"""

from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libuep.so")

OK, EINVAL, EGEOM, EWORKSPACE, EHIP = 0, 1, 2, 3, 4
ERR_ID_RANGE, ERR_DUP_ID, ERR_QUOTA_SUM, ERR_INST_DUP = 1, 2, 4, 8
ERR_BAD_QUOTA, ERR_COVER, ERR_LP, ERR_ROW_RANGE = 16, 32, 64, 128
STAGE_WEIGHTS, STAGE_GRAD_REDUCE = 0, 1

_P = ctypes.c_void_p
_I = ctypes.c_int32
_I64 = ctypes.c_int64
_U64 = ctypes.c_uint64
_SZ = ctypes.c_size_t

# name -> (restype, argtypes); the exact list of symbols include/uep.h declares
SIGNATURES = {
    "uep_version": (ctypes.c_char_p, []),
    "uep_status_string": (ctypes.c_char_p, [_I]),
    "uep_device_copy": (_I, [_P, _P, _I64, _P]),
    "uep_device_fill": (_I, [_P, _I64, ctypes.c_uint32, _P]),
    "uep_load_matrix_workspace_size": (_SZ, [_I, _I, _I, _I]),
    "uep_load_matrix": (_I, [_P, _I, _I, _I, _I, _P, _P, _P, _P, _SZ, _P]),
    "uep_load_matrix_noalloc": (_I, [_P, _I, _I, _I, _I, _P, _P, _P, _P]),
    "uep_solve_quota": (_I, [_P, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P]),
    "uep_identity_quota": (_I, [_P, _I, _I, _I, _P, _P, _P]),
    "uep_reroute_workspace_size": (_SZ, [_I, _I, _I]),
    "uep_reroute_assign": (_I, [_P, _P, _P, _I, _I, _I, _I, _I, _P, _P, _I, _I,
                                _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "uep_plan_workspace_size": (_SZ, [_I, _I, _I, _I, _I]),
    "uep_plan": (_I, [_P, _I, _I, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                      _P, _P, _P, _SZ, _P]),
    "uep_permute": (_I, [_P, _P, _I, _I, _I, _I, _I, _I, _P, _I64, _P, _P, _P]),
    "uep_combine": (_I, [_P, _I64, _P, _P, _I, _I, _I, _I, _I, _I, _P, _P, _P]),
    "uep_stage_replica_weights": (_I, [_I, _I, _I, _I, _P, _I, _I, _P, _P, _P, _P, _I64, _P]),
    "uep_waterfill": (_I, [_P, _P, _P, _I, _I, _I, _I, _U64, _U64, _I, _I, _P, _P, _P, _P, _P,
                           _P]),
    "uep_lplb_struct_size": (_SZ, [_I, _I, _I]),
    "uep_lplb_prepare": (_I, [_P, _I, _I, _I, _P, _SZ, _P]),
    "uep_lplb_sample": (_I, [_P, _I, _I, _I, _P, _P, _U64, _U64, _P, _P, _P]),
    "uep_lplb": (_I, [_P, _P, _I, _P, _P, _P, _P, _P, _P]),
    "uep_lplb_plan_workspace_size": (_SZ, [_I, _I, _I, _I, _I]),
    "uep_lplb_plan": (_I, [_P, _I, _I, _I, _I, _P, _I, _P, _I, _I, _I] + [_P] * 12 + [_SZ, _P]),
}


class UEPError(RuntimeError):
    pass


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run `python -c 'import __graft_entry__ as g; g.build()'`")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


LIB = _load()


def version() -> str:
    return LIB.uep_version().decode()


def _check(status: int, name: str) -> None:
    if status != OK:
        raise UEPError(f"{name}: {LIB.uep_status_string(status).decode()} (status {status})")


def _p(t: Optional[torch.Tensor]):
    """Device pointer of a contiguous GPU tensor (None stays NULL).  A host tensor is
    refused here: its address handed to a kernel would fault the device."""
    if t is None:
        return None
    if not t.is_cuda:
        raise TypeError("the library takes device memory: got a tensor on " + str(t.device))
    if not t.is_contiguous():
        raise TypeError("the library takes contiguous tensors")
    return ctypes.c_void_p(t.data_ptr())


def _s(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _i32(t: torch.Tensor, name: str) -> torch.Tensor:
    if t.dtype != torch.int32 or not t.is_contiguous():
        raise TypeError(f"{name} must be a contiguous int32 tensor")
    return t


def _new(shape, like: torch.Tensor, dtype=torch.int32) -> torch.Tensor:
    return torch.empty(shape, dtype=dtype, device=like.device)


def _buf(t: Optional[torch.Tensor], n: int, name: str, dtype=torch.int32):
    """A caller's buffer for the library to read or write: contiguous, of `dtype` (any
    16-bit type for torch.int16), with at least n elements, since the kernels index it
    by the geometry alone.  None stays None."""
    if t is None:
        return None
    ok_type = t.element_size() == 2 if dtype == torch.int16 else t.dtype == dtype
    if not ok_type or not t.is_contiguous() or t.numel() < n:
        raise TypeError(f"{name} must be a contiguous {dtype} tensor of at least {n} elements")
    return t


# ---------------------------------------------------------------------------
def load_matrix_workspace_size(R, T, K, E) -> int:
    return int(LIB.uep_load_matrix_workspace_size(R, T, K, E))


def load_matrix(topk_ids, E, counts=None, bucket_pos=None, err=None, ws=None, stream=None,
                counts_only=False):
    """counts [R][E] and bucket_pos [R][T][K]; with counts_only=True the positions are
    not computed and None is returned in their place."""
    _i32(topk_ids, "topk_ids")
    R, T, K = topk_ids.shape
    counts = _new((R, E), topk_ids) if counts is None else _buf(counts, R * E, "counts")
    if counts_only:
        bucket_pos = None
    elif bucket_pos is None:
        bucket_pos = _new((R, T, K), topk_ids)
    else:
        _buf(bucket_pos, R * T * K, "bucket_pos")
    _buf(err, 1, "err")
    n = load_matrix_workspace_size(R, T, K, E)
    ws = _new((max(n, 4),), topk_ids, torch.uint8) if ws is None else ws
    _check(LIB.uep_load_matrix(_p(topk_ids), R, T, K, E, _p(counts), _p(bucket_pos), _p(err),
                               _p(ws), ws.numel() * ws.element_size(), _s(stream)),
           "uep_load_matrix")
    return counts, bucket_pos


def load_matrix_noalloc(topk_ids, E, counts=None, bucket_pos=None, err=None, stream=None,
                        counts_only=False):
    """uep_load_matrix_noalloc: as load_matrix, with the library's own per-device scratch
    instead of a workspace (pass counts / bucket_pos to allocate nothing here either)."""
    _i32(topk_ids, "topk_ids")
    R, T, K = topk_ids.shape
    counts = _new((R, E), topk_ids) if counts is None else _buf(counts, R * E, "counts")
    if counts_only:
        bucket_pos = None
    elif bucket_pos is None:
        bucket_pos = _new((R, T, K), topk_ids)
    else:
        _buf(bucket_pos, R * T * K, "bucket_pos")
    _buf(err, 1, "err")
    _check(LIB.uep_load_matrix_noalloc(_p(topk_ids), R, T, K, E, _p(counts), _p(bucket_pos),
                                       _p(err), _s(stream)), "uep_load_matrix_noalloc")
    return counts, bucket_pos


def solve_quota(counts, S, q_min, out=None, stream=None):
    _i32(counts, "counts")
    R, E = counts.shape
    ipr = E // R + S
    o = out or {}
    slot_expert = o.get("slot_expert", _new((R, max(S, 1)), counts))
    inst_expert = o.get("inst_expert", _new((R * ipr,), counts))
    inst_quota = o.get("inst_quota", _new((R * ipr,), counts))
    rank_load = o.get("rank_load", _new((R,), counts))
    stats = o.get("stats", _new((4,), counts))
    for name, t, n in (("slot_expert", slot_expert, R * S), ("inst_expert", inst_expert, R * ipr),
                       ("inst_quota", inst_quota, R * ipr), ("rank_load", rank_load, R),
                       ("stats", stats, 4)):
        _buf(t, n, name)
    _check(LIB.uep_solve_quota(_p(counts), R, E, S, q_min, _p(slot_expert), _p(inst_expert),
                               _p(inst_quota), _p(rank_load), _p(stats), _s(stream)),
           "uep_solve_quota")
    return {"slot_expert": slot_expert[:, :S], "inst_expert": inst_expert,
            "inst_quota": inst_quota, "rank_load": rank_load, "stats": stats,
            "inst_per_rank": ipr}


def identity_quota(counts, inst_expert, inst_quota=None, stream=None):
    _i32(counts, "counts")
    R, E = counts.shape
    _i32(inst_expert, "inst_expert")
    n = inst_expert.numel()
    inst_quota = _new((n,), counts) if inst_quota is None else _buf(inst_quota, n, "inst_quota")
    _check(LIB.uep_identity_quota(_p(counts), R, E, n, _p(inst_expert), _p(inst_quota),
                                  _s(stream)), "uep_identity_quota")
    return inst_quota


def reroute_workspace_size(R, E, inst_per_rank) -> int:
    return int(LIB.uep_reroute_workspace_size(R, E, inst_per_rank))


def reroute_assign(counts, topk_ids, bucket_pos, inst_per_rank, inst_expert, inst_quota,
                   r_begin=0, r_end=None, xfer=None, inst_offset=None, dest_inst=None,
                   dest_row=None, err=None, ws=None, stream=None):
    _i32(counts, "counts")
    _i32(topk_ids, "topk_ids")
    R, E = counts.shape
    _, T, K = topk_ids.shape
    r_end = R if r_end is None else r_end
    I = R * inst_per_rank
    _buf(bucket_pos, R * T * K, "bucket_pos")
    _buf(inst_expert, I, "inst_expert")
    _buf(inst_quota, I, "inst_quota")
    _buf(err, 1, "err")
    xfer = _new((R, I), counts) if xfer is None else _buf(xfer, R * I, "xfer")
    inst_offset = _new((I + 1,), counts) if inst_offset is None else _buf(inst_offset, I + 1,
                                                                           "inst_offset")
    dest_inst = _new((R, T, K), counts) if dest_inst is None else _buf(dest_inst, R * T * K,
                                                                       "dest_inst")
    dest_row = _new((R, T, K), counts) if dest_row is None else _buf(dest_row, R * T * K,
                                                                     "dest_row")
    n = reroute_workspace_size(R, E, inst_per_rank)
    ws = _new((max(n, 4),), counts, torch.uint8) if ws is None else ws
    _check(LIB.uep_reroute_assign(_p(counts), _p(topk_ids), _p(bucket_pos), R, T, K, E,
                                  inst_per_rank, _p(inst_expert), _p(inst_quota), r_begin, r_end,
                                  _p(xfer), _p(inst_offset), _p(dest_inst), _p(dest_row),
                                  _p(err), _p(ws), ws.numel() * ws.element_size(), _s(stream)),
           "uep_reroute_assign")
    return xfer, inst_offset, dest_inst, dest_row


def plan_workspace_size(R, T, K, E, S) -> int:
    return int(LIB.uep_plan_workspace_size(R, T, K, E, S))


def plan(topk_ids, E, S, q_min, r_begin=0, r_end=None, out=None, err=None, ws=None, stream=None):
    """uep_plan: load matrix, quota solve and reroute/assignment in one call.  `out` may
    hold preallocated buffers under the keys below; returns that dict."""
    _i32(topk_ids, "topk_ids")
    R, T, K = topk_ids.shape
    r_end = R if r_end is None else r_end
    ipr = E // R + S
    I = R * ipr
    shapes = {"counts": (R, E), "bucket_pos": (R, T, K), "slot_expert": (R, max(S, 1)),
              "inst_expert": (I,), "inst_quota": (I,), "rank_load": (R,), "stats": (4,),
              "xfer": (R, I), "inst_offset": (I + 1,), "dest_inst": (R, T, K),
              "dest_row": (R, T, K)}
    o = {} if out is None else dict(out)
    for k, shp in shapes.items():
        n = 1
        for d in shp:
            n *= d
        o[k] = _new(shp, topk_ids) if o.get(k) is None else _buf(o[k], n, k)
    _buf(err, 1, "err")
    need = plan_workspace_size(R, T, K, E, S)
    ws = _new((max(need, 4),), topk_ids, torch.uint8) if ws is None else ws
    _check(LIB.uep_plan(_p(topk_ids), R, T, K, E, S, q_min, r_begin, r_end, _p(o["counts"]),
                        _p(o["bucket_pos"]), _p(o["slot_expert"]), _p(o["inst_expert"]),
                        _p(o["inst_quota"]), _p(o["rank_load"]), _p(o["stats"]), _p(o["xfer"]),
                        _p(o["inst_offset"]), _p(o["dest_inst"]), _p(o["dest_row"]), _p(err),
                        _p(ws), ws.numel() * ws.element_size(), _s(stream)), "uep_plan")
    o["inst_per_rank"] = ipr
    return o


def permute(x, dest_row, out, row_src=None, r_begin=0, r_end=None, stream=None, err=None):
    """x [R][T][H] bf16 (or 16-bit) tensor; out [P][H] of the same dtype (P rows bound
    the dispatch rows: an entry of dest_row outside [-1, P) is skipped and flagged)."""
    R, T, H = x.shape
    _i32(dest_row, "dest_row")
    K = dest_row.shape[2]
    r_end = R if r_end is None else r_end
    if x.element_size() != 2 or out.element_size() != 2:
        raise TypeError("x and out must hold 16-bit elements")
    if tuple(dest_row.shape) != (R, T, K) or out.dim() != 2 or out.shape[1] != H:
        raise TypeError("dest_row must be [R][T][K] and out [P][H] for x [R][T][H]")
    if row_src is not None:
        _i32(row_src, "row_src")
        if row_src.numel() != out.shape[0]:
            raise TypeError("row_src must have one entry per row of out")
    _check(LIB.uep_permute(_p(x), _p(dest_row), R, T, K, H, r_begin, r_end, _p(out), out.shape[0],
                           _p(row_src), _p(err), _s(stream)), "uep_permute")
    return out, row_src


def combine(out, dest_row, gate_w, y, r_begin=0, r_end=None, stream=None, err=None):
    """out [P][H] 16-bit dispatch buffer; dest_row [R][T][K] int32; gate_w [R][T][K]
    float32; y [R][T][H] 16-bit (rows of ranks in [r_begin, r_end) are written)."""
    _i32(dest_row, "dest_row")
    if out.dim() != 2 or dest_row.dim() != 3:
        raise TypeError("out must be [P][H] and dest_row [R][T][K]")
    R, T, K = dest_row.shape
    H = out.shape[1]
    r_end = R if r_end is None else r_end
    if out.element_size() != 2 or y.element_size() != 2:
        raise TypeError("out and y must hold 16-bit elements")
    if gate_w.dtype != torch.float32 or tuple(gate_w.shape) != (R, T, K):
        raise TypeError("gate_w must be float32 [R][T][K]")
    if tuple(y.shape) != (R, T, H):
        raise TypeError("y must be [R][T][H]")
    _check(LIB.uep_combine(_p(out), out.shape[0], _p(dest_row), _p(gate_w), R, T, K, H, r_begin,
                           r_end, _p(y), _p(err), _s(stream)), "uep_combine")
    return y


def device_copy(src, dst, stream=None):
    """Plain copy of src into dst (same byte size, both contiguous device tensors)."""
    n = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != n or not (src.is_contiguous() and dst.is_contiguous()):
        raise TypeError("device_copy needs two contiguous tensors of the same byte size")
    _check(LIB.uep_device_copy(_p(src), _p(dst), n, _s(stream)), "uep_device_copy")
    return dst


def device_fill(dst, value=0, stream=None):
    """Writes the 32-bit word `value` over the contiguous device tensor dst (a byte size
    that is a multiple of 16)."""
    if not dst.is_contiguous():
        raise TypeError("device_fill needs a contiguous tensor")
    n = dst.numel() * dst.element_size()
    _check(LIB.uep_device_fill(_p(dst), n, value & 0xFFFFFFFF, _s(stream)), "uep_device_fill")
    return dst


def stage_replica_weights(mode, R, E, S, slot_expert, expert_elems, main_w=None, slot_w=None,
                          main_grad=None, slot_grad=None, r_begin=0, r_end=None, stream=None):
    r_end = R if r_end is None else r_end
    n = int(expert_elems)
    _buf(slot_expert, R * S, "slot_expert")
    _buf(main_w, E * n, "main_w", torch.int16)
    _buf(slot_w, R * S * n, "slot_w", torch.int16)
    _buf(main_grad, E * n, "main_grad", torch.float32)
    _buf(slot_grad, R * S * n, "slot_grad", torch.float32)
    _check(LIB.uep_stage_replica_weights(mode, R, E, S, _p(slot_expert), r_begin, r_end,
                                         _p(main_w), _p(slot_w), _p(main_grad), _p(slot_grad),
                                         int(expert_elems), _s(stream)),
           "uep_stage_replica_weights")


def waterfill(counts, topk_ids, batch_size, seed, layer, local_pref_shift=4, shared_rank=None,
              waterline=None, slack=None, rank_load=None, ext_topk=None, want_ext=True,
              stream=None, all_ranks=False):
    _i32(counts, "counts")
    _i32(topk_ids, "topk_ids")
    R, E = counts.shape
    _, T, K = topk_ids.shape
    _buf(batch_size, R, "batch_size")
    shared_rank = _new((R, T), counts) if shared_rank is None else _buf(shared_rank, R * T,
                                                                       "shared_rank")
    waterline = _new((1,), counts) if waterline is None else _buf(waterline, 1, "waterline")
    slack = _new((R,), counts) if slack is None else _buf(slack, R, "slack")
    rank_load = _new((R,), counts) if rank_load is None else _buf(rank_load, R, "rank_load")
    if ext_topk is None and want_ext:
        ext_topk = _new((R, T, K + 1), counts)
    else:
        _buf(ext_topk, R * T * (K + 1), "ext_topk")
    _check(LIB.uep_waterfill(_p(counts), _p(topk_ids), _p(batch_size), R, T, K, E,
                             ctypes.c_uint64(seed & (2 ** 64 - 1)),
                             ctypes.c_uint64(layer & (2 ** 64 - 1)), local_pref_shift,
                             1 if all_ranks else 0, _p(shared_rank), _p(waterline), _p(slack), _p(rank_load),
                             _p(ext_topk), _s(stream)), "uep_waterfill")
    return shared_rank, waterline, slack, rank_load, ext_topk


def lplb_struct_size(R, E, inst_per_rank) -> int:
    return int(LIB.uep_lplb_struct_size(R, E, inst_per_rank))


@dataclasses.dataclass(frozen=True)
class LPStruct:
    """An LP structure from uep_lplb_prepare: the device buffer plus the host's own
    record of its sizes (ranks, experts, instances per rank, instances, replicated
    experts G and their copies n), which the calls below check every caller buffer
    against before a kernel sees it."""

    buf: torch.Tensor
    R: int
    E: int
    inst_per_rank: int
    I: int
    G: int
    n: int


def lplb_prepare(inst_expert_host, R, E, inst_per_rank, device, stream=None) -> LPStruct:
    """Offline: build the LP structure from a host instance table into a device buffer."""
    import numpy as np
    ie = np.ascontiguousarray(np.asarray(inst_expert_host, dtype=np.int32))
    if ie.size != R * inst_per_rank:
        raise TypeError(f"inst_expert must have R * inst_per_rank = {R * inst_per_rank} entries")
    n = lplb_struct_size(R, E, inst_per_rank)
    buf = torch.empty((max(n, 16),), dtype=torch.uint8, device=device)
    _check(LIB.uep_lplb_prepare(ie.ctypes.data_as(ctypes.c_void_p), R, E, inst_per_rank,
                                _p(buf), buf.numel(), _s(stream)), "uep_lplb_prepare")
    copies = np.bincount(ie[(ie >= 0) & (ie < E)], minlength=E)
    rep = copies >= 2
    return LPStruct(buf, R, E, inst_per_rank, R * inst_per_rank, int(rep.sum()),
                    int(copies[rep].sum()))


def _lp(lp) -> LPStruct:
    if not isinstance(lp, LPStruct):
        raise TypeError("lp must be the LPStruct that lplb_prepare returned")
    return lp


def lplb(counts, lp, n_copies=None, n_inst=None, iters=30, x=None, m=None, inst_quota=None,
         stats=None, err=None, stream=None):
    """The LP split for one batch.  n_copies and n_inst, when given, must equal the
    structure's own counts; every buffer is checked against the structure."""
    lp = _lp(lp)
    _i32(counts, "counts")
    if tuple(counts.shape) != (lp.R, lp.E):
        raise TypeError(f"counts must be [{lp.R}][{lp.E}] for this LP structure, got "
                        f"{list(counts.shape)}")
    if n_copies is not None and n_copies != lp.n:
        raise TypeError(f"n_copies {n_copies} != the structure's {lp.n} copies")
    if n_inst is not None and n_inst != lp.I:
        raise TypeError(f"n_inst {n_inst} != the structure's {lp.I} instances")
    x = torch.empty((max(lp.n, 1),), dtype=torch.float32, device=counts.device) if x is None \
        else _buf(x, max(lp.n, 1), "x", torch.float32)
    m = torch.empty((1,), dtype=torch.float32, device=counts.device) if m is None \
        else _buf(m, 1, "m", torch.float32)
    inst_quota = _new((lp.I,), counts) if inst_quota is None else _buf(inst_quota, lp.I,
                                                                        "inst_quota")
    stats = _new((4,), counts) if stats is None else _buf(stats, 4, "stats")
    _buf(err, 1, "err")
    _check(LIB.uep_lplb(_p(counts), _p(lp.buf), iters, _p(x), _p(m), _p(inst_quota), _p(stats),
                        _p(err), _s(stream)), "uep_lplb")
    return x[:lp.n], m, inst_quota, stats


def lplb_plan_workspace_size(R, T, K, E, inst_per_rank) -> int:
    return int(LIB.uep_lplb_plan_workspace_size(R, T, K, E, inst_per_rank))


def lplb_plan(topk_ids, lp, inst_expert, iters=30, r_begin=0, r_end=None, out=None, err=None,
              ws=None, stream=None):
    """uep_lplb_plan: load matrix, LP split and reroute/assignment in one call, with the
    static instance table `inst_expert` [I] the structure was built from.  `out` may hold
    preallocated buffers under the keys below; returns that dict."""
    lp = _lp(lp)
    _i32(topk_ids, "topk_ids")
    R, T, K = topk_ids.shape
    if R != lp.R:
        raise TypeError(f"topk_ids has {R} ranks, the LP structure {lp.R}")
    _buf(inst_expert, lp.I, "inst_expert")
    r_end = R if r_end is None else r_end
    E, I = lp.E, lp.I
    shapes = {"counts": ((R, E), torch.int32), "bucket_pos": ((R, T, K), torch.int32),
              "x": ((max(lp.n, 1),), torch.float32), "m": ((1,), torch.float32),
              "inst_quota": ((I,), torch.int32), "stats": ((4,), torch.int32),
              "xfer": ((R, I), torch.int32), "inst_offset": ((I + 1,), torch.int32),
              "dest_inst": ((R, T, K), torch.int32), "dest_row": ((R, T, K), torch.int32)}
    o = {} if out is None else dict(out)
    for k, (shp, dt) in shapes.items():
        n = 1
        for d in shp:
            n *= d
        o[k] = _new(shp, topk_ids, dt) if o.get(k) is None else _buf(o[k], n, k, dt)
    _buf(err, 1, "err")
    need = lplb_plan_workspace_size(R, T, K, E, lp.inst_per_rank)
    ws = _new((max(need, 4),), topk_ids, torch.uint8) if ws is None else ws
    _check(LIB.uep_lplb_plan(_p(topk_ids), R, T, K, E, _p(lp.buf), lp.inst_per_rank,
                             _p(inst_expert), iters, r_begin, r_end, _p(o["counts"]),
                             _p(o["bucket_pos"]), _p(o["x"]), _p(o["m"]), _p(o["inst_quota"]),
                             _p(o["stats"]), _p(o["xfer"]), _p(o["inst_offset"]),
                             _p(o["dest_inst"]), _p(o["dest_row"]), _p(err), _p(ws),
                             ws.numel() * ws.element_size(), _s(stream)), "uep_lplb_plan")
    o["inst_per_rank"] = lp.inst_per_rank
    return o


def lplb_sample(topk_ids, lp, x, seed, layer, dest_inst=None, err=None, stream=None):
    """Per-token copy draw from LPLB's split: dest_inst [R][T][K] int32."""
    lp = _lp(lp)
    _i32(topk_ids, "topk_ids")
    R, T, K = topk_ids.shape
    if R != lp.R:
        raise TypeError(f"topk_ids has {R} ranks, the LP structure {lp.R}")
    _buf(x, lp.n, "x", torch.float32)
    dest_inst = _new((R, T, K), topk_ids) if dest_inst is None else _buf(dest_inst, R * T * K,
                                                                         "dest_inst")
    _buf(err, 1, "err")
    _check(LIB.uep_lplb_sample(_p(topk_ids), R, T, K, _p(lp.buf), _p(x),
                               ctypes.c_uint64(seed & (2 ** 64 - 1)),
                               ctypes.c_uint64(layer & (2 ** 64 - 1)), _p(dest_inst), _p(err),
                               _s(stream)), "uep_lplb_sample")
    return dest_inst
