"""CPU-only checks of the C-ABI library: it loads, exports every function that
include/uep.h declares, and its host-side argument checks answer without a GPU."""

import ctypes
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "uep.h")
LIB = os.path.join(ROOT, "moe_expert_load_amd", "libuep.so")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(uep_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("libuep.so is not built (run __graft_entry__.build())")
    return ctypes.CDLL(LIB)


def test_header_declares_the_path():
    names = declared_functions()
    for n in ("uep_load_matrix", "uep_solve_quota", "uep_reroute_assign", "uep_permute",
              "uep_stage_replica_weights", "uep_waterfill", "uep_lplb", "uep_combine"):
        assert n in names


def test_solve_quota_comment_states_the_search_the_kernel_runs():
    """The header's account of uep_solve_quota describes the search as built: plain
    steps, then relays, then the stop; the 'top up an existing replica' branch the
    search no longer has is not described."""
    text = open(HEADER).read()
    block = text[text.index("uep_solve_quota -- "):text.index("uep_status uep_solve_quota(")]
    flat = " ".join(re.sub(r"(?m)^\s*\* ?", " ", block).split())
    assert "Relay" in flat and "Plain step" in flat and "stop" in flat
    assert "d2 = min(q_f, T* - L_y)" in flat
    assert "existing replica under T*" not in flat and "top up" not in flat.lower()


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_binding_signature_table_matches_header():
    src = open(os.path.join(ROOT, "moe_expert_load_amd", "uep.py")).read()
    table = set(re.findall(r'"(uep_[a-z0-9_]+)":', src))
    assert table == set(declared_functions())


def test_host_side_calls_without_gpu(lib):
    lib.uep_version.restype = ctypes.c_char_p
    assert b"gfx950" in lib.uep_version()
    lib.uep_status_string.restype = ctypes.c_char_p
    assert lib.uep_status_string(3) == b"workspace too small"
    lib.uep_load_matrix_workspace_size.restype = ctypes.c_size_t
    # one int32 histogram per (rank, chunk of tokens): grows with the token count
    small = lib.uep_load_matrix_workspace_size(32, 1024, 8, 128)
    big = lib.uep_load_matrix_workspace_size(32, 8192, 8, 128)
    assert small > 0 and big > small and big % (32 * 128 * 4) == 0
    lib.uep_reroute_workspace_size.restype = ctypes.c_size_t
    assert lib.uep_reroute_workspace_size(32, 128, 5) > 0
    lib.uep_lplb_struct_size.restype = ctypes.c_size_t
    assert lib.uep_lplb_struct_size(64, 256, 5) > 0
    null = ctypes.c_void_p(None)
    i32 = ctypes.c_int32
    # invalid geometry is refused before anything touches a device
    assert lib.uep_load_matrix(null, i32(0), i32(1), i32(1), i32(4), null, null, null, null,
                               ctypes.c_size_t(0), null) == 1
    assert lib.uep_load_matrix(null, i32(65), i32(1), i32(1), i32(4), null, null, null, null,
                               ctypes.c_size_t(0), null) == 2
    assert lib.uep_solve_quota(null, i32(3), i32(7), i32(1), i32(1), null, null, null, null, null,
                               null) == 2
    i64 = ctypes.c_int64
    assert lib.uep_permute(null, null, i32(2), i32(4), i32(2), i32(12), i32(0), i32(2), null,
                           i64(16), null, null, null) == 2
    assert lib.uep_permute(null, null, i32(2), i32(4), i32(2), i32(16), i32(1), i32(3), null,
                           i64(16), null, null, null) == 1
    assert lib.uep_permute(null, null, i32(2), i32(4), i32(2), i32(16), i32(0), i32(2), null,
                           i64(-1), null, null, null) == 1
    assert lib.uep_lplb_prepare(null, i32(2), i32(2), i32(2), null, ctypes.c_size_t(0), null) == 1
    assert lib.uep_identity_quota(null, i32(65), i32(130), i32(4), null, null, null) == 2
    assert lib.uep_stage_replica_weights(i32(0), i32(4), i32(8), i32(9), null, i32(0), i32(4), null,
                                         null, null, null, ctypes.c_int64(8), null) == 2
    assert lib.uep_combine(null, i64(16), null, null, i32(2), i32(4), i32(2), i32(12), i32(0),
                           i32(2), null, null, null) == 2
    assert lib.uep_combine(null, i64(16), null, null, i32(2), i32(4), i32(2), i32(16), i32(1),
                           i32(3), null, null, null) == 1
    assert lib.uep_combine(null, i64(16), null, null, i32(2), i32(4), i32(2), i32(16), i32(0),
                           i32(2), null, null, null) == 1
    assert lib.uep_combine(null, i64(-1), null, null, i32(2), i32(4), i32(2), i32(16), i32(0),
                           i32(2), null, null, null) == 1
    assert lib.uep_device_copy(null, null, i64(0), null) == 0
    assert lib.uep_device_copy(null, null, i64(-16), null) == 1
    assert lib.uep_device_copy(null, null, i64(32), null) == 1
    fake_a, fake_b = ctypes.c_void_p(4096), ctypes.c_void_p(8192)
    assert lib.uep_device_copy(fake_a, fake_b, i64(24), null) == 2
    assert lib.uep_device_copy(ctypes.c_void_p(4100), fake_b, i64(32), null) == 2
    u32 = ctypes.c_uint32
    assert lib.uep_device_fill(null, i64(0), u32(7), null) == 0
    assert lib.uep_device_fill(null, i64(-16), u32(7), null) == 1
    assert lib.uep_device_fill(null, i64(32), u32(7), null) == 1
    assert lib.uep_device_fill(fake_a, i64(24), u32(7), null) == 2
    assert lib.uep_device_fill(ctypes.c_void_p(4100), i64(32), u32(7), null) == 2
    # the fused plan: workspace = load matrix + reroute workspaces; host checks first
    lib.uep_plan_workspace_size.restype = ctypes.c_size_t
    wp = lib.uep_plan_workspace_size(32, 8192, 8, 128, 1)
    assert wp >= big + lib.uep_reroute_workspace_size(32, 128, 5)
    assert lib.uep_plan_workspace_size(3, 16, 2, 7, 1) == 0             # E % R != 0
    plan_args = [null] * 12 + [null, ctypes.c_size_t(0), null]      # 12 outputs + err, ws
    assert lib.uep_plan(null, i32(3), i32(16), i32(2), i32(7), i32(1), i32(1), i32(0), i32(3),
                        *plan_args) == 2
    assert lib.uep_plan(null, i32(4), i32(16), i32(2), i32(8), i32(1), i32(1), i32(0), i32(5),
                        *plan_args) == 1
    assert lib.uep_plan(null, i32(4), i32(16), i32(2), i32(8), i32(1), i32(1), i32(0), i32(4),
                        *plan_args) == 1
    fake = ctypes.c_void_p(4096)
    assert lib.uep_plan(fake, i32(4), i32(16), i32(2), i32(8), i32(1), i32(1), i32(0), i32(4),
                        *([fake] * 12), fake, ctypes.c_size_t(16), null) == 3


C_PROGRAM = r"""
#include <stdio.h>
#include <string.h>
#include "uep.h"

typedef void (*any_fn)(void);
static const any_fn table[] = {
%(table)s
};

int main(void) {
  const char* v = uep_version();
  if (!v || !strstr(v, "gfx950")) { printf("version: %%s\n", v ? v : "(null)"); return 1; }
  if (strcmp(uep_status_string(UEP_EWORKSPACE), "workspace too small") != 0) return 2;
  /* geometry errors are answered on the host, before any device work */
  if (uep_load_matrix(NULL, 0, 1, 1, 4, NULL, NULL, NULL, NULL, 0, NULL) != UEP_EINVAL) return 3;
  if (uep_load_matrix(NULL, 65, 1, 1, 4, NULL, NULL, NULL, NULL, 0, NULL) != UEP_EGEOM) return 4;
  if (uep_permute(NULL, NULL, 2, 4, 2, 12, 0, 2, NULL, 16, NULL, NULL, NULL) != UEP_EGEOM) return 5;
  if (UEP_ERR_ROW_RANGE != 128) return 6;
  printf("%%d functions, %%s\n", (int)(sizeof table / sizeof table[0]), v);
  return 0;
}
"""


@pytest.mark.parametrize("compiler,std,suffix", [("gcc", "-std=c99", ".c"),
                                                  ("g++", "-std=c++17", ".cpp")])
def test_header_compiles_and_links_from_c_and_cpp(lib, tmp_path, compiler, std, suffix):
    """A plain C99 (and C++17) program, -pedantic -Werror, that names every declared
    function and calls the host-side checks links against libuep.so and runs."""
    cc = shutil.which(compiler)
    if cc is None:
        pytest.skip(f"{compiler} not available")
    names = declared_functions()
    src = tmp_path / f"abi_check{suffix}"
    src.write_text(C_PROGRAM % {"table": ",\n".join(f"  (any_fn){n}" for n in names)})
    exe = tmp_path / "abi_check"
    libdir = os.path.dirname(LIB)
    build = subprocess.run([cc, std, "-Wall", "-Wextra", "-pedantic", "-Werror",
                            "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe),
                            "-L", libdir, "-l:libuep.so", f"-Wl,-rpath,{libdir}"],
                           capture_output=True, text=True)
    assert build.returncode == 0, build.stderr
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert run.returncode == 0, run.stdout + run.stderr
    assert run.stdout.startswith(f"{len(names)} functions")


def test_lplb_binding_checks_buffers_against_the_structure(lib):
    """The LPLB calls check counts, x, inst_quota and topk_ids against the structure's
    own sizes before any kernel could index them (host tensors here: each check must
    fire before a device pointer is taken)."""
    import torch
    from moe_expert_load_amd import uep as U
    lp = U.LPStruct(buf=torch.zeros(64, dtype=torch.uint8), R=4, E=8, inst_per_rank=3, I=12,
                    G=2, n=4)
    counts = torch.zeros(4, 8, dtype=torch.int32)
    with pytest.raises(TypeError, match="counts must be"):
        U.lplb(torch.zeros(4, 9, dtype=torch.int32), lp)
    with pytest.raises(TypeError, match="n_copies"):
        U.lplb(counts, lp, n_copies=5)
    with pytest.raises(TypeError, match="n_inst"):
        U.lplb(counts, lp, n_inst=11)
    with pytest.raises(TypeError, match="x must be"):
        U.lplb(counts, lp, x=torch.zeros(3, dtype=torch.float32))
    with pytest.raises(TypeError, match="inst_quota must be"):
        U.lplb(counts, lp, x=torch.zeros(4, dtype=torch.float32), m=torch.zeros(1),
               inst_quota=torch.zeros(11, dtype=torch.int32))
    with pytest.raises(TypeError, match="LPStruct"):
        U.lplb(counts, lp.buf)
    ids = torch.zeros(5, 2, 2, dtype=torch.int32)
    with pytest.raises(TypeError, match="ranks"):
        U.lplb_sample(ids, lp, torch.zeros(4, dtype=torch.float32), 1, 1)
    with pytest.raises(TypeError, match="x must be"):
        U.lplb_sample(ids[:4], lp, torch.zeros(3, dtype=torch.float32), 1, 1)
    with pytest.raises(TypeError, match="inst_expert must have"):
        U.lplb_prepare([0, 1, -1], 4, 8, 3, "cpu")
