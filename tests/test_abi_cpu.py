"""The C-ABI library loads on a machine without a GPU, exports every symbol
the header declares, and validates arguments on the host (no compute)."""

import ctypes
import os

import pytest

import draft_verify_sampling_block_amd as dv


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(dv.lib_path()):
        from draft_verify_sampling_block_amd.build import build_library
        build_library()
    return dv.load()


def test_header_symbols_are_exported(lib):
    names = dv.header_names()
    for n in ("dspark_draft_block", "dspark_confidence", "dspark_schedule", "dspark_verify",
              "dspark_draft_block_workspace", "dspark_verify_workspace",
              "dspark_schedule_workspace", "dspark_status_str", "dspark_last_error",
              "dspark_version"):
        assert n in names
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing


def test_no_undeclared_c_symbols_exported(lib):
    # every unmangled function the library exports is one the header declares
    # (helpers inside the extern "C" block must be file-local)
    import shutil
    import subprocess
    if shutil.which("nm") is None:
        pytest.skip("nm not available")
    out = subprocess.run(["nm", "-D", "--defined-only", dv.lib_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines()
                if len(ln.split()) == 3 and ln.split()[1] == "T"}
    c_names = {n for n in exported if not n.startswith("_Z")}
    assert c_names, "no C symbols found"
    assert c_names <= set(dv.header_names()), sorted(c_names - set(dv.header_names()))


def test_status_strings_and_version(lib):
    assert lib.dspark_status_str(0) == b"DSPARK_OK"
    for code in (-1, -2, -3, -4, -5, -6):
        assert lib.dspark_status_str(code).startswith(b"DSPARK_E")
    assert b"gfx950" in lib.dspark_version()


def test_workspace_queries(lib):
    # a 1536-byte header (the pipelined kernel's start barrier), the
    # per-64-entry-tile max, argmax and exp-sum, then the persistent kernel's
    # flag words (4096 groups x 128 bytes, one word per request), then the
    # pipelined kernel's region (a word per request and tile, 256 group words
    # per request, a token flag per request), each part 256-byte aligned
    a256 = lambda n: (n + 255) // 256 * 256
    nT = (151936 + 63) // 64
    expect = 1536 + 3 * a256(128 * nT * 4) + a256(4096 * 32 * 4) + a256(128 * 4)
    expect += a256(128 * nT * 8) + a256(128 * 256 * 8) + a256(128 * 4)
    assert dv.dspark_draft_block_workspace(128, 15, 151936, 256, 1) == expect
    assert dv.dspark_draft_block_workspace(128, 15, 151937, 256, 1) == 0  # invalid V
    assert dv.dspark_verify_workspace(4, 5, 1024, 32, 0) > 0
    # the candidates' ranks (int32, 256-byte aligned) up to 4096 candidates; none beyond
    assert dv.dspark_schedule_workspace(512, 7) == 512 * 7 * 4
    assert dv.dspark_schedule_workspace(3, 5) == 256
    assert dv.dspark_schedule_workspace(1000, 8) == 0


def test_host_validation_rejects_before_launch(lib):
    P = [None] * 11
    rc = lib.dspark_draft_block(4, 5, 1024, 32, 0, *P, None, 0, None)
    assert rc == -1 and b"'U' is NULL" in lib.dspark_last_error()
    assert lib.dspark_draft_block(0, 5, 1024, 32, 0, *P, None, 0, None) == -1
    assert lib.dspark_draft_block(4, 65, 1024, 32, 0, *P, None, 0, None) == -1
    assert lib.dspark_draft_block(4, 5, 1024, 32, 9, *P, None, 0, None) == -2
    assert lib.dspark_draft_block(4, 5, 1020, 32, 0, *P, None, 0, None) == -1
    assert lib.dspark_draft_block(4, 5, 1024, 48, 0, *P, None, 0, None) == -1
    assert lib.dspark_draft_block(4, 5, 1024, 96, 1, *P, None, 0, None) == -1  # bf16 rank
    fake = 4096  # aligned, never dereferenced: validation fails first
    assert lib.dspark_draft_block(4, 5, 1024, 32, 0, *([fake] * 11), fake, 16, None) == -4
    assert lib.dspark_draft_block(4, 5, 1024, 32, 0, *([fake + 8] + [fake] * 10), fake, 1 << 30,
                                  None) == -3
    # the fused draft + confidence call: H a positive multiple of 8, every
    # pointer but temps and status given, the draft's workspace
    cf = lambda H, ptrs, ws, nbytes: lib.dspark_draft_block_conf(
        4, 5, 1024, 32, H, 0, *ptrs[:8], 0.0, None, *ptrs[8:], None, ws, nbytes, None)
    assert cf(20, [fake] * 13, fake, 1 << 30) == -1                      # H % 8
    assert cf(0, [fake] * 13, fake, 1 << 30) == -1
    rc = cf(24, [fake] * 7 + [None] + [fake] * 5, fake, 1 << 30)         # w missing
    assert rc == -1 and b"'w' is NULL" in lib.dspark_last_error()
    assert cf(24, [fake] * 12 + [None], fake, 1 << 30) == -1             # conf missing
    assert cf(24, [fake] * 13, fake, 16) == -4                           # workspace
    assert lib.dspark_schedule(9000, 1, fake, fake, 10, fake, None, None, None, None, 0, None) == -5
    assert lib.dspark_schedule(4, 2, fake, fake, 0, fake, None, None, None, None, 0, None) == -1
    assert lib.dspark_schedule_noalloc(9000, 1, fake, fake, 10, fake, None, None, None, None) == -5
    assert lib.dspark_schedule_noalloc(4, 2, fake, fake, 0, fake, None, None, None, None) == -1
    assert lib.dspark_schedule_noalloc(4, 2, fake + 4, fake, 5, fake, None, None, None, None) == -3
    assert lib.dspark_confidence(4, 5, 60, 1024, 32, 1, *([fake] * 5), ctypes.c_float(0.0), fake,
                                 None, None) == -1  # H % 8
    assert lib.dspark_verify(4, 5, 1024, 32, 1, *([fake] * 15), None, fake, 8, None) == -4
