"""Host replay of the attention kernel's memory accesses (tests/c/attn_replay.cpp),
built with AddressSanitizer and UndefinedBehaviorSanitizer: every global and
LDS address the kernel computes -- through the same functions of
csrc/attn_geom.h -- stays inside its buffer over whole launches of many shapes,
for the launched 8-wavefront shape and the 4-wavefront one; every packed query
row is owned by one lane, every kept block is visited once as a tile and every
pruned column lies in exactly one visited summary sub-tile; and every MFMA
operand read of the tile compute returns the (key, dim) the contraction
expects, from an LDS image filled through the load functions. A second test
plants mistakes in a copy of the address functions and checks the replay
reports them. CPU only."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "c", "attn_replay.cpp")
CSRC = os.path.join(ROOT, "block_sparse_long_estimate_amd", "csrc")
CLANG = "/opt/rocm/llvm/bin/clang++"
ROCM_INC = "/opt/rocm/include"


def build(src, exe):
    cmd = [CLANG, "-std=c++17", "-O1", "-g", "-D__HIP_PLATFORM_AMD__", "-I", ROCM_INC,
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", src, "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr


@pytest.fixture(scope="module")
def have_clang():
    if not os.path.exists(CLANG):
        pytest.skip("ROCm clang++ not found")


def test_every_access_in_bounds(tmp_path, have_clang):
    exe = str(tmp_path / "attn_replay")
    build(SRC, exe)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-3000:]
    assert r.stdout.startswith("ok "), r.stdout


MUTANTS = [
    ("ragged tile rows not clamped to the last key",
     "const int sk = j * BLK + (key < rmax ? key : rmax);", "const int sk = j * BLK + key;"),
    ("summary column not clamped to the last block",
     "const int jp = jc < s.nbk - 1 ? jc : s.nbk - 1;", "const int jp = jc;"),
    ("pieces past the tile loaded",
     "return k < NP - 1 || PIECES % NW == 0 || k * NW + wave < PIECES;", "return true;"),
    ("padding chunks not redirected to the row's data",
     "return PieceLoc{row, ch < data_chunks ? ch : data_chunks - 1};", "return PieceLoc{row, ch};"),
    ("packed rows of a 4-wavefront slice overlap",
     "return slice * 256 + wave * (32 * RG) + rg * 32 + n;", "return slice * 256 + wave * 32 + rg * 32 + n;"),
    ("bf16 V rows read without their rotation", "64 * ((db + rsub) & 3) + 2 * dsub", "64 * db + 2 * dsub"),
    ("fp8 V rows loaded without their rotation", "(ch - 2 * ((row >> 1) & 3)) & 7", "ch & 7"),
    ("K operand dim halves swapped", ": 16 * ks + 8 * lh;", ": 16 * ks + 8 * (lh ^ 1);"),
    ("split parts overlap by a tile", "z = (int)((long long)T * (split + 1) / nsplit);",
     "z = (int)((long long)T * (split + 1) / nsplit) + (split + 1 < nsplit);"),
    ("split units give two workgroups the same part", "return UnitMap{8 * (k8 / per) + xcd, rem % slices, rem / slices};",
     "return UnitMap{8 * (k8 / per) + xcd, rem % slices, rem % nsplit};"),
    ("whole summary sub-tiles read lo rows from the hi array",
     "k_off[k] = has_k(k, wave) ? (part ? lo_delta : 0u)", "k_off[k] = has_k(k, wave) ? (part ? 0u : 0u)"),
    ("whole summary sub-tiles read V without the row rotation",
     "const PieceLoc pv = piece_loc(VSTR, 0, lane, 16);", "const PieceLoc pv = piece_loc(KSTR, 0, lane, 16);"),
    ("fp8 V key permutation dropped from the contiguous loads",
     "const int key = PERM ? vt_slot(pl.row) : pl.row;\n            off[k] = has(k, wave) ? (uint32_t)",
     "const int key = pl.row;\n            off[k] = has(k, wave) ? (uint32_t)"),
]


@pytest.mark.parametrize("what,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistakes_are_reported(tmp_path, have_clang, what, old, new):
    csrc = tmp_path / "block_sparse_long_estimate_amd" / "csrc"
    csrc.mkdir(parents=True)
    (tmp_path / "tests" / "c").mkdir(parents=True)
    shutil.copy(os.path.join(CSRC, "fp_internal.h"), csrc)
    text = open(os.path.join(CSRC, "attn_geom.h")).read()
    assert text.count(old) == 1, what
    (csrc / "attn_geom.h").write_text(text.replace(old, new))
    src = tmp_path / "tests" / "c" / "attn_replay.cpp"
    shutil.copy(SRC, src)
    exe = str(tmp_path / "replay")
    build(str(src), exe)
    r = subprocess.run([exe, "quick"], capture_output=True, text=True, timeout=300)
    assert r.returncode != 0 and any(m in r.stderr for m in ("out of bounds", "owned", "operand layout")), what + r.stderr[-500:]


def test_tile_sequence_mistake_is_reported(tmp_path, have_clang):
    """A tile sequence that skips the kept block after the first must be
    reported (coverage, not bounds)."""
    csrc = tmp_path / "block_sparse_long_estimate_amd" / "csrc"
    csrc.mkdir(parents=True)
    (tmp_path / "tests" / "c").mkdir(parents=True)
    shutil.copy(os.path.join(CSRC, "fp_internal.h"), csrc)
    text = open(os.path.join(CSRC, "attn_geom.h")).read()
    old = "int wd = (code + 1) >> 5;\n        uint32_t w = code + 1 <= i ? kept[wd] & (~0u << ((code + 1) & 31)) : 0u;"
    new = "int wd = (code + 2) >> 5;\n        uint32_t w = code + 2 <= i ? kept[wd] & (~0u << ((code + 2) & 31)) : 0u;"
    assert text.count(old) == 1
    (csrc / "attn_geom.h").write_text(text.replace(old, new))
    src = tmp_path / "tests" / "c" / "attn_replay.cpp"
    shutil.copy(SRC, src)
    exe = str(tmp_path / "replay")
    build(str(src), exe)
    r = subprocess.run([exe, "quick"], capture_output=True, text=True, timeout=300)
    assert r.returncode != 0 and "visited" in r.stderr
