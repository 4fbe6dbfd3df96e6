"""Host-side check of the kernels' LDS tile layouts and lane address maps (no GPU).

The addresses come from the kernels' own layout header (csrc/lds_layout.h), enumerated per
instruction and lane by tests/lds_map.cpp (compiled here with g++).  A bank model is applied to
them; the model is pinned to the counters of the LDS microbenchmark (profiles/lds_banks.txt: the
model's cycles per instruction must match the measured SQ_LDS_IDX_ACTIVE / SQ_INSTS_LDS for every
pattern measured, conflicted or not).

Bank model (64 banks of 4 bytes):
  * 16-byte reads: 4 passes of 16 lanes; a pass costs the largest number of distinct 16-byte chunks
    that share a 16-byte slot modulo 256 bytes;
  * transposing 8-byte reads: 2 passes of 32 lanes; same with 8-byte words modulo 256 bytes;
  * 16-byte stores: 8 passes of 8 lanes; same with 16-byte chunks modulo 128 bytes.
"""

import collections
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "causal_self_attention_flashattention_amd", "csrc")
PROFILE = os.path.join(ROOT, "profiles", "lds_banks.txt")

FORMS = {"direct16": 0, "trans8x2": 1, "store16": 2, "trans16x2": 3}
KINDS = {"padded": 0, "skewed": 1, "skew_tr": 2, "shift16": 3}


@pytest.fixture(scope="module")
def lds_map(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path_factory.mktemp("lds") / "lds_map")
    subprocess.run([gxx, "-O1", "-std=c++17", "-I", CSRC, os.path.join(ROOT, "tests", "lds_map.cpp"), "-o", exe],
                   check=True, capture_output=True, text=True)
    return exe


def _parse(text):
    tiles, cur = {}, None
    for line in text.splitlines():
        f = line.split()
        if f[0] == "T":
            cur = {"kind": int(f[2]), "rb": int(f[3]), "rows": int(f[4]), "data": int(f[5]), "bytes": int(f[6]),
                   "cells": [], "D": [], "R": [], "S": [], "Q": []}
            tiles[f[1]] = cur
        elif f[0] == "P":
            cur = {"D": [], "R": [], "S": [], "Q": []}
            tiles["probe"] = cur
        elif f[0] == "C":
            cur["cells"].append((int(f[1]), int(f[2]), int(f[3])))
        elif f[0] == "D":
            cur["D"].append([int(x) for x in f[3:]])
        elif f[0] == "R":
            cur["R"].append([int(x) for x in f[5:]])
        elif f[0] == "Q":
            cur["Q"].append([int(x) for x in f[3:]])
        elif f[0] == "S":
            cur["S"].append([int(x) for x in f[4:]])
    return tiles


def _cycles(addrs, lanes, unit, window):
    """Cycles of one instruction: per pass of `lanes` lanes, the most distinct `unit`-byte accesses
    that share a slot modulo `window` bytes (inactive lanes: -1)."""
    total = 0
    for p in range(0, 64, lanes):
        grp = {a for a in addrs[p:p + lanes] if a >= 0}
        if not grp:
            continue
        slots = collections.Counter((a // unit) % (window // unit) for a in grp)
        total += max(slots.values())
    return total


def direct_cycles(a):
    return _cycles(a, 16, 16, 256)


def trans_cycles(a):
    return _cycles(a, 32, 8, 256)


def store_cycles(a):
    return _cycles(a, 8, 16, 128)


@pytest.fixture(scope="module")
def tiles(lds_map):
    return _parse(subprocess.run([lds_map], check=True, capture_output=True, text=True).stdout)


def test_layouts_are_injective_and_in_bounds(tiles):
    for name, t in tiles.items():
        seen = {}
        for r, b, off in t["cells"]:
            assert off % 16 == 0, (name, r, b, off)
            assert 0 <= off and off + 16 <= t["bytes"], (name, r, b, off, t["bytes"])
            assert off not in seen, (name, (r, b), seen.get(off))
            seen[off] = (r, b)
        # every instruction's lanes address cells of the tile
        cells = {off for _, _, off in t["cells"]}
        for a in t["D"]:
            assert all(x - x % 16 in cells for x in a), name
        for a in t["R"] + t["Q"]:
            assert all(x - x % 16 in cells for x in a), name
        for a in t["S"]:
            assert all(x in cells for x in a if x >= 0), name


# Tiles whose every read is conflict-free in the kernels (the stage tiles at d = 64 and 128 are read
# both as operands and transposed; forward K tiles only as operands; forward V tiles only
# transposed, conflict-free from d = 64 up).
CONFLICT_FREE_DIRECT = ["stage_d64", "stage_d128", "stage_d80", "fwdK_d16", "fwdK_d32", "fwdK_d64", "fwdK_d80",
                        "fwdK_d128", "stage_d16", "stage_d32"]
CONFLICT_FREE_TRANS = ["stage_d64", "stage_d128", "fwdV_d64", "fwdV_d80", "fwdV_d128"]


@pytest.mark.parametrize("name", CONFLICT_FREE_DIRECT)
def test_operand_reads_conflict_free(tiles, name):
    t = tiles[name]
    assert t["D"]
    assert all(direct_cycles(a) == 4 for a in t["D"]), name


@pytest.mark.parametrize("name", CONFLICT_FREE_TRANS)
def test_transposing_reads_conflict_free(tiles, name):
    t = tiles[name]
    assert t["R"]
    assert all(trans_cycles(a) == 2 for a in t["R"]), name


def test_sixteen_column_reads(tiles):
    """The 16-column transposing reads of the forward's last 16 V columns at d = 80 (rows 16 apart in
    one pass, which the kShift16 rows separate) are conflict-free; each lane's 8 bytes lie in one
    row's data."""
    t = tiles["fwdV_d80"]
    assert len(t["Q"]) == 4 and len(t["R"]) == 16
    assert all(trans_cycles(a) == 2 for a in t["Q"])
    # with plain padded rows of the same pitch the same reads conflict 2-way
    rb = t["rb"]
    flat = [[(x // rb) * rb + (x % rb if (x // rb) % 32 < 16 else x % rb - 32) for x in a] for a in t["Q"]]
    assert all(trans_cycles(a) == 4 for a in flat)


def test_known_conflicts_d80_and_small_dims(tiles):
    """The remaining conflicted forms, pinned as they are: the d = 80 stage tile's transposing reads,
    32- and 16-column (padded rows: 2-way), and the stores of 160-byte rows (d = 80), which straddle
    the 8-lane store passes."""
    assert all(trans_cycles(a) == 4 for a in tiles["stage_d80"]["R"])
    assert len(tiles["stage_d80"]["Q"]) == 4
    assert all(trans_cycles(a) == 4 for a in tiles["stage_d80"]["Q"])
    st = [store_cycles(a) for a in tiles["stage_d80"]["S"]]
    assert max(st) > 8
    for name in ("stage_d64", "stage_d128", "fwdK_d64", "fwdK_d128", "fwdV_d64", "fwdV_d128"):
        assert all(store_cycles(a) == 8 for a in tiles[name]["S"]), name


def test_skewed_layouts_pack_tightly(tiles):
    # skewed stage rows cost no more LDS than the padded rows they replace (to within 2%), and the
    # forward's d = 64 V tile no more than its padded rows
    assert tiles["stage_d128"]["bytes"] <= 1.02 * 64 * 304
    assert tiles["stage_d64"]["bytes"] <= 1.03 * 64 * 144
    assert tiles["fwdV_d64"]["bytes"] <= 64 * 144


def _profile_rows():
    rows = []
    for line in open(PROFILE):
        m = re.match(r"(.+?)\s+(direct16|trans8x2|store16|trans16x2)\s+(padded|skewed|skew_tr|shift16)\s+(\d+)\s+(\d+)\s+"
                     r"[\d.]+\s+[\d.]+\s+"
                     r"([\d.]+)\s+([\d.]+)\s*$", line)
        if m:
            tile, form, kind, rb, db, conf, cyc = m.groups()
            rows.append((tile.strip(), form, kind, int(rb), int(db), float(conf), float(cyc)))
    return rows


def test_bank_model_matches_measured_probe_counters(lds_map):
    """The model's cycles per instruction equal the measured SQ_LDS_IDX_ACTIVE / SQ_INSTS_LDS of every
    microbenchmark pattern (to 1%), including the conflicted ones (2-way and 4-way reads, the
    straddling stores)."""
    rows = _profile_rows()
    assert len(rows) >= 20
    for tile, form, kind, rb, db, conf, cyc in rows:
        out = subprocess.run([lds_map, "probe", str(FORMS[form]), str(KINDS[kind]), str(rb), str(db)], check=True,
                             capture_output=True, text=True).stdout
        t = _parse(out)["probe"]
        if form == "direct16":
            model = [direct_cycles(a) for a in t["D"]]
        elif form == "trans8x2":
            model = [trans_cycles(a) for a in t["R"]]
        elif form == "trans16x2":
            model = [trans_cycles(a) for a in t["Q"]]
        else:
            model = [store_cycles(a) for a in t["S"]]
        got = sum(model) / len(model)
        assert abs(got - cyc) <= 0.01 * cyc, (tile, form, kind, rb, db, got, cyc)
        ideal = {"direct16": 4, "trans8x2": 2, "store16": 8, "trans16x2": 2}[form]
        assert abs((got - ideal) / got - conf) <= 0.01, (tile, form, got, conf)
