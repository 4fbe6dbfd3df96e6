"""Host-side check of the operand orders behind the MFMA products that reduce over an accumulator's
rows (no GPU): the weights (or dS) taken straight from a 32x32 score accumulator as B operands, and
V^T (or dO^T, Q^T, K^T) read transposed from LDS as A operands, must walk the 32 keys of a block in
the same order.  The row maps come from the kernels' layout header (csrc/lds_layout.h) through
tests/lds_map.cpp; the lane layouts are gfx950's, as csrc/attn_device.h states them:

  * 32x32 accumulator: lane l, element e holds row 8 (e / 4) + 4 (l / 32) + e % 4, column l % 32;
    a bf16 fragment c (acc_frag) holds elements 8c .. 8c + 7;
  * ds_read_b64_tr_b16: in each group of 16 lanes, lane i receives element i % 4 of the 8-byte chunks
    read by lanes 4e + i / 4 (e < 4), as its slots e;
  * v_mfma_f32_32x32x16_bf16 A: lane l holds A[l % 32][8 (l / 32) + s]; B: B[8 (l / 32) + s][l % 32];
  * v_mfma_f32_16x16x32_bf16 A: lane l holds A[l % 16][8 (l / 16) + s]; B: B[8 (l / 16) + s][l % 16];
  * v_permlane16_swap(a, b) on rows of 16 lanes: a keeps rows 0 and 2 and takes b's rows 0 and 2 into
    its rows 1 and 3; b takes a's rows 1 and 3 into its rows 0 and 2 and keeps rows 1 and 3.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "causal_self_attention_flashattention_amd", "csrc")


@pytest.fixture(scope="module")
def rows(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path_factory.mktemp("rows") / "lds_map")
    subprocess.run([gxx, "-O1", "-std=c++17", "-I", CSRC, os.path.join(ROOT, "tests", "lds_map.cpp"), "-o", exe],
                   check=True, capture_output=True, text=True)
    out = subprocess.run([exe, "rows"], check=True, capture_output=True, text=True).stdout
    w16, w32 = {}, {}
    for line in out.splitlines():
        f = line.split()
        if f[0] == "W16":
            w16[int(f[1]), int(f[2])] = (int(f[3]), int(f[4]))
        elif f[0] == "W32":
            w32[int(f[1]), int(f[2]), int(f[3])] = int(f[4])
    return w16, w32


def acc_key(e, lane):
    """Accumulator row (key within the 32-key block) of element e in `lane`."""
    return 8 * (e // 4) + 4 * (lane // 32) + e % 4


def tr_source(lane, e):
    """Lane whose 8-byte chunk supplies slot e of `lane` in a transposing read, and the element."""
    g, i = lane // 16, lane % 16
    return 16 * g + 4 * e + i // 4, i % 4


def test_32wide_products_walk_keys_in_accumulator_order(rows):
    _, w32 = rows
    for c in range(2):
        for lane in range(64):
            for s in range(8):
                h, e = s // 4, s % 4
                src, _ = tr_source(lane, e)
                a_key = w32[src, c, h]            # key row of the A operand's slot s
                b_key = acc_key(8 * c + s, lane)  # fragment c, slot s: accumulator element 8c + s
                assert a_key == b_key, (c, lane, s, a_key, b_key)


def swap16(a, b):
    """v_permlane16_swap on per-lane values a, b (lists of 64): the two results."""
    x, y = list(a), list(b)
    for lane in range(64):
        r = lane // 16
        if r in (1, 3):
            x[lane] = b[lane - 16]
            y[lane - 16] = a[lane]
    return x, y


def test_16wide_products_walk_the_same_keys(rows):
    w16, _ = rows
    # per lane and slot: (query column, key) of the bf16 weights of fragments 0 and 1
    frag = [[[(lane % 32, acc_key(8 * c + s, lane)) for s in range(8)] for lane in range(64)] for c in range(2)]
    lo, hi = swap16(frag[0], frag[1])
    for lane in range(64):
        g, i = lane // 16, lane % 16
        for s in range(8):
            h, e = s // 4, s % 4
            src, elem = tr_source(lane, e)
            a_row, a_byte = w16[src, h]
            # A operand: V^T row = the column this lane's slots carry, reduction index = the key
            assert a_byte // 2 + elem == i, (lane, s)
            assert lo[lane][s] == (i, a_row), (lane, s, lo[lane][s], a_row)
            assert hi[lane][s] == (16 + i, a_row), (lane, s, hi[lane][s], a_row)
    # the 32 (lane group, slot) positions of the reduction take each key of the block once
    keys = sorted(w16[16 * g + 4 * (s % 4), s // 4][0] for g in range(4) for s in range(8))
    assert keys == list(range(32))


def test_split16_moves_per_query_factors(rows):
    # a factor held per query column (lane l: query l % 32) reaches the 16-wide accumulators' lanes
    x = [lane % 32 for lane in range(64)]
    lo, hi = swap16(x, x)
    assert lo == [lane % 16 for lane in range(64)]
    assert hi == [16 + lane % 16 for lane in range(64)]
