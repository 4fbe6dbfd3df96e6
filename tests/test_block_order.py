"""Host-side check of the order in which workgroups take work items (csrc/block_order.h), no GPU.

The kernels map block index b to item h * nranks + r (head h, rank r; ranks heaviest first) either
rank-major or XCD-aware.  Blocks reach the 8 XCDs round-robin (XCD b % 8, in order b / 8 there).
Checked for head counts and rank counts of the workloads and of the parity tests: both maps are
bijections onto the items with -1 past the end; each XCD takes its items in non-decreasing rank
(heaviest first); under the XCD-aware map each XCD receives the same number of items in every period
of the rank split (balanced causal work) and every head stays on at most 8 / (nheads mod 8) XCDs
(whole heads on one).
"""

import collections
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "causal_self_attention_flashattention_amd", "csrc")
NX = 8

# (B*H, ranks): the workloads' launches (forward: query tiles of 256 rows at d = 128 and 128 below;
# dQ likewise; dK/dV: key tiles of 256 or 128) and the head counts of the parity tests
CASES = [(36, 64), (36, 128), (80, 32), (80, 16), (128, 16), (48, 4), (36, 8), (12, 8), (5, 8), (7, 16), (9, 8),
         (3, 8), (1, 8), (2, 4), (6, 4), (36, 63), (10, 3), (4, 1), (72, 64), (40, 32)]


@pytest.fixture(scope="module")
def block_map(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path_factory.mktemp("bo") / "block_order_map")
    subprocess.run([gxx, "-O1", "-std=c++17", "-I", CSRC, os.path.join(ROOT, "tests", "block_order_map.cpp"), "-o", exe],
                   check=True, capture_output=True, text=True)
    return exe


def _maps(exe, nheads, nranks):
    out = subprocess.run([exe, str(nheads), str(nranks)], check=True, capture_output=True, text=True).stdout
    rows = [tuple(int(x) for x in line.split()) for line in out.splitlines()]
    n = nheads * nranks
    assert [r[0] for r in rows] == list(range(n + 8))
    return [r[1] for r in rows], [r[2] for r in rows], n


def _check_order(items, n, nheads, nranks):
    assert sorted(items[:n]) == list(range(n)), "not a bijection onto the items"
    assert all(x == -1 for x in items[n:]), "blocks past the end must get -1"
    per_xcd = collections.defaultdict(list)
    for b in range(n):
        per_xcd[b % NX].append(items[b])
    rank_sets = []
    for x, its in per_xcd.items():
        ranks = [it % nranks for it in its]
        assert ranks == sorted(ranks), f"XCD {x} does not take its items heaviest first"
        rank_sets.append(collections.Counter(ranks))
    return per_xcd, rank_sets


@pytest.mark.parametrize("nheads,nranks", CASES)
def test_rank_major(block_map, nheads, nranks):
    rm, _, n = _maps(block_map, nheads, nranks)
    _check_order(rm, n, nheads, nranks)
    # blocks 0 .. nheads - 1 take rank 0 of every head
    assert sorted(rm[:min(n, nheads)]) == [h * nranks for h in range(min(n, nheads))]


@pytest.mark.parametrize("nheads,nranks", CASES)
def test_xcd_order(block_map, nheads, nranks):
    rm, xc, n = _maps(block_map, nheads, nranks)
    hq, hr = divmod(nheads, NX)
    period = NX // hr if hr and NX % hr == 0 else NX
    applies = hr != 0 and nranks % period == 0
    if not applies:
        assert xc == rm, "falls back to rank-major"
        return
    per_xcd, rank_sets = _check_order(xc, n, nheads, nranks)
    if n >= NX:
        # every XCD the same number of items in every period of `period` ranks, so the XCDs' causal
        # work differs only by rank offsets within a period
        per_period = [collections.Counter(r // period for r in c.elements()) for c in rank_sets]
        assert all(c == per_period[0] for c in per_period)
    xcds_of_head = collections.defaultdict(set)
    for b in range(n):
        xcds_of_head[xc[b] // nranks].add(b % NX)
    for h, xs in xcds_of_head.items():
        limit = 1 if h < NX * hq else period
        assert len(xs) <= limit, (h, sorted(xs))
    # each XCD sees its hq whole heads plus its share of the remaining ones
    for x, its in per_xcd.items():
        heads = {it // nranks for it in its}
        assert len(heads) <= hq + (1 if NX % hr == 0 else hr), (x, sorted(heads))


def test_fewer_heads_per_xcd_than_rank_major(block_map):
    """At 36 heads, rank-major order spreads every head over two XCDs and gives each XCD 9 heads;
    the XCD-aware order gives each XCD 5 (4 whole, half of one more)."""
    rm, xc, n = _maps(block_map, 36, 64)
    for items, expect in ((rm, 9), (xc, 5)):
        per = collections.defaultdict(set)
        for b in range(n):
            per[b % NX].add(items[b] // 64)
        assert {len(v) for v in per.values()} == {expect}
