"""The encoder's copy-choice table (csrc/cp_encode_copies.h) is what its
generator writes, and each choice names a copy that exists. The choices only
decide which of several identical copies of a branch cost a thread reads, so
they cannot change an encoding (the GPU encoder tests check records bit for
bit); this pins the table to its stated construction."""
from __future__ import annotations

import re

from trellis_coded_row_amd import gen_encode_copies as gen


def test_header_is_the_generator_output():
    with open(gen.HEADER) as fh:
        assert fh.read() == gen.render(), "regenerate with python -m trellis_coded_row_amd.gen_encode_copies"


def cycles(units) -> int:
    """LDS cycles of 16 lanes' 16-byte loads: distinct units per bank group
    (unit mod 16), at most."""
    groups = [u % 16 for u in units]
    return max(groups.count(g) for g in set(groups))


def test_lane_groups_partition_a_wave():
    groups = gen.lane_groups()
    assert sorted(len(g) for g in groups) == [16] * 4
    assert sorted(lane for g in groups for lane in g) == list(range(64))
    # the groups measured for lanes 0 and 5
    assert [0, 1, 2, 3, 12, 13, 14, 15, 20, 21, 22, 23, 24, 25, 26, 27] in groups
    assert [4, 5, 6, 7, 8, 9, 10, 11, 16, 17, 18, 19, 28, 29, 30, 31] in groups


def test_choices_spread_the_gathers():
    tabs = gen.tables()
    for kv, (packed, mean_cycles) in tabs.items():
        nt, cc = gen.CONFIG[kv]
        bits = cc.bit_length() - 1
        keys = gen.thread_keys(kv, nt)
        assert len(packed) == nt and len(keys) * bits == 64
        for q, row in enumerate(keys):
            for lanes in ([w + lane for lane in g] for w in range(0, nt, 64) for g in gen.lane_groups()):
                units = {gen.unit(row[t], (packed[t] >> (bits * q)) & (cc - 1), cc) for t in lanes}
                # every unit inside the cost buffer of 1024 * cc doubles
                assert all(0 <= u < 512 * cc for u in units)
                # the matching is no worse than any fixed choice in the same
                # layout, e.g. copy = lane mod cc
                fixed = {gen.unit(row[t], t % cc, cc) for t in lanes}
                assert cycles(units) <= cycles(fixed), (kv, q, lanes[0])
        # with key k's copies side by side (unit k * cc + copy) and copy =
        # lane mod cc, the loads take 1.875 cycles per 16 lanes at kv 4 and 5
        assert mean_cycles < {4: 1.2, 5: 1.76}[kv]


def test_header_declares_one_table_per_kv():
    with open(gen.HEADER) as fh:
        text = fh.read()
    assert re.findall(r"kEncodeCopies(\d)\[(\d+)\]", text) == [("4", "1024"), ("5", "512")]
