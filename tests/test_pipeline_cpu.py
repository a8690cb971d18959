"""Host logic of the layer driver that needs no GPU: how k-means problems are
split into ranges that run as separate calls on separate streams."""
import oracle
from sparse_attention_video_head_amd.pipeline import _part_seed, _problem_parts


def test_problem_parts_cover_every_problem_once():
    for bh in range(1, 70):
        parts = _problem_parts(bh, True)
        assert parts[0][0] == 0 and parts[-1][1] == bh
        assert all(a[1] == b[0] for a, b in zip(parts, parts[1:]))
        for lo, hi in parts:
            assert lo == 0 or (lo & (lo - 1)) == 0 and hi - lo <= lo
    assert _problem_parts(24, False) == [(0, 24)]


def test_split_calls_draw_the_same_kmeanspp_numbers():
    """Problem i of a call on problems [lo, hi) with _part_seed(seed, lo) draws
    exactly the numbers problem lo + i draws in one call on every problem."""
    for bh in (2, 3, 24, 40):
        for lo, hi in _problem_parts(bh, True):
            for i in range(hi - lo):
                for pick in (0, 1, 77, 999, 4095):
                    assert (oracle.seeding_uniform(_part_seed(0x5EED0000 + 17, lo), i, pick)
                            == oracle.seeding_uniform(0x5EED0000 + 17, lo + i, pick))
