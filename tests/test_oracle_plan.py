"""Pins of the oracle planner and its byte accounting against the pages."""
from decimal import ROUND_FLOOR, ROUND_HALF_UP, Decimal
from fractions import Fraction

import pytest

import workloads as W
from conftest import golden_rows
from oracle import plan as P


def _printed_matches(printed: str, exact: Fraction) -> bool:
    """The pages print some cells rounded and some truncated at the last printed digit."""
    d = Decimal(printed)
    q = Decimal(1).scaleb(d.as_tuple().exponent)
    x = Decimal(exact.numerator) / Decimal(exact.denominator)
    return d in (x.quantize(q, rounding=ROUND_HALF_UP), x.quantize(q, rounding=ROUND_FLOOR))


def _table1():
    rows = golden_rows("zero_dp_memory_table1.txt")
    header, body = rows[0], rows[1:]
    models = {"7.5B": 7_500_000_000, "128B": 128_000_000_000, "1T": 1_000_000_000_000}
    cells = []
    for r in body:
        n = int(r[0])
        for col, val in zip(header[1:], r[1:]):
            model, stage_name = col.split("_")
            stage = {"os": 1, "osg": 2, "osgp": 3}[stage_name]
            cells.append((models[model], n, stage, val))
    return cells


def test_table1_every_cell():
    """All 54 cells of Table 1 follow 4Psi+12Psi/N, 2Psi+14Psi/N and 16Psi/N (GB = 1e9 B)."""
    cells = _table1()
    assert len(cells) == 54
    bad = [(psi, n, s, v, float(P.model_state_bytes(psi, n, s) / 10**9))
           for psi, n, s, v in cells
           if not _printed_matches(v, P.model_state_bytes(psi, n, s) / 10**9)]
    assert not bad, bad


def test_table1_rejects_plausible_mistakes():
    """The table check is sharp: swapping the stage-1/2 optimizer-state factors, or
    forgetting the fp16 parameter term, breaks it."""
    cells = _table1()

    def wrong_swap(psi, n, s):
        psi, n = Fraction(psi), Fraction(n)
        return {1: 4 * psi + 14 * psi / n, 2: 2 * psi + 12 * psi / n, 3: 16 * psi / n}[s]

    def wrong_no_param(psi, n, s):
        psi, n = Fraction(psi), Fraction(n)
        return {1: 2 * psi + 12 * psi / n, 2: 14 * psi / n + 2 * psi, 3: 14 * psi / n}[s]

    for f in (wrong_swap, wrong_no_param):
        assert any(not _printed_matches(v, f(psi, n, s) / 10**9) for psi, n, s, v in cells)


def test_table2_max_model_size_mp1():
    rows = golden_rows("max_model_size_table2.txt")
    dev = Fraction(int(float(rows[0][1])))
    gpus = int(rows[1][1])
    for stage, printed in rows[3:]:
        per_param = P.model_state_bytes(1, gpus, int(stage))   # bytes per parameter
        psi_max_b = dev / per_param / 10**9                    # billions of parameters
        assert _printed_matches(printed.rstrip("B"), psi_max_b), (stage, printed, float(psi_max_b))


def test_worked_examples():
    for psi, world, stage, gb in golden_rows("worked_examples.txt"):
        exact = P.model_state_bytes(int(float(psi)), int(world), int(stage)) / 10**9
        assert _printed_matches(gb, exact), (psi, world, stage, gb, float(exact))


def test_optimizer_states_are_75_percent():
    """12 of the 16 bytes per parameter are optimizer state (explainer, "先算一笔账")."""
    psi = 7 * 10**9
    assert P.model_state_bytes(psi, 1, 0) == 112 * 10**9
    assert (P.model_state_bytes(psi, 1, 0) - 4 * psi) / P.model_state_bytes(psi, 1, 0) == Fraction(3, 4)


def test_toy_padding_and_state_bytes():
    """zero_check.py prints 57,636 B per rank vs 230,520 B unsharded on 4 ranks;
    only a ceil split of 19,210 over 4 with a zero pad gives 57,636."""
    rows = dict((r[0], r[1]) for r in golden_rows("toy_state_bytes.txt"))
    pl = P.make_plan(W.numels(W.toy_mlp()), int(rows["world"]))
    assert pl.psi == 19_210
    assert pl.shard_numel == 4_803 and pl.padded_numel == 19_212
    assert P.state_bytes(pl) == int(rows["per_rank_state_bytes"])
    assert 3 * 4 * pl.psi == int(rows["unsharded_state_bytes"])
    assert round((3 * 4 * pl.psi) / P.state_bytes(pl)) == 4
    segs = [P.rank_segments(pl, r) for r in range(4)]
    assert [s[0][3] for s in segs] == [4803, 4803, 4803, 4801]   # rank 3 holds the 2 pads


@pytest.mark.parametrize("name,S", [("toy_mlp_n4", 4_803), ("gpt2_1p5b_n8", 194_701_400),
                                    ("flat_7p5b_n64", 117_187_500), ("llama_7b_n8", 842_301_952),
                                    ("llama3_8b_n16_buckets", 501_891_328)])
def test_workload_shard_sizes(name, S):
    w = W.FULL[name]
    pl = P.make_plan(W.numels(w.tensors), w.world, w.bucket_cap)
    assert pl.shard_numel == S


def test_llama3_buckets_greedy_cap():
    w = W.FULL["llama3_8b_n16_buckets"]
    sizes = W.numels(w.tensors)
    pl = P.make_plan(sizes, w.world, w.bucket_cap)
    assert [b.n_tensors for b in pl.buckets] == [1, 22, 19, 19, 21, 22, 19, 19, 21, 22, 19, 19,
                                                  21, 22, 19, 5, 1]
    _check_invariants(pl, sizes, w.bucket_cap)


def _check_invariants(pl, sizes, cap):
    # buckets take the tensors in order, without gaps
    nxt = 0
    for b in pl.buckets:
        assert b.first_tensor == nxt
        nxt += b.n_tensors
        assert b.numel == sum(sizes[b.first_tensor:b.first_tensor + b.n_tensors])
        assert b.padded == pl.world * b.shard and b.shard * pl.world >= b.numel > (b.shard - 1) * pl.world
        if cap > 0:
            nonzero = sum(1 for n in sizes[b.first_tensor:b.first_tensor + b.n_tensors] if n > 0)
            assert b.numel <= cap or nonzero == 1
    assert nxt == len(sizes)
    if cap > 0:   # greedy: the next tensor would not have fit
        for b, b2 in zip(pl.buckets, pl.buckets[1:]):
            assert b.numel > 0 and b.numel + sizes[b2.first_tensor] > cap and sizes[b2.first_tensor] > 0
    # tensors tile each bucket's front, padding sits at its end
    for i, n in enumerate(sizes):
        b = pl.buckets[pl.tensor_bucket[i]]
        assert b.base <= pl.tensor_offset[i] and pl.tensor_offset[i] + n <= b.base + b.numel
    # rank pieces: each rank's local range is covered once, the gather buffer once overall
    covered = []
    for r in range(pl.world):
        segs = P.rank_segments(pl, r)
        local = 0
        for (goff, loff, ln, valid), b in zip(segs, pl.buckets):
            assert loff == local and ln == b.shard and 0 <= valid <= ln
            assert goff == b.base + r * b.shard
            assert valid == max(0, min(ln, b.numel - r * b.shard))
            covered.append((goff, goff + ln))
            local += ln
        assert local == pl.shard_numel
    covered.sort()
    assert covered[0][0] == 0 and covered[-1][1] == pl.padded_numel
    assert all(a[1] == b[0] for a, b in zip(covered, covered[1:]))


@pytest.mark.parametrize("sizes,world,cap", [
    ([3], 4, 0),                        # fewer elements than ranks: rank 3 is all padding
    ([5, 0, 7], 1, 0),                  # N = 1, a zero-size tensor
    ([8, 8], 4, 0),                     # divides exactly, no padding
    ([10, 30, 5, 5, 1], 3, 12),         # a tensor larger than the cap sits alone
    ([1] * 50, 7, 6),                   # many small buckets
    (W.numels(W.toy_mlp()), 4, 300),
    (W.numels(W.llama(3, 128, 2, 32, 448, 2000)), 16, 150_000),
])
def test_plan_invariants(sizes, world, cap):
    pl = P.make_plan(sizes, world, cap)
    _check_invariants(pl, sizes, cap)


def test_zero_size_tensors_never_make_an_empty_bucket():
    pl = P.make_plan([0, 5, 0, 0, 4, 0], 2, 3)
    assert [(b.first_tensor, b.n_tensors, b.numel) for b in pl.buckets] == [(0, 4, 5), (4, 2, 4)]
    assert all(b.shard > 0 for b in pl.buckets)
    _check_invariants(pl, [0, 5, 0, 0, 4, 0], 3)


def test_rank_all_padding():
    pl = P.make_plan([3], 4)
    assert pl.shard_numel == 1
    assert [P.rank_segments(pl, r)[0][3] for r in range(4)] == [1, 1, 1, 0]


def test_padded_accounting_equals_formula_without_padding():
    pl = P.make_plan([8, 8], 4)
    for s in range(4):
        assert P.padded_model_state_bytes(pl, s) == P.model_state_bytes(16, 4, s)
    pl = P.make_plan(W.numels(W.toy_mlp()), 4)
    assert P.padded_model_state_bytes(pl, 1) == 4 * 19_212 + 12 * 4_803


@pytest.mark.parametrize("bad", [dict(numels=[], world=2), dict(numels=[0, 0], world=2),
                                 dict(numels=[4], world=0), dict(numels=[-1, 5], world=2)])
def test_plan_rejects(bad):
    with pytest.raises(ValueError):
        P.make_plan(bad["numels"], bad["world"])
