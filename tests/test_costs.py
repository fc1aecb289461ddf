"""Verify-cost table: interpolation and tree sizing on the host; one tiny measured sweep on the GPU."""
import math

import pytest

from draft_tree_verification_amd.costs import CostRow, VerifyCostTable, choose_nodes


def _table():
    rows = []
    for n in (4, 16):
        for b in (1, 8, 64):
            for L in (1024, 4096, 16384):
                # a cost model the interpolation must reproduce at the grid points
                rows.append(CostRow(b, n, L, 10.0 + 0.05 * b * b * n + 0.001 * b * L, 5.0, 2 * b * L * 8 * 128 * 2))
    return VerifyCostTable(rows)


def test_interpolation_exact_at_grid_and_between():
    t = _table()
    for r in t.rows:
        assert t.cost_us(r.batch, r.nodes, r.prefix) == pytest.approx(r.step_us)
    # linear in batch between 8 and 64 at a grid prefix
    c8, c64 = t.cost_us(8, 16, 4096), t.cost_us(64, 16, 4096)
    assert t.cost_us(36, 16, 4096) == pytest.approx((c8 + c64) / 2)
    # linear in log(prefix) between 1024 and 4096 (2048 is the log midpoint)
    a, b = t.cost_us(8, 4, 1024), t.cost_us(8, 4, 4096)
    assert t.cost_us(8, 4, 2048) == pytest.approx((a + b) / 2)
    # clamped outside the grid
    assert t.cost_us(512, 4, 1 << 20) == pytest.approx(t.cost_us(64, 4, 16384))
    with pytest.raises(KeyError):
        t.cost_us(8, 7, 4096)


def test_json_round_trip_and_markdown():
    t = _table()
    t2 = VerifyCostTable.from_json(t.to_json())
    assert [r.step_us for r in t2.rows] == [r.step_us for r in t.rows]
    md = t.markdown()
    assert md.count("\n") == len(t.rows) + 1 and "tree tokens/s" in md


def test_choose_nodes_trades_accepted_tokens_against_cost():
    t = _table()
    acc = {4: 2.5, 16: 3.9}.get
    # free drafting: at batch 1 the bigger tree wins; at batch 64 its verify cost does not pay off
    assert choose_nodes(t, 1, 4096, acc, lambda b, n: 0.0) == 16
    assert choose_nodes(t, 64, 16384, acc, lambda b, n: 0.0) == 4
    # an expensive drafter per node shifts the choice to the small tree
    assert choose_nodes(t, 1, 4096, acc, lambda b, n: 100.0 * n) == 4


@pytest.mark.gpu
def test_measured_sweep_small():
    from draft_tree_verification_amd import costs
    t = costs.sweep([1, 4], [4, 16], [512], iters=5, log=lambda s: print(s, flush=True))
    assert len(t.rows) == 4
    for r in t.rows:
        assert 0 < r.attention_us < r.step_us < 1e4 and math.isfinite(r.tree_tokens_per_s)
    assert t.cost_us(2, 16, 512) > 0


def test_packaged_mi355x_profile():
    """The shipped table covers the default grid and grows with the work it measures."""
    t = VerifyCostTable.packaged("mi355x")
    assert t.nodes_measured() == [4, 8, 16, 32, 64]
    assert len(t.rows) > 100 and all(r.step_us > r.attention_us > 0 for r in t.rows)
    assert t.cost_us(512, 4, 4096) > t.cost_us(64, 4, 4096) > t.cost_us(1, 4, 4096)
    assert t.cost_us(8, 16, 16384) > t.cost_us(8, 16, 1024)
