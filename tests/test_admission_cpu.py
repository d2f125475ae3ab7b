"""IO-adaptive admission policy (pure host logic in libkvoff.so, no GPU):
thresholds, pinning order from both ends inward, the offload ceiling."""
import numpy as np
import pytest

import sparse_kv_cache_mean_amd as kv


def _plan(p, u, res):
    n = kv.kvoff_admission_plan(p, u, res)
    return n, np.flatnonzero(res).tolist()


def test_defaults_follow_the_guide():
    p = kv.kvoff_admission_defaults()
    assert (p.low, p.high, p.max_offload, p.step_layers) == (0.5, 0.85, 0.9, 2)
    assert p.max_resident == 2**31 - 1  # no HBM cap unless the caller sets one


def test_saturated_link_pins_first_and_last_layers_inward():
    p = kv.kvoff_admission_defaults()
    res = np.zeros(32, np.uint8)
    # from nothing, +2 gives 2, raised to the floor ceil(0.1 * 32) = 4
    assert _plan(p, 0.97, res) == (4, [0, 1, 30, 31])
    res[:] = 0
    p.step_layers = 2
    p.max_offload = 1.0  # no floor: watch the order alone
    assert _plan(p, 0.97, res) == (2, [0, 31])
    assert _plan(p, 0.97, res) == (4, [0, 1, 30, 31])
    assert _plan(p, 0.90, res) == (6, [0, 1, 2, 29, 30, 31])
    assert _plan(p, 0.70, res) == (6, [0, 1, 2, 29, 30, 31])  # inside the band: unchanged
    assert _plan(p, 0.30, res) == (4, [0, 1, 30, 31])          # released in reverse order
    assert _plan(p, 0.30, res) == (2, [0, 31])
    assert _plan(p, 0.30, res) == (0, [])


def test_offload_ceiling_keeps_a_floor_of_resident_layers():
    p = kv.kvoff_admission_defaults()  # at most 90% offloaded
    res = np.zeros(32, np.uint8)
    n, layers = _plan(p, 0.1, res)
    assert n == 4 and layers == [0, 1, 30, 31]  # ceil(0.1 * 32) = 4 stay resident
    res = np.zeros(10, np.uint8)
    assert _plan(p, 0.1, res)[0] == 1           # ceil(0.1 * 10) = 1
    res = np.ones(5, np.uint8)
    assert _plan(p, 0.99, res) == (5, [0, 1, 2, 3, 4])  # cannot exceed every layer


def test_odd_layer_count_meets_in_the_middle():
    p = kv.kvoff_admission_defaults()
    p.max_offload = 1.0
    p.step_layers = 1
    res = np.zeros(5, np.uint8)
    order = []
    for _ in range(5):
        before = set(np.flatnonzero(res).tolist())
        kv.kvoff_admission_plan(p, 0.99, res)
        order += sorted(set(np.flatnonzero(res).tolist()) - before)
    assert order == [0, 4, 1, 3, 2]


def test_hbm_budget_caps_residency_and_wins_over_the_floor():
    p = kv.kvoff_admission_defaults()
    p.max_resident = 3
    res = np.zeros(8, np.uint8)
    assert _plan(p, 0.99, res) == (2, [0, 7])
    assert _plan(p, 0.99, res) == (3, [0, 1, 7])   # +2 would be 4: capped at 3
    assert _plan(p, 0.99, res) == (3, [0, 1, 7])
    p.max_resident = 0                               # no HBM to spare
    res = np.zeros(32, np.uint8)
    assert _plan(p, 0.1, res) == (0, [])             # below the floor of 4: the budget wins


@pytest.mark.parametrize("bad", [dict(low=0.9, high=0.5), dict(max_offload=1.5), dict(step_layers=0),
                                 dict(max_resident=-1)])
def test_bad_policy_is_rejected(bad):
    p = kv.kvoff_admission_defaults()
    for k, v in bad.items():
        setattr(p, k, v)
    with pytest.raises(kv.KvoffError) as e:
        kv.kvoff_admission_plan(p, 0.5, np.zeros(4, np.uint8))
    assert e.value.status == kv.KVOFF_EINVAL
