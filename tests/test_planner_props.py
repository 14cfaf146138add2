"""Property tests of the host planner (no GPU): for random valid sizes the
plan exists, fits the hardware (LDS, threads) and covers the grid exactly
with its workgroups; batches are planned consistently."""
import math

from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import neighborhood_attention_amd as na

MAX_LDS = 160 * 1024


@st.composite
def problems(draw):
    B = draw(st.integers(1, 3))
    T = draw(st.integers(1, 40))
    H = draw(st.integers(1, 80))
    W = draw(st.integers(1, 200))
    NH = draw(st.integers(1, 16))
    HD = draw(st.sampled_from([16, 32, 64, 128, 256]))
    KT = draw(st.integers(1, min(T, 13)))
    KH = draw(st.integers(1, min(H, 13)))
    KW = draw(st.integers(1, min(W, 33)))
    return (B, T, H, W, NH, HD), (KT, KH, KW)


@settings(max_examples=300, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(problems())
def test_plan_fits_and_covers(prob):
    shape, ks = prob
    B, T, H, W, NH, HD = shape
    p = na.plan(shape, ks)
    assert p["family"] in (1, 2)
    assert 64 <= p["threads"] <= 1024 and p["threads"] % 64 == 0
    assert 0 < p["lds_bytes"] <= MAX_LDS
    tiles = B * NH * math.ceil(H / p["tile_h"]) * math.ceil(W / p["tile_w"])
    if p["family"] == 2:
        assert p["workgroups"] == tiles * p["runs"]
        assert 1 <= p["runs"]
        assert na.plan(shape, ks, 2, p["variant"], 0) == p      # the explicit form agrees
    else:
        assert p["workgroups"] == tiles * T
    # the general family can always run the sizes
    g = na.plan(shape, ks, 1, 0, 0)
    assert g["family"] == 1 and g["workgroups"] == B * NH * T * math.ceil(H / g["tile_h"]) * \
        math.ceil(W / g["tile_w"])


@settings(max_examples=150, deadline=None)
@given(st.lists(st.tuples(st.integers(1, 2), st.integers(3, 20), st.integers(7, 48),
                          st.integers(7, 64)), min_size=0, max_size=40),
       st.sampled_from([32, 64, 128]), st.integers(1, 8))
def test_batch_plan_is_consistent(dims, HD, NH):
    p = na.plan_batch(dims, NH, HD, (3, 7, 7))
    n = len(dims)
    assert 0 <= p["shared_tiles"] <= n
    solo = n - p["shared_tiles"]
    assert p["launches"] >= solo + math.ceil(p["shared_tiles"] / 16)
    if n:
        lead = max(range(n), key=lambda i: (dims[i][0] * dims[i][1] * dims[i][2] * dims[i][3], -i))
        single = na.plan(tuple(dims[lead]) + (NH, HD), (3, 7, 7))
        if single["family"] == 2:
            assert p["variant"] == single["variant"]
            assert p["shared_tiles"] >= 1
        else:
            assert p["shared_tiles"] == 0 and p["launches"] == n
    else:
        assert p == {"launches": 0, "variant": -1, "shared_tiles": 0, "workgroups": 0}
