"""Pins for the CPU oracle (no GPU).

None of the expected values here come from the oracle itself or from the GPU
library.  They come from: hand-worked window starts (tests/golden), a search
over all candidate intervals instead of the clamp formula, dense attention
with an explicit mask (numpy, float64), torch's dense SDPA when the window
covers the grid, and closed forms (K=1 gives v, q=0 gives the window mean,
constant v gives the constant) plus symmetry invariants.

Page: ROCm/aiter PR "Add 3D neighborhood flash attention (na3d_flash)",
Motivation (each token attends to its KT x KH x KW neighbours) and Technical
Details (inward border shift, exactly KT*KH*KW keys per window; Q pre-scaled).
"""
import itertools
import os

import numpy as np
import pytest
import torch

from na3d_inputs import WORKLOADS, make_inputs, workload_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "window_starts.txt")


# ---------------------------------------------------------------- helpers
def searched_start(i, K, L):
    """Window start found by search: among all K-long intervals [s, s+K) that
    fit in [0, L), the one whose K//2-th key is nearest to i.  Consecutive s
    give consecutive offsets, so the minimiser is unique."""
    best = None
    for s in range(0, L - K + 1):
        d = abs(s + K // 2 - i)
        if best is None or d < best[0]:
            best = (d, s)
    return best[1]


def axis_mask(L, K):
    m = np.zeros((L, L), dtype=bool)
    for i in range(L):
        s = searched_start(i, K, L)
        m[i, s:s + K] = True
    return m


def f64(t):
    return t.to(torch.float64).numpy()


def dense_masked(q, k, v, ks):
    """softmax(Q K^T + log M) V per (batch, head), float64, M explicit."""
    q, k, v = f64(q), f64(k), f64(v)
    B, T, H, W, NH, HD = q.shape
    mt, mh, mw = axis_mask(T, ks[0]), axis_mask(H, ks[1]), axis_mask(W, ks[2])
    M = (mt[:, None, None, :, None, None] & mh[None, :, None, None, :, None]
         & mw[None, None, :, None, None, :]).reshape(T * H * W, T * H * W)
    out = np.empty_like(q)
    N = T * H * W
    for b in range(B):
        for n in range(NH):
            Q = q[b, ..., n, :].reshape(N, HD)
            Kt = k[b, ..., n, :].reshape(N, HD)
            V = v[b, ..., n, :].reshape(N, HD)
            S = Q @ Kt.T
            S = np.where(M, S, -np.inf)
            S = S - S.max(axis=1, keepdims=True)
            P = np.exp(S)
            P /= P.sum(axis=1, keepdims=True)
            out[b, ..., n, :] = (P @ V).reshape(T, H, W, HD)
    return out, M


def read_golden():
    rows = []
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            lhs, rhs = line.split(":")
            L, K = (int(x) for x in lhs.split())
            rows.append((L, K, [int(x) for x in rhs.split()]))
    return rows


# ---------------------------------------------------------------- window rule
def test_golden_window_starts(oracle_mod):
    rows = read_golden()
    assert len(rows) >= 10
    for L, K, starts in rows:
        assert len(starts) == L, (L, K)
        got = [oracle_mod.window_start(i, K, L) for i in range(L)]
        assert got == starts, (L, K, got)


def test_window_start_matches_interval_search(oracle_mod):
    for L in range(1, 21):
        for K in range(1, L + 1):
            for i in range(L):
                s = oracle_mod.window_start(i, K, L)
                assert s == searched_start(i, K, L), (i, K, L)
                # every window lies inside the axis, holds K keys and contains i
                assert 0 <= s <= L - K and s <= i < s + K


def test_window_start_rejects_undefined(oracle_mod):
    assert oracle_mod.window_start(0, 0, 5) == -1
    assert oracle_mod.window_start(0, 6, 5) == -1
    assert oracle_mod.window_start(5, 3, 5) == -1
    assert oracle_mod.window_start(-1, 3, 5) == -1


# ---------------------------------------------------------------- brute force
BRUTE_CASES = []
for ks in [(1, 1, 1), (3, 3, 3), (3, 5, 5), (5, 3, 1), (1, 5, 3), (2, 4, 3)]:
    for extra in [(0, 0, 0), (1, 2, 3), (3, 1, 0)]:
        grid = tuple(k + e for k, e in zip(ks, extra))
        BRUTE_CASES.append((grid, ks))


@pytest.mark.parametrize("grid,ks", BRUTE_CASES)
@pytest.mark.parametrize("hd", [8, 32])
def test_oracle_vs_dense_masked(oracle_mod, grid, ks, hd):
    T, H, W = grid
    shape = (2, T, H, W, 2, hd)
    q, k, v = make_inputs(shape, seed=100 + sum(grid) * 7 + hd, device="cpu")
    ref, M = dense_masked(q, k, v, ks)
    # the mask has exactly KT*KH*KW keys per query
    assert (M.sum(axis=1) == ks[0] * ks[1] * ks[2]).all()
    got = oracle_mod.fwd(q, k, v, ks)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_oracle_vs_dense_masked_tiny_workload(oracle_mod):
    w = WORKLOADS["tiny"]
    q, k, v = workload_inputs("tiny")
    ref, _ = dense_masked(q, k, v, w.window)
    got = oracle_mod.fwd(q, k, v, w.window)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_weights_match_dense_masked_in_window_order(oracle_mod):
    """Every weight row equals the row of the dense masked softmax P (numpy,
    float64, mask from the interval search) read at the window's keys in
    (dt, dh, dw) lexicographic order: pins both the values and their order."""
    shape, ks = (1, 4, 5, 6, 2, 8), (3, 3, 5)
    q, k, v = make_inputs(shape, seed=8)
    wts, _ = oracle_mod.weights(q, k, v, ks)
    qq, kk = f64(q), f64(k)
    B, T, H, W, NH, HD = shape
    mt, mh, mw = axis_mask(T, ks[0]), axis_mask(H, ks[1]), axis_mask(W, ks[2])
    M = (mt[:, None, None, :, None, None] & mh[None, :, None, None, :, None]
         & mw[None, None, :, None, None, :]).reshape(T * H * W, T * H * W)
    N = T * H * W
    flat = lambda t, h, w: (t * H + h) * W + w
    for n in range(NH):
        S = qq[0, ..., n, :].reshape(N, HD) @ kk[0, ..., n, :].reshape(N, HD).T
        S = np.where(M, S, -np.inf)
        P = np.exp(S - S.max(axis=1, keepdims=True))
        P /= P.sum(axis=1, keepdims=True)
        for t, h, w in itertools.product(range(T), range(H), range(W)):
            st, sh, sw = (searched_start(t, ks[0], T), searched_start(h, ks[1], H),
                          searched_start(w, ks[2], W))
            keys = [flat(st + a, sh + b, sw + c) for a in range(ks[0])
                    for b in range(ks[1]) for c in range(ks[2])]
            np.testing.assert_allclose(wts[0, t, h, w, n], P[flat(t, h, w), keys],
                                       rtol=0, atol=1e-12)


def test_weights_rows_and_starts(oracle_mod):
    shape, ks = (1, 4, 6, 7, 2, 16), (3, 5, 5)
    q, k, v = make_inputs(shape, seed=7)
    wts, starts = oracle_mod.weights(q, k, v, ks)
    assert wts.shape == shape[:5] + (75,)
    np.testing.assert_allclose(wts.sum(axis=-1), 1.0, rtol=0, atol=1e-12)
    assert (wts > 0).all()
    B, T, H, W, NH, _ = shape
    for t, h, w in itertools.product(range(T), range(H), range(W)):
        exp = (searched_start(t, 3, T), searched_start(h, 5, H), searched_start(w, 5, W))
        assert tuple(starts[0, t, h, w, 0]) == exp


# ---------------------------------------------------------------- closed forms
def test_window_equal_to_grid_is_dense_attention(oracle_mod):
    shape = (2, 3, 4, 5, 3, 16)
    q, k, v = make_inputs(shape, seed=11)
    got = oracle_mod.fwd(q, k, v, (3, 4, 5))
    B, T, H, W, NH, HD = shape

    def heads(x):  # (B,T,H,W,NH,HD) -> (B,NH,N,HD) float64
        return x.to(torch.float64).reshape(B, T * H * W, NH, HD).permute(0, 2, 1, 3)

    ref = torch.nn.functional.scaled_dot_product_attention(
        heads(q), heads(k), heads(v), scale=1.0)
    ref = ref.permute(0, 2, 1, 3).reshape(shape).numpy()
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_unit_window_returns_v_exactly(oracle_mod):
    shape = (1, 3, 5, 6, 2, 32)
    q, k, v = make_inputs(shape, seed=12)
    got = oracle_mod.fwd(q, k, v, (1, 1, 1))
    np.testing.assert_array_equal(got, f64(v))


def test_zero_query_gives_window_mean(oracle_mod):
    shape, ks = (1, 5, 6, 9, 2, 8), (3, 3, 5)
    _, k, v = make_inputs(shape, seed=13)
    q = torch.zeros(shape, dtype=torch.bfloat16)
    got = oracle_mod.fwd(q, k, v, ks)
    vv = f64(v)
    B, T, H, W, NH, HD = shape
    for t, h, w in itertools.product(range(T), range(H), range(W)):
        st, sh, sw = (searched_start(t, ks[0], T), searched_start(h, ks[1], H),
                      searched_start(w, ks[2], W))
        box = vv[0, st:st + ks[0], sh:sh + ks[1], sw:sw + ks[2]]
        np.testing.assert_allclose(got[0, t, h, w], box.mean(axis=(0, 1, 2)),
                                   rtol=0, atol=1e-12)


def test_constant_v_gives_constant(oracle_mod):
    shape, ks = (1, 4, 6, 6, 2, 16), (3, 5, 3)
    q, k, _ = make_inputs(shape, seed=14)
    v = torch.full(shape, 1.5, dtype=torch.bfloat16)
    got = oracle_mod.fwd(q, k, v, ks)
    np.testing.assert_allclose(got, 1.5, rtol=0, atol=1e-12)


def test_dominant_key_is_selected(oracle_mod):
    """A query aligned with exactly one key of its window (score 40 vs 0)
    takes that key's v: checks which key index feeds which output."""
    T, H, W, HD = 3, 5, 7, 16
    ks = (3, 3, 3)
    q = torch.zeros((1, T, H, W, 1, HD), dtype=torch.bfloat16)
    k = torch.zeros_like(q)
    v = torch.arange(T * H * W * HD, dtype=torch.float32).reshape(1, T, H, W, 1, HD)
    v = (v % 97).to(torch.bfloat16)
    qt, qh, qw = 1, 4, 0  # high-h border, low-w border
    key = (2, 2, 2)       # inside the shifted window [0,3)x[2,5)x[0,3)
    q[0, qt, qh, qw, 0, 0] = 8.0
    k[0, key[0], key[1], key[2], 0, 0] = 5.0
    got = oracle_mod.fwd(q, k, v, ks)
    np.testing.assert_allclose(got[0, qt, qh, qw, 0], f64(v)[0, key[0], key[1], key[2], 0],
                               rtol=0, atol=1e-12 + 1e-15 * 97 * 27)


def test_extreme_scores_stay_finite(oracle_mod):
    """Keys with scores of +-1000 (exp of them overflows or underflows any
    float format without the max subtracted): every output stays finite and
    matches the dense masked softmax, and a query whose window holds the +1000
    key returns that key's v exactly (every other weight is e^-1000 = 0)."""
    from na3d_inputs import make_spike_inputs
    shape, ks = (1, 4, 6, 7, 2, 16), (3, 3, 5)
    spike = (1, 2, 3)
    q, k, v = make_spike_inputs(shape, 5, [spike + (1000,), (3, 5, 6, -1000)])
    got = oracle_mod.fwd(q, k, v, ks)
    assert np.isfinite(got).all()
    ref, M = dense_masked(q, k, v, ks)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)
    T, H, W = shape[1:4]
    sid = (spike[0] * H + spike[1]) * W + spike[2]
    hits = 0
    for t, h, w in itertools.product(range(T), range(H), range(W)):
        if M[(t * H + h) * W + w, sid]:
            np.testing.assert_array_equal(got[0, t, h, w], f64(v)[0, spike[0], spike[1], spike[2]])
            hits += 1
    assert 0 < hits < T * H * W


# ---------------------------------------------------------------- invariants
@pytest.mark.parametrize("axis", [1, 2, 3])
def test_flip_equivariance_odd_window(oracle_mod, axis):
    shape, ks = (1, 5, 6, 7, 2, 16), (3, 5, 3)
    q, k, v = make_inputs(shape, seed=20 + axis)
    base = oracle_mod.fwd(q, k, v, ks)
    fl = oracle_mod.fwd(q.flip(axis), k.flip(axis), v.flip(axis), ks)
    np.testing.assert_allclose(np.flip(fl, axis=axis), base, rtol=0, atol=1e-12)


def test_head_and_batch_permutation(oracle_mod):
    shape, ks = (3, 3, 5, 5, 4, 8), (3, 3, 3)
    q, k, v = make_inputs(shape, seed=30)
    base = oracle_mod.fwd(q, k, v, ks)
    hp, bp = [2, 0, 3, 1], [1, 2, 0]
    got = oracle_mod.fwd(q[bp][..., hp, :], k[bp][..., hp, :], v[bp][..., hp, :], ks)
    np.testing.assert_array_equal(got, base[bp][..., hp, :])


def test_interior_translation_equivariance(oracle_mod):
    shape, ks = (1, 3, 4, 12, 1, 8), (3, 3, 3)
    q, k, v = make_inputs(shape, seed=31)
    base = oracle_mod.fwd(q, k, v, ks)
    rolled = oracle_mod.fwd(q.roll(1, 3), k.roll(1, 3), v.roll(1, 3), ks)
    W = shape[3]
    for w in range(1, W - 2):  # window of w and of w+1 (rolled) stay unclamped
        np.testing.assert_array_equal(rolled[:, :, :, w + 1], base[:, :, :, w])


def test_points_match_full_grid(oracle_mod):
    shape, ks = (2, 4, 6, 5, 3, 16), (3, 5, 3)
    q, k, v = make_inputs(shape, seed=32)
    full = oracle_mod.fwd(q, k, v, ks)
    rng = np.random.default_rng(0)
    pts = np.stack([rng.integers(0, s, 40) for s in shape[:5]], axis=1)
    got = oracle_mod.fwd_points(q, k, v, ks, pts)
    for p, row in zip(pts, got):
        np.testing.assert_array_equal(row, full[tuple(p)])


def test_oracle_rejects_bad_arguments(oracle_mod):
    q, k, v = make_inputs((1, 2, 3, 4, 1, 8), seed=1)
    with pytest.raises(ValueError):
        oracle_mod.fwd(q, k, v, (3, 3, 3))  # KT > T
    with pytest.raises(ValueError):
        oracle_mod.fwd(q, k, v, (1, 0, 1))
    with pytest.raises(ValueError):
        oracle_mod.fwd_points(q, k, v, (1, 1, 1), [[0, 0, 0, 4, 0]])


def test_thread_count_does_not_change_result(oracle_mod):
    shape, ks = (1, 4, 8, 8, 2, 32), (3, 5, 5)
    q, k, v = make_inputs(shape, seed=33)
    a = oracle_mod.fwd(q, k, v, ks, nthreads=1)
    b = oracle_mod.fwd(q, k, v, ks, nthreads=4)
    np.testing.assert_array_equal(a, b)
