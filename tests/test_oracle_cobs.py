"""Pins of the second-order block statistic oracle (oracle.cobs).

The pages give no formula for the statistic (parity unpinned by the pages), so
these pin the reading against the mathematics it rests on: the block mean and
variance against closed forms and numpy, the first- and second-order terms of
the cumulant expansion of the block's log-mass against an exactly computed
mass, and the first-order selection against the block path's own oracle.
"""
import numpy as np
import pytest

import oracle
from oracle import SelectParams


def test_block_stats_closed_forms():
    d = 8
    L = 64 * 3 + 17                                   # the partial last block has no statistics
    K = np.zeros((L, d), dtype=np.float32)
    K[:64] = 1.5                                      # constant block
    K[64:128, 0] = np.arange(64)                      # ramp 0..63 in channel 0
    K[128:192, 1] = np.tile([2.0, -2.0], 32)          # two-point block: mean 0, variance 4
    mu, var = oracle.block_stats(K, L, "f32")
    assert mu.shape == var.shape == (3, d)
    assert np.all(mu[0] == 1.5) and np.all(var[0] == 0)
    assert mu[1, 0] == 31.5 and var[1, 0] == (64 * 64 - 1) / 12.0      # 341.25, exact
    assert np.all(var[1, 1:] == 0)
    assert mu[2, 1] == 0 and var[2, 1] == 4.0
    assert oracle.block_stats(K, 63, "f32")[0].shape == (0, d)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_block_stats_match_numpy_and_grow_by_prefix(dtype):
    rng = np.random.default_rng(1)
    K = rng.standard_normal((64 * 10, 16)).astype(np.float32) * 3 + 1
    mu, var = oracle.block_stats(K, 64 * 10, dtype)
    blocks = K.reshape(10, 64, 16).astype(np.float64)
    tol = 1e-5 if dtype == "f32" else 8e-3
    assert np.allclose(mu, blocks.mean(axis=1), rtol=tol, atol=tol)
    assert np.allclose(var, blocks.var(axis=1), rtol=tol, atol=tol)
    mu6, var6 = oracle.block_stats(K, 64 * 6 + 5, dtype)
    assert np.array_equal(mu6, mu[:6]) and np.array_equal(var6, var[:6])


def _exact_log_mass(q, K):
    z = K.astype(np.float64) @ q
    m = z.max()
    return m + np.log(np.exp(z - m).sum()) - np.log(64.0)


def test_expansion_orders_on_a_two_point_block():
    """Keys mu +- a e_0 (32 each): the exact log-mass is q.mu + log cosh(q_0 a).
    First order misses x^2 / 2 (x = q_0 a), second order only x^4 / 12 + ...:
    halving a divides the errors by 4 and by 16."""
    rng = np.random.default_rng(2)
    d = 8
    mu_true = rng.integers(-4, 5, d).astype(np.float32) / 4
    q = rng.standard_normal(d)
    q[0] = 1.0
    errs1, errs2 = [], []
    for k in range(2, 7):
        a = np.float32(2.0 ** -k)
        K = np.tile(mu_true, (64, 1))
        K[0::2, 0] += a
        K[1::2, 0] -= a
        mu, var = oracle.block_stats(K, 64, "f32")
        exact = _exact_log_mass(q, K)
        assert np.isclose(exact, q @ mu_true + np.log(np.cosh(q[0] * a)), rtol=0, atol=1e-12)
        e1 = oracle.cobs_log_mass(q[None], mu, var, order=1)[0, 0]
        e2 = oracle.cobs_log_mass(q[None], mu, var, order=2)[0, 0]
        errs1.append(exact - e1)
        errs2.append(exact - e2)
        x = q[0] * a
        # log cosh x = x^2/2 - x^4/12 + x^6/45 - ... (alternating, decreasing terms)
        assert abs(errs1[-1] - x * x / 2) <= x ** 4 / 12 * 1.001
        assert abs(errs2[-1] + x ** 4 / 12) <= x ** 6 / 45 * 1.001 + 1e-15
    r1 = np.array(errs1[:-1]) / np.array(errs1[1:])
    r2 = np.array(errs2[:-1]) / np.array(errs2[1:])
    assert np.all(np.diff(r1) > 0) and abs(r1[-1] - 4) < 2e-3      # second order in a
    assert abs(r2[-1] - 16) < 2e-2                                # fourth order in a


def test_constant_blocks_estimate_is_exact():
    rng = np.random.default_rng(3)
    d, nb = 16, 12
    w = rng.integers(-8, 9, (nb, d)).astype(np.float32) / 4    # block sums exact in fp32
    K = np.repeat(w, 64, axis=0)
    mu, var = oracle.block_stats(K, 64 * nb, "f32")
    q = rng.standard_normal((2, d))
    est = oracle.cobs_log_mass(q, mu, var, order=2)
    for h in range(2):
        for b in range(nb):
            assert np.isclose(est[h, b], _exact_log_mass(q[h], K[64 * b:64 * (b + 1)]),
                              rtol=0, atol=1e-12)


@pytest.mark.parametrize("seed", range(3))
def test_raw_selection_on_constant_blocks_equals_the_block_path(seed):
    """Constant blocks: zero variance, and every compressed entry inside a
    block is the block's key, so the COBS raw selection (either order) is the
    block path's Eq. 4 selection."""
    rng = np.random.default_rng(seed)
    nb, d = 40, 16
    L = 64 * nb - 20                                  # partial last block (local)
    w = rng.integers(-3, 4, (nb, d)).astype(np.float32)
    K = np.repeat(w, 64, axis=0)[:L]
    sel = rng.integers(-2, 3, (1, d)).astype(np.float32)
    mu, var = oracle.block_stats(K, L, "f32")
    Kc = oracle.compressed_keys(K, L, "f32")
    for k in (1, 5, 20, 50):
        p = SelectParams(top_k=k, n_init=1, n_local=2, score_mode=oracle.RAW_SUM)
        ref = oracle.select_blocks(sel, Kc, L, p)
        assert oracle.select_blocks_cobs(sel, mu, var, L, p, order=1) == ref
        assert oracle.select_blocks_cobs(sel, mu, var, L, p, order=2) == ref


def test_second_order_finds_high_spread_blocks_the_first_order_misses():
    """Blocks whose keys spread along q (same mean) hold more attention mass;
    only the second-order score sees them, and its selection captures more of
    the exact mass (oracle.quality)."""
    rng = np.random.default_rng(4)
    nb, d = 64, 32
    L = 64 * nb
    K = rng.standard_normal((L, d)).astype(np.float32) * 0.5
    q = rng.standard_normal(d)
    q /= np.linalg.norm(q)
    u = q.astype(np.float32)
    spread = [7, 19, 33, 48]
    for b in spread:
        K[64 * b:64 * (b + 1)] += np.tile([2.0, -2.0], 32)[:, None].astype(np.float32) * u
    mu, var = oracle.block_stats(K, L, "f32")
    p = SelectParams(top_k=4, n_init=1, n_local=2, score_mode=oracle.SOFTMAX_SUM)
    s1 = oracle.select_blocks_cobs(q[None], mu, var, L, p, order=1)
    s2 = oracle.select_blocks_cobs(q[None], mu, var, L, p, order=2)
    assert set(spread) <= set(s2)
    assert not set(spread) <= set(s1)
    mass = oracle.block_mass(q, K, L, 1.0)
    assert oracle.recall(mass, s2) > oracle.recall(mass, s1) + 0.1


# ---- rounding once to the key dtype (numerics.round_once), pinned by
# construction: points placed between two neighbouring values of the dtype at
# known fractions of the gap, so the nearest value (ties to the even pattern)
# is known without any rounding routine.

def _neighbour_cases(dtype, rng, n=400):
    if dtype == "bf16":
        pats = rng.integers(0x0001, 0x7F7F, n).astype(np.uint32)      # finite, below the largest
        lo = (pats << 16).view(np.float32).astype(np.float64)
        hi = ((pats + 1) << 16).view(np.float32).astype(np.float64)
        even_lo = (pats & 1) == 0
    else:
        pats = rng.integers(0x00000001, 0x7F7FFFFF, n, dtype=np.int64).astype(np.uint32)
        lo = pats.view(np.float32).astype(np.float64)
        hi = (pats + 1).view(np.float32).astype(np.float64)
        even_lo = (pats & 1) == 0
    return lo, hi, even_lo


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_round_once_nearest_and_ties_to_even(dtype):
    rng = np.random.default_rng(11)
    lo, hi, even_lo = _neighbour_cases(dtype, rng)
    gap = hi - lo
    for frac, expect_lo in ((0.25, np.ones_like(even_lo)), (0.75, np.zeros_like(even_lo)),
                            (0.5, even_lo), (0.0, np.ones_like(even_lo)),
                            (0.5 - 2.0 ** -20, np.ones_like(even_lo)),
                            (0.5 + 2.0 ** -20, np.zeros_like(even_lo))):
        x = lo + frac * gap                               # exact in fp64 (dyadic fractions)
        want = np.where(expect_lo.astype(bool), lo, hi).astype(np.float32)
        for sign in (1.0, -1.0):
            got = oracle.round_once(sign * x, dtype)
            assert np.array_equal(got, (sign * want).astype(np.float32)), (dtype, frac, sign)


def test_round_once_special_values():
    assert oracle.round_once(np.array([0.0]), "bf16")[0] == 0.0
    # the smallest subnormal bf16 is 2^-133: half of it is a tie to 0, a bit more rounds up
    assert oracle.round_once(np.array([2.0 ** -134]), "bf16")[0] == 0.0
    assert oracle.round_once(np.array([1.5 * 2.0 ** -134]), "bf16")[0] == np.float32(2.0 ** -133)
    assert oracle.round_once(np.array([3 * 2.0 ** -134]), "bf16")[0] == np.float32(2.0 ** -132)
    big = float(np.float32(3.3895313892515355e38))          # largest bf16 (0x7F7F)
    assert oracle.round_once(np.array([big]), "bf16")[0] == big
    assert np.isinf(oracle.round_once(np.array([2.0 ** 128]), "bf16")[0])
    # a value just above 1 + 2^-8 (the tie between 1 and 1 + 2^-7) goes up, one
    # rounding only: rounding through fp32 first would make it the tie and go down
    x = 1.0 + 2.0 ** -8 + 2.0 ** -40
    assert oracle.round_once(np.array([x]), "bf16")[0] == np.float32(1.0 + 2.0 ** -7)
    assert oracle.bf16_round(np.float32(x)) == np.float32(1.0)


def test_block_stats_equal_exact_rational_mean_and_variance_rounded_once():
    """Exact rational mean and population variance (fractions), then the
    nearest value of the dtype by comparing exact distances to the stored
    value's neighbours."""
    from fractions import Fraction
    rng = np.random.default_rng(12)
    d = 6
    for dtype in ("bf16", "f32"):
        K = oracle.round_to(rng.standard_normal((64 * 3, d)) * 3 + 0.7, dtype)
        mu, var = oracle.block_stats(K, 64 * 3, dtype)
        for b in range(3):
            for c in range(d):
                xs = [Fraction(float(v)) for v in K[64 * b:64 * (b + 1), c]]
                m = sum(xs) / 64
                v = sum((x - m) ** 2 for x in xs) / 64
                for got, exact in ((mu[b, c], m), (var[b, c], v)):
                    g = np.float32(got)
                    if dtype == "bf16":
                        bits = int(g.view(np.uint32)) >> 16
                        nbrs = [np.uint32(p << 16).view(np.float32) for p in (bits - 1, bits + 1)
                                if 0 <= p < 0xFFFF]
                    else:
                        nbrs = [np.nextafter(g, np.float32(np.inf)), np.nextafter(g, np.float32(-np.inf))]
                    dg = abs(Fraction(float(g)) - exact)
                    for nb in nbrs:
                        dn = abs(Fraction(float(nb)) - exact)
                        assert dg <= dn, (dtype, b, c, float(g), float(nb), float(exact))


# ---- the group form of the score for G > 1 heads (Eq. 6 form over the
# estimates: sum over heads of each head's softmax over the blocks)

def _stats_for_scores(seed, nbc=30, d=16):
    rng = np.random.default_rng(seed)
    K = rng.standard_normal((64 * nbc, d)).astype(np.float32)
    K[64 * 5:64 * 6] += 1.5
    return oracle.block_stats(K, 64 * nbc, "f32"), rng


@pytest.mark.parametrize("G", [2, 4, 8])
def test_cobs_softmax_sum_identical_heads_scale_by_G(G):
    (mu, var), rng = _stats_for_scores(20 + G)
    q = rng.standard_normal((1, mu.shape[1])) * 0.5
    nb = mu.shape[0] + 2
    one = oracle.cobs_block_scores(q, mu, var, nb, oracle.SOFTMAX_SUM)
    many = oracle.cobs_block_scores(np.repeat(q, G, axis=0), mu, var, nb, oracle.SOFTMAX_SUM)
    fin = np.isfinite(one)
    assert np.array_equal(fin, np.isfinite(many)) and not fin[-1] and not fin[-2]
    assert np.allclose(many[fin], G * one[fin], rtol=1e-13, atol=0)
    assert np.isclose(many[fin].sum(), G, rtol=1e-12)     # each head's softmax sums to 1


@pytest.mark.parametrize("order", [1, 2])
def test_cobs_softmax_sum_head_permutation_and_single_head_ranking(order):
    (mu, var), rng = _stats_for_scores(31)
    d = mu.shape[1]
    q = rng.standard_normal((8, d)) * 0.4
    nb = mu.shape[0]
    s = oracle.cobs_block_scores(q, mu, var, nb, oracle.SOFTMAX_SUM, order)
    for perm in (rng.permutation(8), np.arange(8)[::-1]):
        sp = oracle.cobs_block_scores(q[perm], mu, var, nb, oracle.SOFTMAX_SUM, order)
        assert np.allclose(sp, s, rtol=1e-13, atol=0)
    # one head: the softmax is a monotone map of the estimate, so both modes rank alike
    L = 64 * nb
    for k in (1, 4, 12):
        ps = SelectParams(top_k=k, n_init=1, n_local=2, score_mode=oracle.SOFTMAX_SUM)
        pr = SelectParams(top_k=k, n_init=1, n_local=2, score_mode=oracle.RAW_SUM)
        assert (oracle.select_blocks_cobs(q[:1], mu, var, L, ps, order)
                == oracle.select_blocks_cobs(q[:1], mu, var, L, pr, order))
    # the group sum differs from any single head's ranking in general, and a
    # head with a dominant direction decides the blocks it prefers
    spike = np.zeros((2, d))
    spike[0, 0] = 40.0
    mu2 = mu.copy()
    mu2[7, 0] = 3.0
    s2 = oracle.cobs_block_scores(spike, mu2, np.zeros_like(var), nb, oracle.SOFTMAX_SUM, order)
    assert np.argmax(s2) == 7 and s2[7] > 1.0                      # head 0 puts ~all its mass there
