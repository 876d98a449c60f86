"""The requantisation modes the kernels choose between, checked on the CPU against the
oracle's round-half-away-from-zero requantisation.

The kernels compute q = round_half_away(y * m / 2^(31+s)) three ways (device_common.h): a
general 64-bit form, a one-multiply form without the tie correction, and a form with it.  The
one-multiply form is used only when every channel of a wave has s >= 2 and either a multiplier
with at most s - 2 trailing zero bits (no halfway tie can occur for any int32 sum, -2^31
included) or ReLU without a shortcut.
These tests model that arithmetic in Python integers and require it to agree with the oracle,
including on the values most likely to tie.
"""
import numpy as np
import pytest

from oracle import ref as orc


def one_multiply(y, m, s):
    """hi(y*m + 2^(30+s)) >> (s-1): round half up, the kernels' mode 1 (bias folded in y)."""
    p = y * m + (1 << (30 + s))
    return (p >> 32) >> (s - 1)


def tie_free(m, s):
    """The kernels' predicate: m == 0, or ctz(m) + 1 < s."""
    return m == 0 or (m & -m).bit_length() - 1 + 1 < s


def candidates(rng, m, s, count=400):
    """Random sums plus the sums nearest to every halfway point reachable in int32."""
    ys = list(rng.integers(-(1 << 31), 1 << 31, size=count))
    k = 31 + s
    for j in range(-200, 200):  # y*m close to (j + 1/2) * 2^k
        target = (2 * j + 1) << (k - 1)
        if m:
            for y0 in (target // m - 1, target // m, target // m + 1, -(-target // m)):
                if -(1 << 31) <= y0 < (1 << 31):
                    ys.append(y0)
    for e in range(0, 31):  # high powers of two in y
        ys += [1 << e, -(1 << e), 3 << e if (3 << e) < (1 << 31) else 1]
    ys += [-(1 << 31), (1 << 31) - 1]  # both ends of the int32 range (the oracle accepts both)
    return [int(y) for y in ys]


@pytest.mark.parametrize("s", [2, 3, 8, 16, 31])
def test_tie_free_multipliers_need_no_tie_correction(s):
    rng = np.random.default_rng(s)
    mults = [int(m) for m in rng.integers(1 << 30, 1 << 31, size=6)]
    mults += [m | 1 for m in mults] + [(1 << 30) | (1 << (s - 1)), 0]  # trailing zeros just below s
    for m in mults:
        if not tie_free(m, s):
            continue
        for y in candidates(rng, m, s):
            assert one_multiply(y, m, s) == orc.requant(y, 0, m, s), (y, m, s)


@pytest.mark.parametrize("m,s,want", [(128, 8, -1), ((1 << 30) | (1 << 15), 16, -16385)])
def test_int32_min_ties_with_s_minus_1_trailing_zeros(m, s, want):
    """y = -2^31 has 31 trailing zero bits, so a multiplier with exactly s - 1 of them puts it on
    a tie: the one-multiply form rounds it up, the oracle away from zero.  The predicate must
    send such a channel to the tie-correcting form."""
    y = -(1 << 31)
    assert orc.requant(y, 0, m, s) == want
    assert one_multiply(y, m, s) == want + 1
    assert not tie_free(m, s)


def test_multipliers_with_many_trailing_zeros_do_tie():
    """The condition is needed: with m = 2^30 and s = 2, y = -4 sits exactly halfway."""
    m, s, y = 1 << 30, 2, -4
    assert not tie_free(m, s)
    assert orc.requant(y, 0, m, s) == -1 and one_multiply(y, m, s) == 0


@pytest.mark.parametrize("s", [2, 5, 20])
def test_relu_without_shortcut_hides_negative_ties(s):
    """ReLU, no shortcut: wherever the one-multiply form differs from the oracle, both clamp to 0."""
    rng = np.random.default_rng(100 + s)
    for m in [1 << 30, 3 << 28, int(rng.integers(1 << 30, 1 << 31))]:
        for y in candidates(rng, m, s, 200):
            a, b = one_multiply(y, m, s), orc.requant(y, 0, m, s)
            assert a == b or (max(a, 0) == 0 and max(b, 0) == 0), (y, m, s)


def test_bias_folded_into_the_addend():
    """acc*m + (bias*m + 2^(30+s)) equals (acc + bias)*m + 2^(30+s) for the full int32 ranges."""
    rng = np.random.default_rng(7)
    for _ in range(2000):
        acc = int(rng.integers(-(1 << 30), 1 << 30))
        bias = int(rng.integers(-(1 << 30), 1 << 30))
        m = int(rng.integers(0, 1 << 31))
        s = int(rng.integers(2, 32))
        folded = ((acc * m + bias * m + (1 << (30 + s))) >> 32) >> (s - 1)
        assert folded == one_multiply(acc + bias, m, s)
