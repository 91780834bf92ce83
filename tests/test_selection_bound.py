"""The rules behind the bound-then-rank top-16 selections -- the selecting
attention's (select.hpp) and the one-wave form (topk_wave.hpp) -- modelled on
the CPU and checked against brute force.

Each wave of NT/64 finds the largest 16-bit key prefix x that at least C of its
keys reach; the R-th largest such x over the waves (C * R >= 15, C = max(2,
ceil(15 / full waves))) is reached by at least 15 keys, so it never exceeds the
row's 15th-best key: every winner survives the filter, and ranking the
survivors exactly gives the brute-force selection.  When more than 64 keys
survive, a second pass sets the low 16 bits of each wave's bound over the keys'
upper 32 bits (the same argument).  Keys are the library's:
order-preserving score bits over the complemented block id (NaN lowest, -0 ==
+0), so they are distinct.  This checks the rule, not the kernel; the GPU tests
check the kernel against msa_block_topk and the oracle.
"""
import numpy as np
import pytest


def order_keys(s):
    s = np.asarray(s, np.float32).copy()
    s[s == 0] = 0.0
    u = s.view(np.uint32).astype(np.uint64)
    k = np.where(u & 0x80000000, (~u) & 0xFFFFFFFF, u | 0x80000000)
    return np.where(np.isnan(s), 0, k).astype(np.uint64)


def keys_of(scores, own):
    i = np.arange(own, dtype=np.uint64)
    return (order_keys(scores[:own]) << np.uint64(32)) | (np.uint64(0xFFFFFFFF) - i)


def bound_rank(scores, own, NT):
    """The kernel's rule: the winners (15 block ids, ascending with own) or None when
    more than 64 keys reach the bound (the radix fallback's case); and the bound."""
    NW = NT // 64
    E = -(-own // NT)
    keys = keys_of(scores, own)
    slot_keys = np.zeros((E, NT), np.uint64)         # thread t holds blocks t, t + NT, ...
    for e in range(E):
        part = keys[e * NT:(e + 1) * NT]
        slot_keys[e, :len(part)] = part
    nwa = max(1, min(NW, min(own, NT) // 64))
    C = max(2, -(-15 // nwa))
    R = -(-15 // C)
    hi = (slot_keys >> np.uint64(32)).astype(np.int64)
    xs = [0] * NW
    for bits in (range(31, 15, -1), range(15, -1, -1)):   # the second pass only when needed
        for w in range(NW):
            h = hi[:, 64 * w:64 * w + 64]
            for bit in bits:
                c = xs[w] | (1 << bit)
                if int((h >= c).sum()) >= C:
                    xs[w] = c
        tau = np.uint64(sorted(xs, reverse=True)[R - 1]) << np.uint64(32)
        cand = keys[keys >= tau]
        if len(cand) <= 64:
            winners = np.sort(cand)[::-1][:15]
            ids = sorted([int(np.uint64(0xFFFFFFFF) - (k & np.uint64(0xFFFFFFFF))) for k in winners] + [own])
            return ids, tau
    return None, tau


def brute(scores, own):
    keys = np.sort(keys_of(scores, own))[::-1]
    return sorted([int(np.uint64(0xFFFFFFFF) - (k & np.uint64(0xFFFFFFFF))) for k in keys[:15]] + [own]), keys[14]


@pytest.mark.parametrize("kind", ["normal", "block_max", "rounded", "nan", "flat", "hot", "offset", "negative"])
@pytest.mark.parametrize("NT", [1024, 256])
def test_bound_never_drops_a_winner(kind, NT):
    rng = np.random.default_rng([NT] + [ord(ch) for ch in kind])
    fast = 0
    for trial in range(12):
        own = int(rng.integers(16, 3 * NT))
        n = own + 1
        if kind == "block_max":
            s = (rng.standard_normal((n, 64)) * 8).max(axis=1)
        else:
            s = rng.standard_normal(n)
        if kind == "rounded":
            s = np.round(s * 2)
        if kind == "nan":
            s[rng.random(n) < 0.1] = np.nan
        if kind == "flat":
            s[:] = 1.0
        if kind == "hot":
            s[rng.permutation(own)[:8]] += 40.0
        if kind == "offset":
            s = 1000.0 + 0.01 * s                   # the top 16 bits of every score agree
        if kind == "negative":
            s = -np.abs(s) - 1000.0
        s = s.astype(np.float32)
        ids, tau = bound_rank(s, own, NT)
        want, kth = brute(s, own)
        assert tau <= kth                      # the bound is at most the 15th-best key
        if ids is not None:
            fast += 1
            assert ids == want
    if kind in ("normal", "block_max", "hot", "offset", "negative"):
        assert fast >= 9                       # the ranked list covers typical rows


# ---------------------------------------------------------------- the one-wave form

def wave_keys(s):
    """The one-wave form's 32-bit score keys: non-negative scores keep their bits with
    the top bit set, negative ones take the two's-complement negation of their bits,
    NaN is 0."""
    s = np.asarray(s, np.float32)
    u = s.view(np.uint32).astype(np.uint64)
    sgn = np.where(u & 0x80000000, 0xFFFFFFFF, 0).astype(np.uint64)
    k = ((u ^ (sgn | 0x80000000)) - sgn) & 0xFFFFFFFF
    return np.where(np.isnan(s), 0, k).astype(np.uint64)


def test_wave_keys_order_like_the_selection_keys():
    """Same order as the selection keys on every pair: special values (signed zeros,
    denormals, infinities, NaN of both signs) and random scores of all magnitudes."""
    sp = np.array([0.0, -0.0, 1e-45, -1e-45, 1.17549435e-38, -1.17549435e-38, 1.0, -1.0,
                   3.4028235e38, -3.4028235e38, np.inf, -np.inf, np.nan, -np.nan], np.float32)
    rng = np.random.default_rng(11)
    bits = rng.integers(0, 2 ** 32, size=2000, dtype=np.uint64).astype(np.uint32).view(np.float32)
    s = np.concatenate([sp, bits, rng.standard_normal(500).astype(np.float32)])
    a, b = order_keys(s).astype(np.int64), wave_keys(s).astype(np.int64)
    assert np.array_equal(np.sign(a[:, None] - a[None, :]), np.sign(b[:, None] - b[None, :]))
    assert wave_keys(np.float32([np.nan]))[0] == 0 and wave_keys(np.float32([-np.inf]))[0] > 0


def wave_bound_rank(scores, own):
    """The one-wave rule: lane l holds blocks l, l + 64, ...; x is the largest 16-bit
    prefix that at least 15 lanes' largest keys reach, refined to all 32 bits (the 15th
    largest lane maximum) when more than 64 keys reach it; None when x is 0 (fewer than
    15 lanes hold a number) or more than 64 keys reach the refined x (the radix
    fallback's cases)."""
    k32 = wave_keys(scores[:own])
    E = -(-own // 64)
    lanes = np.zeros((E, 64), np.uint64)
    lanes.reshape(-1)[:own] = k32
    lmax = lanes.max(axis=0)
    x = 0
    for bits in (range(31, 15, -1), range(15, -1, -1)):
        for bit in bits:
            c = x | (1 << bit)
            if int((lmax >= c).sum()) >= 15:
                x = c
        if x == 0:
            return None, 0
        idx = np.nonzero(k32 >= x)[0]
        if len(idx) <= 64:
            keys = (k32[idx] << np.uint64(32)) | (np.uint64(0xFFFFFFFF) - idx.astype(np.uint64))
            win = np.sort(keys)[::-1][:15]
            return sorted([int(np.uint64(0xFFFFFFFF) - (k & np.uint64(0xFFFFFFFF))) for k in win] + [own]), x
    return None, x


@pytest.mark.parametrize("kind", ["normal", "block_max", "rounded", "nan", "mostly_nan", "flat", "hot",
                                  "negative"])
def test_wave_bound_never_drops_a_winner(kind):
    rng = np.random.default_rng([64] + [ord(ch) for ch in kind])
    fast = 0
    for trial in range(16):
        own = int(rng.integers(16, 1025))
        n = own + 1
        if kind == "block_max":
            s = (rng.standard_normal((n, 64)) * 8).max(axis=1)
        else:
            s = rng.standard_normal(n)
        if kind == "rounded":
            s = np.round(s * 2)                     # ties, and -0 beside +0
        if kind == "nan":
            s[rng.random(n) < 0.1] = np.nan
        if kind == "mostly_nan":
            s[rng.random(n) < 0.97] = np.nan
        if kind == "flat":
            s[:] = 1.0
        if kind == "hot":
            s[rng.permutation(own)[:8]] += 40.0
        if kind == "negative":
            s = -np.abs(s) - 1000.0
        s = s.astype(np.float32)
        ids, x = wave_bound_rank(s, own)
        want, kth = brute(s, own)
        assert x <= np.sort(wave_keys(s[:own]))[::-1][14]   # at most the 15th-best score's key
        if ids is not None:
            fast += 1
            assert ids == want
    if kind in ("normal", "block_max", "hot", "negative"):
        assert fast >= 12                      # the ranked list covers typical rows
