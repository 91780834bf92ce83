"""The rule behind the selecting attention's bound-then-rank top-16 (select.hpp),
modelled on the CPU and checked against brute force.

Each wave of NT/64 finds the largest 16-bit key prefix x that at least C of its
keys reach; the R-th largest such x over the waves (C * R >= 15, C = max(2,
ceil(15 / full waves))) is reached by at least 15 keys, so it never exceeds the
row's 15th-best key: every winner survives the filter, and ranking the
survivors exactly gives the brute-force selection.  Keys are the library's:
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
    hi = (slot_keys >> np.uint64(48)).astype(np.int64)
    valid = slot_keys != 0
    xs = []
    for w in range(NW):
        h, v = hi[:, 64 * w:64 * w + 64], valid[:, 64 * w:64 * w + 64]
        x = 0
        for bit in range(15, -1, -1):
            c = x | (1 << bit)
            if int(((h >= c) & v).sum()) >= C:
                x = c
        xs.append(x)
    tau = np.uint64(sorted(xs, reverse=True)[R - 1]) << np.uint64(48)
    cand = keys[keys >= tau]
    if len(cand) > 64:
        return None, tau
    winners = np.sort(cand)[::-1][:15]
    ids = sorted([int(np.uint64(0xFFFFFFFF) - (k & np.uint64(0xFFFFFFFF))) for k in winners] + [own])
    return ids, tau


def brute(scores, own):
    keys = np.sort(keys_of(scores, own))[::-1]
    return sorted([int(np.uint64(0xFFFFFFFF) - (k & np.uint64(0xFFFFFFFF))) for k in keys[:15]] + [own]), keys[14]


@pytest.mark.parametrize("kind", ["normal", "block_max", "rounded", "nan", "flat", "hot"])
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
        s = s.astype(np.float32)
        ids, tau = bound_rank(s, own, NT)
        want, kth = brute(s, own)
        assert tau <= kth                      # the bound is at most the 15th-best key
        if ids is not None:
            fast += 1
            assert ids == want
    if kind in ("normal", "block_max", "hot"):
        assert fast >= 9                       # the ranked list covers typical rows
