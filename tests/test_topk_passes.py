"""The top-lp kernel's pass structure, re-derived on the CPU (no GPU).

topk_kernel (csrc/score.hip) skips the leading bits that the list's smallest
and largest order keys share, then selects the lp-th largest key 8 bits at a
time: every wave reads the 256 bins of a pass in 64 lanes of four bins from
the top and takes the digit from the one lane whose count range holds the
rank still sought.  Its emit gives each thread its first output position
from one scan of (keys above the threshold, keys equal to it).  This module
walks the same steps over the same thread split for lists with heavy ties,
negative values, signed zeros and a single distinct value, and checks that
one lane always owns the rank, that at most four passes run, that every
write position lies in [0, lp) and that the kept set is the lp largest
scores with ties to the lowest index (the Spava page, Figure 2 caption: each
block keeps its lp highest-scoring KVs).
"""
import numpy as np
import pytest

THREADS = 1024


def order_key(f):
    u = np.asarray(f, np.float32).view(np.uint32).astype(np.uint64)
    return np.where(u & 0x80000000, (~u) & 0xFFFFFFFF, u | 0x80000000)


def kernel_steps(scores, lp):
    keys = order_key(scores)
    L = len(keys)
    lo, hi = int(keys.min()), int(keys.max())
    top = 0 if lo == hi else (lo ^ hi).bit_length()
    pmask = 0 if top >= 32 else (~((1 << top) - 1)) & 0xFFFFFFFF
    prefix, need, passes = lo & pmask, lp, 0
    while top > 0:
        w = min(8, top)
        shift, dm = top - w, (1 << w) - 1
        match = (keys & pmask) == prefix
        h = np.bincount(((keys[match] >> shift) & dm).astype(np.int64), minlength=256)
        c = h[::-1].reshape(64, 4)                 # lane l: bins 255-4l .. 252-4l
        incl = np.cumsum(c.sum(1))
        above = incl - c.sum(1)
        mine = np.flatnonzero((above < need) & (need <= incl))
        assert len(mine) == 1, "exactly one lane holds the rank"
        l = int(mine[0])
        a = above[l] + np.concatenate([[0], np.cumsum(c[l])[:-1]])
        i = int(np.flatnonzero((a < need) & (need <= a + c[l]))[0])
        prefix |= ((255 - 4 * l - i) & dm) << shift
        pmask |= dm << shift
        need = int(need - a[i])
        top, passes = shift, passes + 1
    thr, take_eq = prefix, need
    chunk = (L + THREADS - 1) // THREADS
    j0 = np.minimum(L, np.arange(THREADS) * chunk)
    j1 = np.minimum(L, j0 + chunk)
    gt = np.array([(keys[a:b] > thr).sum() for a, b in zip(j0, j1)])
    eq = np.array([(keys[a:b] == thr).sum() for a, b in zip(j0, j1)])
    gt_before, eq_before = np.cumsum(gt) - gt, np.cumsum(eq) - eq
    out = np.full(lp, -1, np.int64)
    for t in range(THREADS):
        pos, q = gt_before[t] + min(eq_before[t], take_eq), eq_before[t]
        for j in range(j0[t], j1[t]):
            keep = keys[j] > thr
            if keys[j] == thr:
                keep, q = q < take_eq, q + 1
            if keep:
                assert 0 <= pos < lp
                out[pos] = j
                pos += 1
    return out, passes


def lists(seed=5, count=48):
    rng = np.random.default_rng(seed)
    for i in range(count):
        L = int(rng.choice([1, 2, 7, 1023, 1024, 1025, 3840, 8128, 17000]))
        lp = int(rng.choice([1, L, int(rng.integers(1, L + 1))]))
        kind = i % 6
        if kind == 0:
            s = rng.random(L)
        elif kind == 1:
            s = rng.random(L) * 0.01 + 1.0
        elif kind == 2:
            s = rng.integers(0, 4, L).astype(float)
        elif kind == 3:
            s = rng.standard_normal(L)
        elif kind == 4:
            s = np.full(L, 0.5)
        else:
            s = np.where(rng.random(L) < 0.5, 0.0, -0.0)
        yield pytest.param(np.asarray(s, np.float32), lp, id=f"{i}_L{L}_lp{lp}_k{kind}")


@pytest.mark.parametrize("scores,lp", list(lists()))
def test_topk_passes(scores, lp):
    out, passes = kernel_steps(scores, lp)
    assert passes <= 4
    keys = order_key(scores).astype(np.int64)
    want = np.sort(np.lexsort((np.arange(len(keys)), -keys))[:lp])
    np.testing.assert_array_equal(out, want)
