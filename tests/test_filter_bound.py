"""CPU check of pass 2's bound walk (csrc/passes.hip raise_bound_regs).

The streaming filter keeps, per query row, a histogram of its candidates over
mass bins and a bound bin bt with at least k candidates in bins >= bt. After
appends it raises bt while the candidates above bt still number at least k:
    while bt < last and cg - count(bt) >= k: cg -= count(bt); bt += 1
The kernel evaluates the first seven moves without branches, from the four
histogram words it reads (prefix sums of the bin counts: the moves are a
prefix because the sums only grow), and continues with the loop only past
them. The two formulations are restated below from the source and must agree
on every histogram, bound and count, including bounds at the last bins.
"""
import random

KBINS = 49 * 8          # kFBins
KWORDS = KBINS // 2     # two 16-bit counts per word


def walk_loop(words, bt, cg, budget):
    b = bt
    while True:
        hb = (words[b >> 1] >> ((b & 1) * 16)) & 0xFFFF
        if b >= KBINS - 1 or cg - hb < budget:
            break
        cg -= hb
        b += 1
    return cg, b, hb


def walk_prefix(words, bt, cg, budget):
    w0 = bt >> 1
    wv = [words[min(w0 + j, KWORDS - 1)] for j in range(4)]
    odd = bt & 1
    cnt = [(wv[h >> 1] >> ((h & 1) * 16)) & 0xFFFF for h in range(8)]
    s = total = moved = 0
    hb = cnt[1] if odd else cnt[0]
    for t in range(7):
        c = cnt[t + 1] if odd else cnt[t]
        total += c
        step = bt + t < KBINS - 1 and cg - total >= budget
        s += 1 if step else 0
        moved += c if step else 0
        if t < 6 and step:
            hb = cnt[t + 2] if odd else cnt[t + 1]
    cg -= moved
    b = bt + s
    if s == 7:
        while True:
            hb = (words[b >> 1] >> ((b & 1) * 16)) & 0xFFFF
            if b >= KBINS - 1 or cg - hb < budget:
                break
            cg -= hb
            b += 1
    return cg, b, hb


def test_bound_walk_prefix_form_matches_the_loop():
    rng = random.Random(7)
    for _ in range(30000):
        counts = [rng.choice([0, 0, 0, 1, 2, 3, 5, 8, 20, 100]) for _ in range(KBINS)]
        words = [counts[2 * i] | (counts[2 * i + 1] << 16) for i in range(KWORDS)]
        if rng.random() < 0.9:
            bt = rng.randrange(KBINS)
        else:
            bt = rng.choice([KBINS - 1, KBINS - 2, KBINS - 3, KBINS - 8, KBINS - 9])
        budget = rng.randint(1, 60)
        cg = sum(counts[bt:]) + rng.randint(0, 5)
        assert walk_loop(words, bt, cg, budget) == walk_prefix(words, bt, cg, budget)


def test_bound_walk_long_and_edge_walks():
    # many empty bins: the walk runs past the four words in hand
    counts = [0] * KBINS
    counts[300] = 50
    words = [counts[2 * i] | (counts[2 * i + 1] << 16) for i in range(KWORDS)]
    for bt in (0, 1, 290, 299):
        assert walk_prefix(words, bt, 50, 10) == walk_loop(words, bt, 50, 10) == (50, 300, 50)
    # a bound that may not pass the last bin
    counts = [1] * KBINS
    words = [counts[2 * i] | (counts[2 * i + 1] << 16) for i in range(KWORDS)]
    assert walk_prefix(words, KBINS - 3, 10 ** 6, 1) == walk_loop(words, KBINS - 3, 10 ** 6, 1)
