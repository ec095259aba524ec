"""CPU checks of the schedule model the 256x256-tile down kernel uses to choose
its K split on the device (csrc/ffn_dma.hip, two_part_makespan): one XCD's 32
CUs take n tiles of cost a, then n tiles of cost b, each CU the next tile as
soon as it is free. The kernel evaluates that finish time in closed form; here
the closed form, restated from the kernel's comment, is compared with the
definition itself, a literal greedy list schedule, on random costs and on every
tile cost the kernel's candidates produce. (On the GPU, test_down_split_choice
pins the kernel's choice to the restated rule bit for bit.)"""
import random

CUS = 32
FIX = 12  # fixed cost of a tile in K steps


def greedy(n, a, b):
    """Finish time of the list schedule: each tile to the CU free first."""
    busy = [0] * CUS
    for c in [a] * n + [b] * n:
        i = busy.index(min(busy))
        busy[i] += c
    return max(busy)


def closed_form(n, a, b):
    """After the first parts, r = n % 32 CUs are at L + a and the others at L
    (L = (n // 32) a). The second parts start at the n smallest of L + m b
    (each for the lower CUs) and L + a + m b (each for the upper ones); the
    finish is the n-th smallest start plus b, or L + a if that is later."""
    L, r = (n // CUS) * a, n % CUS
    nlo = CUS - r
    t = (-(-n // nlo) - 1) * b          # the n-th start if the lower CUs took all
    if r > 0 and t >= a:
        al = a // b
        up = al + (1 if a % b else 0)
        mhi = max(0, -(-(n - nlo * al) // CUS) - 1)
        mlo = max(up, -(-(n + r * up) // CUS) - 1)
        t = min(a + mhi * b, mlo * b)
    return L + max(t + b, a if r > 0 else 0)


def test_closed_form_equals_the_greedy_schedule_on_random_costs():
    rng = random.Random(2024)
    for _ in range(3000):
        n = rng.randint(1, 256)
        a = rng.randint(1, 700)
        b = rng.randint(1, 700)      # either part may be the longer one
        assert closed_form(n, a, b) == greedy(n, a, b), (n, a, b)


def test_closed_form_on_the_kernels_candidates():
    """First parts of 8/16 .. 13/16 of K rounded down to whole 4-step trips
    (at least 4 steps in each part), plus the fixed cost, for every K of 8 to
    1024 steps in multiples of 4 and every tile count of one to eight rounds."""
    for nsteps in range(8, 1025, 44):
        for j in range(8, 14):
            s0 = (nsteps * j // 16) & ~3
            if s0 < 4 or nsteps - s0 < 4:
                continue
            a, b = s0 + FIX, nsteps - s0 + FIX
            for n in range(1, 8 * CUS + 1, 5):
                assert closed_form(n, a, b) == greedy(n, a, b), (nsteps, j, n)


def test_special_cases():
    # fewer tiles than CUs: the second parts go to the idle CUs first
    assert closed_form(10, 300, 100) == 300
    assert closed_form(20, 300, 100) == 300    # 12 idle CUs take 12, then 8 of them one more
    assert closed_form(1, 50, 70) == 70
    # whole rounds of equal parts
    assert closed_form(64, 100, 100) == 400
    # a last round a quarter full: 8 CUs run three first parts
    assert closed_form(72, 348, 124) == 1068
    assert closed_form(72, 376, 96) == 1128
