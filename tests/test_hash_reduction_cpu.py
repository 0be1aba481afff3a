"""The hash kernel's Horner step reduces y = x*V0 + t (x < V < 2^31, V0 < 2^31, t < 2^32)
modulo V by Barrett reduction with m = floor((2^64 - 1) / V): q = floor(y*m / 2^64), r = y - q*V,
one conditional subtraction. This re-derives that claim in exact integers at the edges of the
range the kernel accepts (the GPU tests compare the kernel itself with the oracle)."""
import random

M64 = (1 << 64) - 1


def barrett_step(x, V0, t, V):
    y = x * V0 + t
    assert y < (1 << 63)
    m = M64 // V
    q = (y * m) >> 64
    r = y - q * V
    assert 0 <= r < 2 * V
    return r - V if r >= V else r


def test_barrett_step_edges():
    big = (1 << 31) - 1
    for V in (1, 2, 3, 7, 65536, 65537, big - 1, big):
        for V0 in (1, 2, 131072, big - 1, big):
            for x in {0, 1, V - 1, V // 2}:
                for t in (0, 1, V0 - 1, (1 << 32) - 1):
                    assert barrett_step(x, V0, t, V) == (x * V0 + t) % V


def test_barrett_step_random():
    rng = random.Random(0)
    for _ in range(200000):
        V = rng.randrange(1, 1 << 31)
        V0 = rng.randrange(1, 1 << 31)
        x = rng.randrange(0, V)
        t = rng.randrange(0, 1 << 32)
        assert barrett_step(x, V0, t, V) == (x * V0 + t) % V
