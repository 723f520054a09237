"""Host-side checks of the decode kernel's fixed-point schemes (no GPU).

The p.V products w = p S of one head are made fixed point per page: 2^sh is set from the
rounded product top = p_max S_max (sh = 21 - e, e the exponent of top, clamped to [-126, 126]),
p 2^sh comes from one exp2, and x = rne(p 2^sh S) is formed as the float 2^23 + 0x8080 + x,
whose bytes 0 and 1, each xor 0x80, are x's balanced base-256 digits and whose byte 2 is the
top digit read by a signed int8 matrix instruction.  These checks replay that arithmetic in
float32 and pin the two facts the kernel relies on: the digits reconstruct x, and the top digit
never reaches the int8 sign bit, also at the corner p = 1 - 2^-24 with the largest scale of the
page (where a scheme without headroom would round x up to 2^23).

The per-page q.K exponent 2^sigma keeps |qt S 2^sigma| < 2^30 for every head; the last check
replays it over the fp16 range of S and queries.
"""
import numpy as np

F32 = np.float32


def _exp_bits(v):
    return int((np.array([v], dtype=np.float32).view(np.uint32)[0] >> 23) & 0xFF) - 127


def _sh(top):
    e = _exp_bits(top) if top > 0 else 0
    return min(max(21 - e, -126), 126)


def _digits(pw, s):
    """x + 0x8080 in the float's bits: (balanced digit 0, balanced digit 1, top digit, x)."""
    # the kernel's fma rounds p 2^sh S + 2^23 + 0x8080 once: the exact value in float64, then
    # one rounding to float32
    exact = np.float64(pw) * np.float64(s) + 8421504.0
    f = np.array([exact], dtype=np.float64).astype(np.float32)
    bits = int(f.view(np.uint32)[0])
    b0, b1, b2 = bits & 0xFF, (bits >> 8) & 0xFF, (bits >> 16) & 0xFF
    d0 = np.int8(np.uint8(b0 ^ 0x80))
    d1 = np.int8(np.uint8(b1 ^ 0x80))
    x = int(np.float64(f[0])) - 8421504
    return int(d0), int(d1), b2, x


def test_digit_split_reconstructs_and_keeps_the_sign_bit_clear():
    rng = np.random.default_rng(7)
    xs = np.concatenate([np.arange(0, 70000), rng.integers(0, 2 ** 22 + 2 ** 16, 200000),
                         np.arange(2 ** 22 - 70000, 2 ** 22 + 65536)])
    f = (xs.astype(np.float64) + 8421504.0).astype(np.float32)
    assert np.all(f.astype(np.float64) == xs + 8421504.0)  # exact integers below 2^24
    bits = f.view(np.uint32).astype(np.int64)
    d0 = ((bits & 0xFF) ^ 0x80).astype(np.uint8).view(np.int8).astype(np.int64)
    d1 = (((bits >> 8) & 0xFF) ^ 0x80).astype(np.uint8).view(np.int8).astype(np.int64)
    b2 = (bits >> 16) & 0xFF
    assert np.all(d0 + 256 * d1 + 65536 * b2 == xs)
    assert b2.max() <= 65  # far from 128, the int8 sign bit


def test_p_v_headroom_at_the_rounding_corner():
    p = np.nextafter(F32(1.0), F32(0.0))  # 1 - 2^-24
    for s in [1.0, np.nextafter(F32(1.0), F32(0.0)), 65504.0, 2.0 ** -24, 2.0 ** -14, 0.333251953125,
              1.9990234375, 3.0]:
        s = F32(s)
        top = F32(p * s)
        sh = _sh(top)
        # p 2^sh from one exp2: exact power-of-two scaling of p here
        pw = np.float64(p) * 2.0 ** sh
        d0, d1, b2, x = _digits(pw, s)
        assert x <= 2 ** 22 + 1, (s, sh, x)
        assert b2 <= 65
        assert d0 + 256 * d1 + 65536 * b2 == x


def test_p_v_headroom_random_pages():
    """Random pages: p = 2^(lg - mn) <= 1 in float32, S fp16 >= 0; every x <= 2^22 (+1)."""
    rng = np.random.default_rng(11)
    for _ in range(2000):
        lg = rng.normal(0, 4, 128).astype(np.float32)
        s = np.minimum(np.abs(rng.normal(0, 1, 128) * np.exp(rng.normal(0, 3))), 65504.0)
        s = s.astype(np.float16).astype(np.float32)  # finite fp16 scales
        mn = lg.max()
        top = F32(F32(np.exp2(F32(lg.max() - mn))) * s.max())
        sh = _sh(top)
        pw = np.exp2((lg - F32(mn - F32(sh))).astype(np.float32)).astype(np.float64)
        x = np.rint(pw * s.astype(np.float64))
        assert x.max() <= 2 ** 22 * (1 + 2 ** -20) + 1


def test_q_k_exponent_bounds_every_head():
    """2^sigma from the group's largest |qt| and the page's largest S: |qt S 2^sigma| < 2^30."""
    rng = np.random.default_rng(3)
    for _ in range(5000):
        q = np.clip(rng.normal(0, 1, (8, 128)) * np.exp(rng.normal(0, 2)), -65504.0, 65504.0)
        q = q.astype(np.float16).astype(np.float32) * F32(0.1275)  # finite fp16 queries, scaled
        s = np.minimum(np.abs(rng.normal(0, 1, 128) * np.exp(rng.normal(0, 3))), 65504.0)
        s = s.astype(np.float16).astype(np.float32)
        qmax = F32(np.abs(q).max())
        m = F32(qmax * s.max())
        sigma = min(max(29 - _exp_bits(m), -126), 126) if m > 0 else 0
        prod = np.abs(q.astype(np.float64) * s.astype(np.float64)) * 2.0 ** sigma
        assert prod.max() < 2 ** 30
