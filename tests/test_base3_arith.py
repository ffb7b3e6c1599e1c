"""The arithmetic the matrix-core contraction of the base-3 layout relies on,
checked on the CPU with numpy: the fraction form of a byte, the 16-bit-lane
multiplies that leave the top digits in bytes 1 and 3 (with the 0x8000 added
for the last step), and the two linear forms C0, C1 whose combination
C0 - 3 C1 + 128 X5 - X is the ternary contraction.  This emulates the
kernel's operations word by word in integer arithmetic, independently of the
oracle; the GPU parity tests compare the kernel itself with the oracle."""
import numpy as np

import oracle

M32 = np.uint64(0xFFFFFFFF)


def fraction_form(v):
    return (256 * np.asarray(v, np.uint64) + 242) // 243


def test_fraction_form_bijection_and_top_digits():
    v = np.arange(243, dtype=np.uint64)
    q = fraction_form(v)
    assert len(set(q.tolist())) == 243 and int(q.max()) <= 255
    assert np.array_equal((243 * q) >> np.uint64(8), v)
    for s in range(1, 6):
        assert np.array_equal((3 ** s * q) >> np.uint64(8), v // 3 ** (5 - s))
    # the low byte after the last step never reaches 243
    assert int(((243 * q) & np.uint64(255)).max()) <= 242


def lane_products(w):
    """The kernel's per-dword work on stored bytes w (uint32 as uint64): for
    s = 1 .. 5 the byte-1/byte-3 values of 3^s * e and 3^s * o (e = bytes 0
    and 2, o = bytes 1 and 3 moved down), the s = 5 word with 0x80008000
    added modulo 2^32; returns digit-step values [s][4 bytes] as signed."""
    e = w & np.uint64(0x00FF00FF)
    o = (w >> np.uint64(8)) & np.uint64(0x00FF00FF)
    out = []
    for s in range(1, 6):
        mul = np.uint64(3 ** s)
        E = (e * mul) & M32
        O = (o * mul) & M32
        if s == 5:
            E = (E + np.uint64(0x80008000)) & M32
            O = (O + np.uint64(0x80008000)) & M32
        # byte p of the dword: p = 0 -> E byte 1, 1 -> O byte 1, 2 -> E byte 3, 3 -> O byte 3
        b = [(E >> np.uint64(8)) & np.uint64(255), (O >> np.uint64(8)) & np.uint64(255),
             (E >> np.uint64(24)) & np.uint64(255), (O >> np.uint64(24)) & np.uint64(255)]
        vals = np.stack(b, axis=-1).astype(np.int64)
        if s == 5:
            vals = np.where(vals >= 128, vals - 256, vals)   # read as signed bytes
        out.append(vals)
    return out


def test_lane_products_every_byte_pair():
    # every stored byte in every position, against the digits of v
    q = fraction_form(np.arange(243)).astype(np.uint64)
    a, b = np.meshgrid(q, q, indexing="ij")
    w = (a | (b << np.uint64(8)) | (b << np.uint64(16)) | (a << np.uint64(24))).ravel()
    vals = lane_products(w)
    va = (243 * a.ravel()) >> np.uint64(8)
    vb = (243 * b.ravel()) >> np.uint64(8)
    for s in range(1, 6):
        ta, tb = va // 3 ** (5 - s), vb // 3 ** (5 - s)
        if s == 5:
            ta, tb = ta.astype(np.int64) - 128, tb.astype(np.int64) - 128
        got = vals[s - 1]
        assert np.array_equal(got[:, 0], ta.astype(np.int64))
        assert np.array_equal(got[:, 1], tb.astype(np.int64))
        assert np.array_equal(got[:, 2], tb.astype(np.int64))
        assert np.array_equal(got[:, 3], ta.astype(np.int64))


def test_two_forms_give_the_contraction():
    rng = np.random.default_rng(5)
    N, K = 37, 800                                  # ten 80-k blocks
    Wt = rng.integers(-1, 2, (N, K)).astype(np.int8)
    x = rng.integers(-128, 128, K).astype(np.int64)
    x[:7] = -128
    canon = oracle.pack3(Wt).astype(np.uint64)      # [N][K/5], byte p holds k = 5p + j at 3^j
    words = fraction_form(canon).reshape(N, K // 20, 4)
    w = words[..., 0] | (words[..., 1] << np.uint64(8)) | (words[..., 2] << np.uint64(16)) | \
        (words[..., 3] << np.uint64(24))
    vals = lane_products(w.ravel())                 # [s] -> [N * K/20][4]
    xs = x.reshape(K // 5, 5)                       # byte p: x[5p + j]
    xbyte = xs.reshape(K // 20, 4, 5)
    C0 = np.zeros(N, np.int64)
    C1 = np.zeros(N, np.int64)
    for s in range(1, 6):
        T = vals[s - 1].reshape(N, K // 20, 4)
        C0 += np.einsum("ndp,dp->n", T, xbyte[..., 5 - s])
        if s < 5:
            C1 += np.einsum("ndp,dp->n", T, xbyte[..., 4 - s])
    X, X5 = int(x.sum()), int(x[0::5].sum())
    y = C0 - 3 * C1 + 128 * X5 - X
    assert np.array_equal(y, Wt.astype(np.int64) @ x)
