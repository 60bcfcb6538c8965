"""Pins for the CPU oracle: checks against facts other than the oracle itself.

Each pin is a function of an ``oracle.Oracle`` instance that raises
AssertionError on a mismatch. ``test_oracle_pins.py`` runs them against the
real oracle; ``test_oracle_mutants.py`` runs them against oracles with a
planted mistake and requires that some pin fails for every mistake.

Kinds of pin (none of them re-types the oracle's own code):
* library routine: numpy's IEEE fp16 decoding, numpy float64 matmul;
* hand-worked blocks from ``tests/golden`` (constructed, with derivations);
* closed forms and invariants (x = ones, one-hot x, linearity, batching);
* round trip: requantizing the oracle's dequantized weights with the block's
  own scales must give back the generator's integer codes;
* brute force: exact rational sums (``fractions.Fraction``) on tiny shapes.
"""
from __future__ import annotations

import os
from fractions import Fraction

import numpy as np

import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def read_golden(name: str) -> dict:
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, v = (s.strip() for s in line.split("=", 1))
            out[k] = v
    return out


def _hex(s: str) -> np.ndarray:
    return np.frombuffer(bytes.fromhex(s), dtype=np.uint8).copy()


def _onehot(K, k):
    x = np.zeros((1, K), np.float32)
    x[0, k] = 1.0
    return x


# ---------------------------------------------------------------- fp16 decode
def pin_f16_exhaustive(o):
    """All 65,536 binary16 patterns decode exactly as numpy's float16."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = o.f16_to_f64(bits)
    ref = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # signed zero is kept
    assert np.signbit(got[0x8000]) and not np.signbit(got[0])


# --------------------------------------------------------------- hand-worked
def pin_q4_0_worked(o):
    g = read_golden("q4_0_block.txt")
    W = _hex(g["block_hex"])
    K = 32
    cases = {"ones": np.ones((1, K), np.float32), "e1": _onehot(K, 1),
             "e16": _onehot(K, 16), "e31": _onehot(K, 31),
             "ramp": np.arange(K, dtype=np.float32)[None]}
    for key, x in cases.items():
        y = o.gemv_q4_0(W, x, 1, K)
        assert y[0, 0] == float(g[key]), (key, y[0, 0])
        yh = o.gemv_q4_0(_hex(g["d_half_block_hex"]), x, 1, K)
        assert yh[0, 0] == float(g[key]) / 2, (key, yh[0, 0])


def pin_q8_0_worked(o):
    g = read_golden("q8_0_block.txt")
    K = 32
    for blk, keys in (("a", {"ones": None, "e0": 0, "e31": 31}),
                      ("b", {"ones": None, "e0": 0, "e1": 1})):
        W = _hex(g[f"{blk}_hex"])
        for key, k in keys.items():
            X = np.ones((1, K), np.float16) if k is None else _onehot(K, k).astype(np.float16)
            Y = o.gemm_q8_0_f16(W, X, 1, K)
            assert Y[0, 0] == float(g[f"{blk}_{key}"]), (blk, key, Y[0, 0])


def pin_q4_k_worked(o):
    g = read_golden("q4_k_block.txt")
    K = 256
    head = _hex("003c0038" + g["scales_hex"])
    qa = np.full(128, 0x11, np.uint8)
    i = np.arange(128)
    qb = ((i % 16) | ((15 - i % 16) << 4)).astype(np.uint8)
    Wa = np.concatenate([head, qa])
    Wb = np.concatenate([head, qb])
    ones = np.ones((1, K), np.float32)
    assert o.gemv_q4_k(Wa, ones, 1, K)[0, 0] == float(g["a_ones"])
    assert o.gemv_q4_k(Wa, _onehot(K, 167), 1, K)[0, 0] == float(g["a_e167"])
    assert o.gemv_q4_k(Wa, _onehot(K, 128), 1, K)[0, 0] == float(g["a_e128"])
    assert o.gemv_q4_k(Wb, ones, 1, K)[0, 0] == float(g["b_ones"])
    for k in (3, 35, 180, 223):
        assert o.gemv_q4_k(Wb, _onehot(K, k), 1, K)[0, 0] == float(g[f"b_e{k}"]), k


def pin_q8_0_gemv_worked(o):
    """The Q8_0 worked blocks through the decode GEMV (fp32 activations)."""
    g = read_golden("q8_0_block.txt")
    K = 32
    for blk, keys in (("a", {"ones": None, "e0": 0, "e31": 31}),
                      ("b", {"ones": None, "e0": 0, "e1": 1})):
        W = _hex(g[f"{blk}_hex"])
        for key, k in keys.items():
            x = np.ones((1, K), np.float32) if k is None else _onehot(K, k)
            assert o.gemv_q8_0(W, x, 1, K)[0, 0] == float(g[f"{blk}_{key}"]), (blk, key)


def pin_gemm_q4_worked(o):
    """The Q4_0 and Q4_K worked blocks through the prefill GEMMs (fp16 X rows
    of ones and one-hots are exact)."""
    g = read_golden("q4_0_block.txt")
    W = _hex(g["block_hex"])
    for key, x in {"ones": np.ones((1, 32), np.float32), "e1": _onehot(32, 1),
                   "e16": _onehot(32, 16), "e31": _onehot(32, 31),
                   "ramp": np.arange(32, dtype=np.float32)[None]}.items():
        Y = o.gemm_q4_0_f16(W, x.astype(np.float16), 1, 32)
        assert Y[0, 0] == float(g[key]), (key, Y[0, 0])
    gk = read_golden("q4_k_block.txt")
    Wa = np.concatenate([_hex("003c0038" + gk["scales_hex"]), np.full(128, 0x11, np.uint8)])
    X = np.zeros((3, 256), np.float16)
    X[0] = 1
    X[1, 167] = 1
    X[2, 128] = 1
    Y = o.gemm_q4_k_f16(Wa, X, 1, 256)[:, 0]
    assert list(Y) == [float(gk["a_ones"]), float(gk["a_e167"]), float(gk["a_e128"])], Y


def pin_q6_k_worked(o):
    g = read_golden("q6_k_block.txt")
    K = 256
    for blk in ("a", "b", "c"):
        W = _hex(g[f"{blk}_hex"])
        assert W.size == 210
        for key, v in g.items():
            if not key.startswith(blk + "_") or key.endswith("hex"):
                continue
            what = key[2:]
            x = np.ones((1, K), np.float32) if what == "ones" else _onehot(K, int(what[1:]))
            assert o.gemv_q6_k(W, x, 1, K)[0, 0] == float(v), (key, o.gemv_q6_k(W, x, 1, K))


def pin_q2_k_worked(o):
    g = read_golden("q2_k_block.txt")
    K = 256
    for blk in ("a", "b"):
        W = _hex(g[f"{blk}_hex"])
        assert W.size == 84
        for key, v in g.items():
            if not key.startswith(blk + "_") or key.endswith("hex"):
                continue
            what = key[2:]
            x = np.ones((1, K), np.float32) if what == "ones" else _onehot(K, int(what[1:]))
            assert o.gemv_q2_k(W, x, 1, K)[0, 0] == float(v), (key, o.gemv_q2_k(W, x, 1, K))


def pin_q1_0_worked(o):
    g = read_golden("q1_0_block.txt")
    K = 32
    for blk in ("a", "b"):
        W = _hex(g[f"{blk}_hex"])
        assert W.size == 6
        for key, v in g.items():
            if not key.startswith(blk + "_") or key.endswith("hex"):
                continue
            what = key[2:]
            x = np.ones((1, K), np.float32) if what == "ones" else _onehot(K, int(what[1:]))
            assert o.gemv_q1_0(W, x, 1, K)[0, 0] == float(v), (key, o.gemv_q1_0(W, x, 1, K))


def pin_i4g32_worked(o):
    g = read_golden("i4g32_block.txt")
    K = 64
    Wq = np.frombuffer(bytes.fromhex(g["words_hex"]), dtype="<u4").copy()
    sc = np.array([[float(v) for v in g["scales"].split()]], np.float32)
    z = np.array([[float(v) for v in g["zeros"].split()]], np.float32)
    for key, v in g.items():
        if key in ("words_hex", "scales", "zeros"):
            continue
        x = np.ones((1, K), np.float32) if key == "ones" else _onehot(K, int(key[1:]))
        assert o.gemv_i4g32(Wq, sc, z, x, 1, K)[0, 0] == float(v), key


def pin_packers_match_golden(o):
    """The generator's packers reproduce the hand-worked bytes (so the
    round-trip pins below test the oracle against the stated layout)."""
    g = read_golden("q4_0_block.txt")
    j = np.arange(16)
    q = np.concatenate([j, 15 - j]).astype(np.uint8)[None]
    got = synth.pack_q4_0(np.array([[1.0]], np.float16), q)
    assert got.tobytes().hex() == g["block_hex"]
    g8 = read_golden("q8_0_block.txt")
    q8 = (np.arange(32) - 16).astype(np.int8)[None]
    assert synth.pack_q8_0(np.array([[0.25]], np.float16), q8).tobytes().hex() == g8["a_hex"]
    gk = read_golden("q4_k_block.txt")
    sc = np.array([[1, 2, 3, 4, 63, 33, 17, 48]], np.uint8)
    m = np.array([[0, 1, 2, 3, 63, 40, 5, 32]], np.uint8)
    assert synth.pack_q4_k_scales(sc, m).tobytes().hex() == gk["scales_hex"]
    qk = np.ones((1, 256), np.uint8)
    blk = synth.pack_q4_k(np.array([[1.0]], np.float16), np.array([[0.5]], np.float16),
                          sc[None], m[None], qk)
    assert blk.tobytes().hex() == "003c0038" + gk["scales_hex"] + "11" * 128
    one = np.array([[1.0]], np.float16)
    k = np.arange(256)
    g6 = read_golden("q6_k_block.txt")
    a6 = synth.pack_q6_k(one, (np.arange(16) + 1).astype(np.int8)[None, None],
                         np.full((1, 256), 33, np.uint8))
    assert a6.tobytes().hex() == g6["a_hex"]
    b6 = synth.pack_q6_k(one, np.ones((1, 1, 16), np.int8), (k % 64).astype(np.uint8)[None])
    assert b6.tobytes().hex() == g6["b_hex"]
    g2 = read_golden("q2_k_block.txt")
    gg = np.arange(16)
    a2 = synth.pack_q2_k(one, np.array([[0.5]], np.float16), gg[None, None], (15 - gg)[None, None],
                         np.full((1, 256), 3, np.uint8))
    assert a2.tobytes().hex() == g2["a_hex"]
    qb = ((k % 32) + (k % 128) // 32) % 4
    b2 = synth.pack_q2_k(one, np.array([[0.0]], np.float16), np.ones((1, 1, 16)),
                         np.zeros((1, 1, 16)), qb.astype(np.uint8)[None])
    assert b2.tobytes().hex() == g2["b_hex"]
    g1 = read_golden("q1_0_block.txt")
    cb = np.unpackbits(np.array([0x01, 0x80, 0xF0, 0x0F], np.uint8), bitorder="little")[None]
    assert synth.pack_q1_0(np.array([[0.5]], np.float16), cb).tobytes().hex() == g1["b_hex"]
    gi = read_golden("i4g32_block.txt")
    codes = np.concatenate([np.arange(8), np.arange(-8, 0)] * 4)[None]
    assert synth.pack_i4g32(codes).astype("<u4").tobytes().hex() == gi["words_hex"]


# ---------------------------------------------------------------- round trip
def pin_round_trip(o):
    """Requantize the oracle's dequantized weights with each block's own
    scale(s): the generator's integer codes come back exactly."""
    c = synth.q4_0_case(37, 256, seed=3)
    w = o.dequant_q4_0(c.W, c.N, c.K)
    d = c.d.astype(np.float64).repeat(32, axis=1)
    nz = d != 0
    assert np.array_equal(w[nz] / d[nz] + 8, c.q.astype(np.float64)[nz])
    assert np.all(w[~nz] == 0)

    c8 = synth.q8_0_case(1, 29, 320, seed=4)
    w8 = o.dequant_q8_0(c8.W, c8.N, c8.K)
    d8 = c8.d.astype(np.float64).repeat(32, axis=1)
    nz = d8 != 0
    assert np.array_equal(w8[nz] / d8[nz], c8.q.astype(np.float64)[nz])

    ck = synth.q4_k_case(23, 512, seed=5)
    wk = o.dequant_q4_k(ck.W, ck.N, ck.K)
    N, nsb = ck.N, ck.K // 256
    dd = np.repeat(ck.d.astype(np.float64), 256, axis=1)
    dm = np.repeat(ck.dmin.astype(np.float64), 256, axis=1)
    sc = np.repeat(ck.sc.reshape(N, nsb * 8).astype(np.float64), 32, axis=1)
    mm = np.repeat(ck.m.reshape(N, nsb * 8).astype(np.float64), 32, axis=1)
    ok = (dd * sc) != 0
    qrec = (wk[ok] + dm[ok] * mm[ok]) / (dd[ok] * sc[ok])
    assert np.allclose(qrec, ck.q.astype(np.float64)[ok], rtol=0, atol=1e-9)
    assert np.array_equal(np.rint(qrec), ck.q.astype(np.float64)[ok])
    # where sc = 0 the weight is -dmin * m whatever q is
    z = ~ok & (dd != 0)
    assert np.array_equal(wk[z], -(dm[z] * mm[z]))

    c6 = synth.q6_k_case(9, 512, seed=31)
    w6 = o.dequant_q6_k(c6.W, c6.N, c6.K)
    ds = (np.repeat(c6.d.astype(np.float64), 256, axis=1)
          * np.repeat(c6.sc.reshape(c6.N, -1).astype(np.float64), 16, axis=1))
    nz = ds != 0
    assert np.array_equal(w6[nz] / ds[nz] + 32, c6.q.astype(np.float64)[nz])

    c2 = synth.q2_k_case(9, 512, seed=32)
    w2 = o.dequant_q2_k(c2.W, c2.N, c2.K)
    d2 = np.repeat(c2.d.astype(np.float64), 256, axis=1)
    m2 = np.repeat(c2.dmin.astype(np.float64), 256, axis=1)
    s2 = np.repeat(c2.sc.reshape(c2.N, -1).astype(np.float64), 16, axis=1)
    mm2 = np.repeat(c2.m.reshape(c2.N, -1).astype(np.float64), 16, axis=1)
    ok2 = (d2 * s2) != 0
    q2rec = (w2[ok2] + m2[ok2] * mm2[ok2]) / (d2[ok2] * s2[ok2])
    assert np.array_equal(np.rint(q2rec), c2.q.astype(np.float64)[ok2])
    assert np.allclose(q2rec, c2.q.astype(np.float64)[ok2], rtol=0, atol=1e-9)

    c1 = synth.q1_0_case(9, 256, seed=35)
    w1 = o.dequant_q1_0(c1.W, c1.N, c1.K)
    d1 = c1.d.astype(np.float64).repeat(32, axis=1)
    nz = d1 != 0
    assert np.array_equal((w1[nz] / d1[nz] + 1) / 2, c1.c.astype(np.float64)[nz])

    ci = synth.i4g32_case(7, 128, seed=33)
    wi = o.dequant_i4g32(ci.Wq, ci.scales, ci.zeros, ci.N, ci.K)
    scl = np.repeat(ci.scales.astype(np.float64), 32, axis=1)
    zr = np.repeat(ci.zeros.astype(np.float64), 32, axis=1)
    nz = scl != 0
    assert np.array_equal(wi[nz] / scl[nz] + zr[nz], ci.s.astype(np.float64)[nz])


# --------------------------------------------------- closed forms, invariants
def pin_closed_forms_q4_0(o):
    c = synth.q4_0_case(19, 192, seed=7)
    N, K = c.N, c.K
    ones = np.ones((1, K), np.float32)
    y = o.gemv_q4_0(c.W, ones, N, K)[0]
    # x = ones: y_n = sum over blocks of d * (sum q - 256)
    qs = c.q.reshape(N, K // 32, 32).astype(np.int64).sum(-1) - 256
    ref = (c.d.astype(np.float64) * qs).sum(-1)
    assert np.allclose(y, ref, rtol=1e-13, atol=0)
    # one-hot x extracts a column exactly
    for k in (0, 15, 16, 31, 100, 191):
        col = o.gemv_q4_0(c.W, _onehot(K, k), N, K)[0]
        ref = c.d[:, k // 32].astype(np.float64) * (c.q[:, k].astype(np.float64) - 8)
        assert np.array_equal(col, ref), k
    # linearity and batch independence
    rng = np.random.default_rng(11)
    xa = rng.standard_normal((1, K)).astype(np.float32)
    xb = rng.standard_normal((1, K)).astype(np.float32)
    ya, yb = o.gemv_q4_0(c.W, xa, N, K), o.gemv_q4_0(c.W, xb, N, K)
    ysum = o.gemv_q4_0(c.W, (xa.astype(np.float64) + xb).astype(np.float32), N, K)
    assert np.allclose(ysum, ya + yb, rtol=1e-6, atol=1e-6)  # x rounding to fp32 only
    yab = o.gemv_q4_0(c.W, np.concatenate([xa, xb]), N, K)
    assert np.array_equal(yab[0], ya[0]) and np.array_equal(yab[1], yb[0])
    # a row subset returns the same rows
    rows = [18, 0, 5]
    assert np.array_equal(o.gemv_q4_0(c.W, xa, N, K, rows=rows)[0], ya[0, rows])


def pin_closed_forms_q4_k(o):
    ck = synth.q4_k_case(11, 512, seed=8)
    N, K = ck.N, ck.K
    nsb = K // 256
    ones = np.ones((1, K), np.float32)
    y = o.gemv_q4_k(ck.W, ones, N, K)[0]
    qsum = ck.q.reshape(N, nsb, 8, 32).astype(np.int64).sum(-1)
    ref = (ck.d.astype(np.float64)[..., None] * ck.sc * qsum
           - 32 * ck.dmin.astype(np.float64)[..., None] * ck.m).sum((-1, -2))
    assert np.allclose(y, ref, rtol=1e-13, atol=1e-13)
    for k in (0, 31, 32, 63, 255, 256 + 77, 511):
        col = o.gemv_q4_k(ck.W, _onehot(K, k), N, K)[0]
        sb, s = k // 256, (k % 256) // 32
        ref = (ck.d[:, sb].astype(np.float64) * ck.sc[:, sb, s] * ck.q[:, k]
               - ck.dmin[:, sb].astype(np.float64) * ck.m[:, sb, s])
        assert np.array_equal(col, ref), k


def pin_closed_forms_gemm(o):
    c = synth.q8_0_case(5, 13, 96, seed=9)
    X1 = np.ones((1, c.K), np.float16)
    Y = o.gemm_q8_0_f16(c.W, X1, c.N, c.K)[0]
    ref = (c.d.astype(np.float64) * c.q.reshape(c.N, -1, 32).astype(np.int64).sum(-1)).sum(-1)
    assert np.allclose(Y, ref, rtol=1e-13, atol=0)
    # one-hot row of X extracts column k of W (row n of the weight matrix)
    Xe = np.zeros((1, c.K), np.float16)
    Xe[0, 40] = 1
    col = o.gemm_q8_0_f16(c.W, Xe, c.N, c.K)[0]
    assert np.array_equal(col, c.d[:, 1].astype(np.float64) * c.q[:, 40])
    cols = [12, 3]
    full = o.gemm_q8_0_f16(c.W, c.X, c.N, c.K)
    assert np.array_equal(o.gemm_q8_0_f16(c.W, c.X, c.N, c.K, cols=cols), full[:, cols])


def pin_closed_forms_new_formats(o):
    """x = ones gives integer-sum closed forms; one-hot x (or one-hot X rows
    for the GEMMs) gives a column, rebuilt from the generator's fields."""
    c8 = synth.q8_0_gemv_case(7, 160, seed=41)
    y = o.gemv_q8_0(c8.W, np.ones((1, c8.K), np.float32), c8.N, c8.K)[0]
    ref = (c8.d.astype(np.float64) * c8.q.reshape(c8.N, -1, 32).astype(np.int64).sum(-1)).sum(-1)
    assert np.allclose(y, ref, rtol=1e-13, atol=0)
    col = o.gemv_q8_0(c8.W, _onehot(c8.K, 77), c8.N, c8.K)[0]
    assert np.array_equal(col, c8.d[:, 2].astype(np.float64) * c8.q[:, 77])

    g0 = synth.q4_0_gemm_case(3, 6, 128, seed=42)
    X = np.zeros((2, g0.K), np.float16)
    X[0, 45] = 1
    X[1] = 1
    Y = o.gemm_q4_0_f16(g0.W, X, g0.N, g0.K)
    w = g0.w
    assert np.array_equal(Y[0], w.d[:, 1].astype(np.float64) * (w.q[:, 45].astype(np.float64) - 8))
    qs = w.q.reshape(w.N, -1, 32).astype(np.int64).sum(-1) - 256
    assert np.allclose(Y[1], (w.d.astype(np.float64) * qs).sum(-1), rtol=1e-13, atol=0)

    gk = synth.q4_k_gemm_case(2, 5, 512, seed=43)
    wk = gk.w
    X = np.zeros((1, gk.K), np.float16)
    X[0, 300] = 1
    Y = o.gemm_q4_k_f16(gk.W, X, gk.N, gk.K)[0]
    ref = (wk.d[:, 1].astype(np.float64) * wk.sc[:, 1, 1] * wk.q[:, 300]
           - wk.dmin[:, 1].astype(np.float64) * wk.m[:, 1, 1])
    assert np.array_equal(Y, ref)

    c6 = synth.q6_k_case(5, 256, seed=44)
    for k in (0, 47, 130, 255):
        col = o.gemv_q6_k(c6.W, _onehot(256, k), c6.N, 256)[0]
        ref = c6.d[:, 0].astype(np.float64) * c6.sc[:, 0, k // 16] * (c6.q[:, k].astype(np.int64) - 32)
        assert np.array_equal(col, ref), k
    c2 = synth.q2_k_case(5, 256, seed=45)
    y = o.gemv_q2_k(c2.W, np.ones((1, 256), np.float32), c2.N, 256)[0]
    qsum = c2.q.reshape(c2.N, 16, 16).astype(np.int64).sum(-1)
    ref = (c2.d[:, :1].astype(np.float64) * (c2.sc[:, 0] * qsum).sum(-1, keepdims=True)
           - 16 * c2.dmin[:, :1].astype(np.float64) * c2.m[:, 0].sum(-1, keepdims=True))[:, 0]
    assert np.allclose(y, ref, rtol=1e-13, atol=1e-13)
    c1 = synth.q1_0_case(6, 96, seed=47)
    y = o.gemv_q1_0(c1.W, np.ones((1, 96), np.float32), c1.N, 96)[0]
    pop = c1.c.reshape(c1.N, 3, 32).astype(np.int64).sum(-1)
    assert np.array_equal(y, (c1.d.astype(np.float64) * (2 * pop - 32)).sum(-1))
    col = o.gemv_q1_0(c1.W, _onehot(96, 70), c1.N, 96)[0]
    assert np.array_equal(col, c1.d[:, 2].astype(np.float64) * (2 * c1.c[:, 70].astype(np.int64) - 1))
    ci = synth.i4g32_case(4, 64, seed=46)
    col = o.gemv_i4g32(ci.Wq, ci.scales, ci.zeros, _onehot(64, 50), ci.N, 64)[0]
    ref = (ci.s[:, 50].astype(np.float64) - ci.zeros[:, 1]) * ci.scales[:, 1].astype(np.float64)
    assert np.array_equal(col, ref)


def pin_sgemm_identity(o):
    rng = np.random.default_rng(12)
    A = rng.uniform(-1, 1, (7, 5)).astype(np.float32)
    I5 = np.eye(5, dtype=np.float32)
    assert np.array_equal(o.sgemm(A, I5), A.astype(np.float64))
    B = rng.uniform(-1, 1, (5, 3)).astype(np.float32)
    E = np.zeros((7, 5), np.float32)
    E[2, 4] = 1
    C = o.sgemm(E, B)
    assert np.array_equal(C[2], B[4].astype(np.float64)) and not C[[0, 1, 3, 4, 5, 6]].any()
    # a row subset (any order) gives those rows of A * I = A
    rows = [6, 0, 3]
    assert np.array_equal(o.sgemm(A, I5, rows=rows), A[rows].astype(np.float64))


# ------------------------------------------------------ library-routine pins
def pin_numpy_crosscheck(o):
    """Medium shapes against numpy float64 products of weights rebuilt from the
    generator's integer fields (not from the bytes)."""
    c = synth.q4_0_case(64, 1024, batch=3, seed=13)
    W = c.d.astype(np.float64).repeat(32, axis=1) * (c.q.astype(np.float64) - 8)
    ref = c.x.astype(np.float64) @ W.T
    y = o.gemv_q4_0(c.W, c.x, c.N, c.K)
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())

    ck = synth.q4_k_case(32, 1024, batch=2, seed=14)
    N, nsb = ck.N, ck.K // 256
    dd = np.repeat(ck.d.astype(np.float64), 256, axis=1)
    dm = np.repeat(ck.dmin.astype(np.float64), 256, axis=1)
    sc = np.repeat(ck.sc.reshape(N, nsb * 8).astype(np.float64), 32, axis=1)
    mm = np.repeat(ck.m.reshape(N, nsb * 8).astype(np.float64), 32, axis=1)
    Wk = dd * sc * ck.q - dm * mm
    refk = ck.x.astype(np.float64) @ Wk.T
    yk = o.gemv_q4_k(ck.W, ck.x, ck.N, ck.K)
    assert np.allclose(yk, refk, rtol=1e-12, atol=1e-12 * np.abs(refk).max())

    c8 = synth.q8_0_case(24, 40, 512, seed=15)
    W8 = c8.d.astype(np.float64).repeat(32, axis=1) * c8.q.astype(np.float64)
    ref8 = c8.X.astype(np.float64) @ W8.T
    Y8 = o.gemm_q8_0_f16(c8.W, c8.X, c8.N, c8.K)
    assert np.allclose(Y8, ref8, rtol=1e-12, atol=1e-12 * np.abs(ref8).max())

    def close(got, ref):
        assert np.allclose(got, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())

    q8 = synth.q8_0_gemv_case(20, 512, batch=3, seed=17)
    W8v = q8.d.astype(np.float64).repeat(32, axis=1) * q8.q.astype(np.float64)
    close(o.gemv_q8_0(q8.W, q8.x, q8.N, q8.K), q8.x.astype(np.float64) @ W8v.T)

    g0 = synth.q4_0_gemm_case(9, 17, 256, seed=18)
    W0 = g0.w.d.astype(np.float64).repeat(32, axis=1) * (g0.w.q.astype(np.float64) - 8)
    close(o.gemm_q4_0_f16(g0.W, g0.X, g0.N, g0.K), g0.X.astype(np.float64) @ W0.T)

    gk = synth.q4_k_gemm_case(9, 11, 512, seed=19)
    w = gk.w
    n, nsb = w.N, w.K // 256
    Wg = (np.repeat(w.d.astype(np.float64), 256, axis=1)
          * np.repeat(w.sc.reshape(n, nsb * 8).astype(np.float64), 32, axis=1) * w.q
          - np.repeat(w.dmin.astype(np.float64), 256, axis=1)
          * np.repeat(w.m.reshape(n, nsb * 8).astype(np.float64), 32, axis=1))
    close(o.gemm_q4_k_f16(gk.W, gk.X, gk.N, gk.K), gk.X.astype(np.float64) @ Wg.T)

    c6 = synth.q6_k_case(13, 512, batch=2, seed=20)
    W6 = (np.repeat(c6.d.astype(np.float64), 256, axis=1)
          * np.repeat(c6.sc.reshape(c6.N, -1).astype(np.float64), 16, axis=1)
          * (c6.q.astype(np.float64) - 32))
    close(o.gemv_q6_k(c6.W, c6.x, c6.N, c6.K), c6.x.astype(np.float64) @ W6.T)

    c2 = synth.q2_k_case(13, 512, batch=2, seed=25)
    W2 = (np.repeat(c2.d.astype(np.float64), 256, axis=1)
          * np.repeat(c2.sc.reshape(c2.N, -1).astype(np.float64), 16, axis=1) * c2.q
          - np.repeat(c2.dmin.astype(np.float64), 256, axis=1)
          * np.repeat(c2.m.reshape(c2.N, -1).astype(np.float64), 16, axis=1))
    close(o.gemv_q2_k(c2.W, c2.x, c2.N, c2.K), c2.x.astype(np.float64) @ W2.T)

    c1 = synth.q1_0_case(13, 256, batch=2, seed=36)
    W1 = c1.d.astype(np.float64).repeat(32, axis=1) * (2 * c1.c.astype(np.float64) - 1)
    close(o.gemv_q1_0(c1.W, c1.x, c1.N, c1.K), c1.x.astype(np.float64) @ W1.T)

    ci = synth.i4g32_case(13, 256, batch=2, seed=26)
    Wi = ((ci.s.astype(np.float64) - np.repeat(ci.zeros.astype(np.float64), 32, axis=1))
          * np.repeat(ci.scales.astype(np.float64), 32, axis=1))
    close(o.gemv_i4g32(ci.Wq, ci.scales, ci.zeros, ci.x, ci.N, ci.K), ci.x.astype(np.float64) @ Wi.T)

    s = synth.sgemm_case(33, 47, 129, seed=16)
    refs = s.A.astype(np.float64) @ s.B.astype(np.float64)
    Cs = o.sgemm(s.A, s.B)
    assert np.allclose(Cs, refs, rtol=1e-12, atol=1e-12 * np.abs(refs).max())


# ------------------------------------------------------------- brute force
def _F(v) -> Fraction:
    return Fraction(float(v))


def pin_brute_force(o):
    """Exact rational sums on tiny shapes; the double oracle agrees to 1e-12
    relative (only its summation rounds)."""
    c = synth.q4_0_case(4, 64, batch=2, seed=21)
    y = o.gemv_q4_0(c.W, c.x, c.N, c.K)
    for b in range(c.batch):
        for n in range(c.N):
            ex = sum(_F(c.d[n, k // 32]) * (int(c.q[n, k]) - 8) * _F(c.x[b, k]) for k in range(c.K))
            assert abs(Fraction(y[b, n]) - ex) <= Fraction(1, 10**12) * max(abs(ex), Fraction(1, 10**6))

    ck = synth.q4_k_case(3, 256, batch=2, seed=22)
    yk = o.gemv_q4_k(ck.W, ck.x, ck.N, ck.K)
    for b in range(ck.batch):
        for n in range(ck.N):
            ex = Fraction(0)
            for k in range(ck.K):
                s = k // 32
                w = (_F(ck.d[n, 0]) * int(ck.sc[n, 0, s]) * int(ck.q[n, k])
                     - _F(ck.dmin[n, 0]) * int(ck.m[n, 0, s]))
                ex += w * _F(ck.x[b, k])
            assert abs(Fraction(yk[b, n]) - ex) <= Fraction(1, 10**12) * max(abs(ex), Fraction(1, 10**6))

    c8 = synth.q8_0_case(3, 4, 64, seed=23)
    Y8 = o.gemm_q8_0_f16(c8.W, c8.X, c8.N, c8.K)
    for m in range(c8.M):
        for n in range(c8.N):
            ex = sum(_F(c8.X[m, k]) * _F(c8.d[n, k // 32]) * int(c8.q[n, k]) for k in range(c8.K))
            assert abs(Fraction(Y8[m, n]) - ex) <= Fraction(1, 10**12) * max(abs(ex), Fraction(1, 10**6))

    def exact_ok(got, ex):
        assert abs(Fraction(got) - ex) <= Fraction(1, 10**12) * max(abs(ex), Fraction(1, 10**6))

    c6 = synth.q6_k_case(2, 256, batch=1, seed=27)
    y6 = o.gemv_q6_k(c6.W, c6.x, c6.N, c6.K)
    for n in range(c6.N):
        exact_ok(y6[0, n], sum(_F(c6.d[n, 0]) * int(c6.sc[n, 0, k // 16]) * (int(c6.q[n, k]) - 32)
                               * _F(c6.x[0, k]) for k in range(256)))
    c2 = synth.q2_k_case(2, 256, batch=1, seed=28)
    y2 = o.gemv_q2_k(c2.W, c2.x, c2.N, c2.K)
    for n in range(c2.N):
        exact_ok(y2[0, n], sum((_F(c2.d[n, 0]) * int(c2.sc[n, 0, k // 16]) * int(c2.q[n, k])
                                - _F(c2.dmin[n, 0]) * int(c2.m[n, 0, k // 16])) * _F(c2.x[0, k])
                               for k in range(256)))
    ci = synth.i4g32_case(2, 64, batch=2, seed=29)
    yi = o.gemv_i4g32(ci.Wq, ci.scales, ci.zeros, ci.x, ci.N, ci.K)
    for b in range(2):
        for n in range(ci.N):
            exact_ok(yi[b, n], sum((int(ci.s[n, k]) - _F(ci.zeros[n, k // 32]))
                                   * _F(ci.scales[n, k // 32]) * _F(ci.x[b, k]) for k in range(64)))
    c1 = synth.q1_0_case(2, 64, batch=2, seed=37)
    y1 = o.gemv_q1_0(c1.W, c1.x, c1.N, c1.K)
    for b in range(2):
        for n in range(c1.N):
            exact_ok(y1[b, n], sum(_F(c1.d[n, k // 32]) * (2 * int(c1.c[n, k]) - 1) * _F(c1.x[b, k])
                                   for k in range(64)))
    q8 = synth.q8_0_gemv_case(2, 64, batch=1, seed=30)
    y8 = o.gemv_q8_0(q8.W, q8.x, q8.N, q8.K)
    for n in range(q8.N):
        exact_ok(y8[0, n], sum(_F(q8.d[n, k // 32]) * int(q8.q[n, k]) * _F(q8.x[0, k])
                               for k in range(64)))
    gk = synth.q4_k_gemm_case(2, 2, 256, seed=34)
    Yk = o.gemm_q4_k_f16(gk.W, gk.X, gk.N, gk.K)
    w = gk.w
    for m in range(2):
        for n in range(2):
            exact_ok(Yk[m, n], sum(_F(gk.X[m, k]) * (_F(w.d[n, 0]) * int(w.sc[n, 0, k // 32])
                                                      * int(w.q[n, k])
                                                      - _F(w.dmin[n, 0]) * int(w.m[n, 0, k // 32]))
                                   for k in range(256)))

    s = synth.sgemm_case(3, 5, 7, seed=24)
    Cs = o.sgemm(s.A, s.B)
    for i in range(3):
        for j in range(5):
            ex = sum(_F(s.A[i, k]) * _F(s.B[k, j]) for k in range(7))
            assert abs(Fraction(Cs[i, j]) - ex) <= Fraction(1, 10**12) * max(abs(ex), Fraction(1, 10**6))


def pin_subnormal_scales(o):
    """fp16 subnormal scales are honoured: d = 0x0001 is 2^-24."""
    j = np.arange(16)
    q = np.concatenate([j, 15 - j]).astype(np.uint8)[None]
    d = np.array([[0x0001]], np.uint16).view(np.float16)
    W = synth.pack_q4_0(d, q)
    y = o.gemv_q4_0(W, np.ones((1, 32), np.float32), 1, 32)
    assert y[0, 0] == -16 * 2.0 ** -24


PINS = [pin_f16_exhaustive, pin_q4_0_worked, pin_q8_0_worked, pin_q4_k_worked,
        pin_q8_0_gemv_worked, pin_gemm_q4_worked, pin_q6_k_worked, pin_q2_k_worked,
        pin_q1_0_worked, pin_i4g32_worked, pin_packers_match_golden, pin_round_trip, pin_closed_forms_q4_0,
        pin_closed_forms_q4_k, pin_closed_forms_gemm, pin_closed_forms_new_formats,
        pin_sgemm_identity, pin_numpy_crosscheck, pin_brute_force, pin_subnormal_scales]
