"""The kernels' scalar helpers (bf16 directed rounding, 8x8 bit transpose),
compiled for the host and checked against the oracle's bf16 rounding and a
direct bit-by-bit transpose."""
import os
import subprocess

import numpy as np
import pytest

import oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def probe(tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("probe") / "bitops_probe")
    r = subprocess.run(["g++", "-O2", "-std=c++17", "-I",
                        os.path.join(ROOT, "query_adaptive_decode_amd", "csrc"),
                        os.path.join(ROOT, "tests", "cpu", "bitops_probe.cpp"), "-o", exe],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return exe


def _run(exe, lines):
    r = subprocess.run([exe], input="\n".join(lines) + "\n", capture_output=True, text=True)
    assert r.returncode == 0
    return r.stdout.split()


def test_bf16_directed_rounding_matches_oracle(probe):
    rng = np.random.default_rng(0)
    v = np.concatenate([
        rng.standard_normal(3000) * 10.0 ** rng.integers(-45, 39, 3000),
        np.array([0.0, -0.0, 1.0, -1.0, 3.3e38, -3.3e38, 3.4e38, 1e-39, -1e-39, 2.0 ** -133,
                  2.0 ** -134, 2.0 ** -126, 1.5 * 2.0 ** -126, 0.1, -0.1]),
        # float32 values and exact bf16 values
        rng.standard_normal(500).astype(np.float32).astype(np.float64),
        (rng.integers(0, 0x7F7F, 500).astype(np.uint32) << 16).view(np.float32).astype(np.float64),
    ])
    v = v[np.isfinite(v)]
    lines = []
    for x in v:
        b = np.float64(x).view(np.uint64)
        lines += [f"r {int(b):x} 0", f"r {int(b):x} 1"]
    out = [int(s, 16) for s in _run(probe, lines)]
    got_dn = np.array(out[0::2], dtype=np.uint32)
    got_up = np.array(out[1::2], dtype=np.uint32)

    def tobits(x):
        x = np.where(x == 0, 0.0, x)              # +0 for zero results
        return (x.astype(np.float32).view(np.uint32) >> 16).astype(np.uint32)

    assert np.array_equal(got_dn, tobits(O.bf16_down(v)))
    assert np.array_equal(got_up, tobits(O.bf16_up(v)))


def test_transpose8_is_bit_transpose(probe):
    rng = np.random.default_rng(1)
    xs = [int(x) for x in rng.integers(0, 2 ** 63, 200, dtype=np.int64)] + [0, 1, 1 << 63, 0xFF, 2 ** 64 - 1]
    out = [int(s, 16) for s in _run(probe, [f"t {x:x}" for x in xs])]
    for x, y in zip(xs, out):
        want = 0
        for r in range(8):
            for c in range(8):
                if (x >> (8 * r + c)) & 1:
                    want |= 1 << (8 * c + r)
        assert y == want


def test_transpose8_halves_matches_64bit_form(probe):
    rng = np.random.default_rng(2)
    xs = [int(x) for x in rng.integers(0, 2 ** 63, 300, dtype=np.int64)] + [0, 2 ** 64 - 1, 1 << 63, 0xFF]
    want = [int(s, 16) for s in _run(probe, [f"t {x:x}" for x in xs])]
    got = [int(s, 16) for s in _run(probe, [f"h {x:x}" for x in xs])]
    assert got == want


def _perm_ref(a, b, sel):
    v = (a << 32) | b
    r = 0
    for i in range(4):
        s = (sel >> (8 * i)) & 0xFF
        byte = (v >> (8 * s)) & 0xFF if s < 8 else (0 if s == 0x0C else 0xFF)
        r |= byte << (8 * i)
    return r


def test_byte_gather_and_unplane_give_prefix_codes(probe):
    """The kernels' un-plane: gather byte `ob` of plane words w0..w7 with two
    levels of byte permutes, transpose, and read token i's code from byte i.
    Checked against direct bit extraction, with the permute model itself
    checked against a direct byte-select reference."""
    rng = np.random.default_rng(3)
    lines = []
    cases = []
    for _ in range(60):
        w = [int(x) for x in rng.integers(0, 2 ** 32, 8, dtype=np.uint64)]
        t = int(rng.integers(1, 9))
        w = [w[p] if p < t else 0 for p in range(8)]
        ob = int(rng.integers(0, 4))
        sel = 0x0C0C0000 | ((4 + ob) << 8) | ob
        cases.append((w, t, ob, sel))
        lines += [f"p {w[0]:x} {w[1]:x} {sel:x}", f"p {w[2]:x} {w[3]:x} {sel:x}",
                  f"p {w[4]:x} {w[5]:x} {sel:x}", f"p {w[6]:x} {w[7]:x} {sel:x}"]
    out = [int(s, 16) for s in _run(probe, lines)]
    lines2 = []
    for k, (w, t, ob, sel) in enumerate(cases):
        r01, r23, r45, r67 = out[4 * k:4 * k + 4]
        assert r01 == _perm_ref(w[0], w[1], sel) and r67 == _perm_ref(w[6], w[7], sel)
        lines2 += [f"p {r01:x} {r23:x} 5040100", f"p {r45:x} {r67:x} 5040100"]
    out2 = [int(s, 16) for s in _run(probe, lines2)]
    lines3 = [f"h {(out2[2 * k] << 32) | out2[2 * k + 1]:x}" for k in range(len(cases))]
    ys = [int(s, 16) for s in _run(probe, lines3)]
    for (w, t, ob, sel), y in zip(cases, ys):
        for i in range(8):
            tok = 8 * ob + i
            want = sum(((w[p] >> tok) & 1) << (7 - p) for p in range(8))
            assert (y >> (8 * i)) & 0xFF == want
