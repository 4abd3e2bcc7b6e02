"""The library's exact-sum code (csrc/exact_sum.h, used by the device pooling
of frame and block selection) built for the host with g++ under the address
and undefined-behaviour sanitizers, against exact rational arithmetic: every
sum must be the exact sum rounded once to float64 (fractions.Fraction, whose
conversion to float rounds correctly), and whenever the cheap test
exact_by_range accepts a set of values, plain float64 sums in two orders must
give that same value."""

import os
import shutil
import struct
import subprocess
from fractions import Fraction

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(os.path.dirname(HERE), "frame_sparse_attention_amd", "csrc")
SRC = os.path.join(HERE, "host", "exact_sum_check.cpp")

BF16, F32 = 7, 23


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ is not available")
    exe = str(tmp_path_factory.mktemp("exact") / "exact_sum_check")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-DFSA_HD=", f"-I{CSRC}",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", SRC, "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    return exe


def _f32_bits(x: float) -> int:
    return struct.unpack("<I", struct.pack("<f", x))[0]


def _value(b: int) -> float:
    return struct.unpack("<f", struct.pack("<I", b))[0]


def _run(exe, cases):
    text = "".join(f"{mb} {len(bs)} " + " ".join(f"{b:x}" for b in bs) + "\n"
                   for mb, bs in cases)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", UBSAN_OPTIONS="halt_on_error=1")
    r = subprocess.run([exe], input=text, capture_output=True, text=True, env=env)
    assert r.returncode == 0, r.stderr[-2000:]
    out = []
    for line in r.stdout.split("\n")[:len(cases)]:
        a, c, f, b = line.split()
        out.append((struct.unpack("<d", bytes.fromhex(a)[::-1])[0], c == "1",
                    struct.unpack("<d", bytes.fromhex(f)[::-1])[0],
                    struct.unpack("<d", bytes.fromhex(b)[::-1])[0]))
    return out


def _exact(bits) -> float:
    return float(sum(Fraction(_value(b)) for b in bits)) + 0.0


def _check(exe, cases):
    res = _run(exe, cases)
    n_cheap = 0
    for (mb, bits), (got, cheap, fwd, bwd) in zip(cases, res):
        want = _exact(bits)
        assert struct.pack("<d", got) == struct.pack("<d", want), (mb, bits[:8], got, want)
        if cheap:
            n_cheap += 1
            assert fwd == want and bwd == want, (bits[:8], fwd, bwd, want)
    return n_cheap


def test_special_cases(driver):
    p = 2.0
    cases = [
        (F32, [_f32_bits(p**100), _f32_bits(p**47)]),                    # tie -> even (down)
        (F32, [_f32_bits(p**100), _f32_bits(p**48), _f32_bits(p**47)]),  # tie -> even (up)
        (F32, [_f32_bits(p**100), _f32_bits(p**47), 1]),                 # just above the tie
        (F32, [_f32_bits(-p**100), _f32_bits(-p**47), 0x80000001]),      # the same, negative
        (F32, [_f32_bits(3e38), _f32_bits(1e-38), _f32_bits(-3e38)]),    # extremes cancel
        (F32, [0x7F7FFFFF] * 7 + [0xFF7FFFFF] * 3),                      # largest floats
        (F32, [1, 1, 0x80000003]),                                       # subnormals: -1 ulp
        (F32, [0x80000000, 0x80000000]),                                 # -0 + -0 = +0
        (F32, []),
        (BF16, [_f32_bits(1e16) & 0xFFFF0000, 0x3F800000, _f32_bits(-1e16) & 0xFFFF0000,
                0x3F800000]),
        (F32, [_f32_bits(0.1)] * 10),
    ]
    _check(driver, cases)


@pytest.mark.parametrize("seed", range(6))
def test_random_sums_match_rational_arithmetic(driver, seed):
    rng = np.random.default_rng(900 + seed)
    cases = []
    for n in (1, 2, 3, 17, 120, 1560):
        # bf16 values of normal spread (the cheap case), and of 250 binades
        x = rng.standard_normal(n).astype(np.float32).view(np.uint32) & 0xFFFF0000
        cases.append((BF16, [int(b) for b in x]))
        e = rng.integers(1, 255, n)
        m = rng.integers(0, 1 << 7, n)
        s = rng.integers(0, 2, n)
        cases.append((BF16, [int((sv << 31) | (ev << 23) | (mv << 16))
                             for sv, ev, mv in zip(s, e, m)]))
        # float32 values, with some subnormals and exact negatives of others
        y = (rng.standard_normal(n) * np.exp2(rng.integers(-30, 30, n))).astype(np.float32)
        b = y.view(np.uint32).astype(np.int64)
        if n > 4:
            b[: n // 4] = rng.integers(1, 1 << 23, n // 4)
            b[n // 4: n // 2] = b[n // 2: n // 2 + (n // 2 - n // 4)] ^ 0x80000000
        cases.append((F32, [int(v) for v in b]))
    n_cheap = _check(driver, cases)
    assert n_cheap >= 6     # the normal-spread bf16 cases take the cheap path


def test_long_segment(driver):
    rng = np.random.default_rng(7)
    x = (rng.standard_normal(5000) * 8).astype(np.float32).view(np.uint32) & 0xFFFF0000
    x[17] = 0x7E800000            # one value 2^126: the cheap test must refuse
    assert _check(driver, [(BF16, [int(b) for b in x])]) == 0
