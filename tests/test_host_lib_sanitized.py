"""The library's host code -- frame-set capacity, construction and validation,
the chunk-aware growth schedule and the error text (csrc/frame_sets_host.cpp
with the per-frame routine the device kernel runs, csrc/cag.cpp,
csrc/errors.cpp) -- built with g++ under the address and undefined-behaviour
sanitizers and driven through a small host program: its results must equal
the oracle's, and the sanitizers must stay silent (any report fails the run)."""

import os
import shutil
import struct
import subprocess

import numpy as np
import pytest

import workloads as wl
from oracle import cag as ocag
from oracle import frame_sets as ofs

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "frame_sparse_attention_amd", "csrc")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
FIELDS = ("kind", "n_sink", "window", "budget", "t_per", "step", "topk", "n_recent", "lo", "hi")


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.exists(os.path.join(ROCM, "include", "hip")):
        pytest.skip("g++ or the HIP headers are not available")
    exe = str(tmp_path_factory.mktemp("hostlib") / "host_lib_check")
    srcs = [os.path.join(HERE, "host", "host_lib_check.cpp")] + [
        os.path.join(CSRC, f) for f in ("frame_sets_host.cpp", "cag.cpp", "errors.cpp")]
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-DFSA_HD=", "-D__HIP_PLATFORM_AMD__",
           f"-I{ROOT}/include", f"-I{CSRC}", f"-I{ROCM}/include",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", *srcs, "-o", exe,
           f"-L{ROCM}/lib", "-lamdhip64", f"-Wl,-rpath,{ROCM}/lib"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    return exe


def _run(exe, text):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="halt_on_error=1")
    r = subprocess.run([exe], input=text, capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0 and "runtime error" not in r.stderr, r.stderr[-3000:]
    return r.stdout.strip().split("\n")


def _pol(p):
    return " ".join(str(int(p.get(f, 1 if f == "t_per" else (-1 if f == "hi" else 0))))
                    for f in FIELDS)


def _build_cmd(pols, B, Tq, Tk, off, chunk, topk, cap, sel=None):
    s = f"B {B} {len(pols)} {Tq} {Tk} {off} {chunk} {topk} {cap} " + " ".join(_pol(p) for p in pols)
    if topk > 0:
        s += " " + " ".join(str(int(v)) for v in sel.ravel())
    return s + "\n"


def _cases():
    rng = np.random.default_rng(3)
    out = []
    for make in (wl.tiny_f32, wl.lvsa_shaped, wl.ar_chunk, wl.decomposable, wl.long_video):
        w = make()
        for s in range(min(w.steps, 3)):
            ws = w.with_step(s)
            out.append((ws.policies, ws.B, ws.Tq, ws.Tk, ws.offset, ws.chunk))
            out.extend((p, ws.B, ws.Tq, ws.Tk, ws.offset, ws.chunk) for p in ws.branches.values())
    for Tk in (1, 3, 8, 20):
        for chunk in (1, 2, 4):
            off = max(0, Tk - 2 * chunk)
            Tq = ((Tk - off) // chunk) * chunk
            if Tq == 0:
                continue
            pols = [wl.policy(wl.SINK_WINDOW, n_sink=ns, window=w_) for ns in (0, 2, 30)
                    for w_ in (0, 1, 5)]
            pols += [wl.policy(wl.MEMORY, topk=2, n_recent=nr) for nr in (0, 1, 3)]
            pols += [wl.policy(wl.LVSA, window=int(rng.integers(0, 6)), budget=int(rng.integers(0, 9)),
                               t_per=int(rng.integers(1, 5)), step=int(rng.integers(-3, 7)))
                     for _ in range(4)]
            pols += [wl.policy(wl.RANGE, lo=-2, hi=Tk + 3), wl.policy(wl.FULL)]
            out.append((pols, 2, Tq, Tk, off, chunk))
    return out


def test_frame_sets_match_oracle_under_sanitizers(driver):
    rng = np.random.default_rng(4)
    text, refs = "", []
    for pols, B, Tq, Tk, off, chunk in _cases():
        cap = max(1, max(len(ofs.frame_set_for(p, Tq, Tk, off, chunk, t, list(range(Tk))))
                         for p in pols for t in range(Tq)))
        topk = max([p["topk"] for p in pols if p["kind"] == wl.MEMORY], default=0)
        sel = None
        sel_lists = None
        if topk:
            # selections include frames outside [0, Tk): the library skips them
            sel = rng.integers(-2, Tk + 2, size=(B, len(pols), Tq // chunk, topk)).astype(np.int32)
            sel_lists = [[[[f for f in sel[b, h, g, :pols[h]["topk"]] if 0 <= f < Tk]
                           for g in range(Tq // chunk)] for h in range(len(pols))]
                         for b in range(B)]
        text += f"C {len(pols)} {Tq} {Tk} {off} {chunk} " + " ".join(_pol(p) for p in pols) + "\n"
        text += _build_cmd(pols, B, Tq, Tk, off, chunk, topk, cap, sel)
        refs.append(ofs.build(pols, B, Tq, Tk, off, chunk, sel_lists, cap=cap))
    lines = _run(driver, text)
    assert len(lines) == 2 * len(refs)
    for i, (oidx, ocnt) in enumerate(refs):
        st, lib_cap = map(int, lines[2 * i].split())
        assert st == 0 and lib_cap >= ocnt.max()
        vals = list(map(int, lines[2 * i + 1].split()))
        assert vals[0] == 0, f"case {i}: status {vals[0]}"
        n = ocnt.size
        assert vals[1:1 + n] == ocnt.ravel().tolist(), f"case {i}: counts"
        assert vals[1 + n:] == oidx.ravel().tolist(), f"case {i}: lists"


def test_validator_under_sanitizers(driver):
    good = np.array([[[[0, 2, 5, -1], [1, -1, -1, -1]]]], dtype=np.int32)
    cnt = np.array([[[3, 1]]], dtype=np.int32)
    cases = [(good, cnt, 6, 0)]
    bad = good.copy(); bad[0, 0, 0, 1] = 0
    cases.append((bad, cnt, 6, 5))                           # duplicate
    bad = good.copy(); bad[0, 0, 0, 2] = 1
    cases.append((bad, cnt, 6, 5))                           # unsorted
    cases.append((good, cnt, 5, 5))                          # out of range
    cases.append((good, np.array([[[5, 1]]], np.int32), 6, 5))   # cnt > cap
    cases.append((good, np.array([[[-1, 1]]], np.int32), 6, 5))  # negative cnt
    text = "".join(f"V 1 1 2 {Tk} 4 " + " ".join(map(str, i.ravel())) + " "
                   + " ".join(map(str, c.ravel())) + "\n" for i, c, Tk, _ in cases)
    lines = _run(driver, text)
    assert [int(x) for x in lines] == [want for *_, want in cases]


def _hx(x: float) -> str:
    return struct.pack(">d", x).hex()


def test_cag_schedule_matches_oracle_under_sanitizers(driver):
    rng = np.random.default_rng(5)
    cases = []
    for seed in range(10):
        n = int(rng.integers(1, 70))
        cost = (np.arange(1, n + 1, dtype=np.float64) if seed % 2 else rng.uniform(0.5, 4.0, n))
        s_max = float(rng.uniform(0.5, 0.98))
        s_base = float(rng.uniform(0.0, 1.0))
        reach = s_max * (cost[1:].sum() / cost.sum()) if n > 1 else 0.0
        s_target = float(rng.uniform(0.0, 0.95 * reach)) if reach > 0 else 0.0
        cand = rng.integers(1, 200, n)
        cases.append((cost, s_target, s_base, s_max, cand))
    cases.append((np.array([1.0, 0.0]), 0.3, 0.5, 0.8, np.array([3, 3])))    # bad cost
    text = "".join(f"S {len(c)} {_hx(a)} {_hx(b)} {_hx(m)} " + " ".join(_hx(x) for x in c) + " "
                   + " ".join(map(str, k)) + "\n" for c, a, b, m, k in cases)
    lines = _run(driver, text)
    for (cost, st_, sb, sm, cand), line in zip(cases, lines):
        parts = line.split()
        if cost.min() <= 0:
            assert parts == ["1", "error-text"]
            continue
        assert parts[0] == "0"
        n = len(cost)
        dec = [struct.unpack(">d", bytes.fromhex(p.zfill(16)))[0] for p in parts[1:2 + n]]
        osp, obeta = ocag.schedule(cost.tolist(), st_, sb, sm)
        assert dec[0] == obeta and dec[1:] == osp
        assert list(map(int, parts[2 + n:])) == ocag.frame_budgets(osp, cand.tolist())
