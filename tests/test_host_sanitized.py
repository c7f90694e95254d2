"""The C ABI's host side (argument checks and ring bookkeeping) built with
AddressSanitizer and UndefinedBehaviorSanitizer and driven on
bookkeeping-only caches: every command's return code and the resulting
page list must match the float64 oracle's naive ring cache, and the
sanitizers must stay silent.  The kernel launchers are stubs that abort
(tests/host_asan/stubs.cpp); nothing here touches a GPU."""
import os
import random
import shutil
import subprocess

import numpy as np
import pytest

from oracle import CacheConfig, NaiveRingCache, RingError

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "sliding_window_kv_amd", "csrc")
CLANG = "/opt/rocm/llvm/bin/clang++"


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    if not os.path.exists(CLANG) or not os.path.exists("/opt/rocm/lib/libamdhip64.so"):
        pytest.skip("ROCm clang++ or the HIP runtime library not available")
    out = tmp_path_factory.mktemp("asan")
    exe = str(out / "driver")
    # host code only: plain C++ compiles, no device code, sanitizers on the host
    flags = ["-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
             "-D__HIP_PLATFORM_AMD__", "-I" + os.path.join(ROOT, "include"), "-I" + CSRC, "-I/opt/rocm/include"]
    srcs = [os.path.join(CSRC, "swa_api.cpp"), os.path.join(CSRC, "ring.cpp"),
            os.path.join(HERE, "host_asan", "stubs.cpp"), os.path.join(HERE, "host_asan", "driver.cpp")]
    r = subprocess.run([CLANG] + flags + srcs + ["-L/opt/rocm/lib", "-Wl,-rpath,/opt/rocm/lib", "-lamdhip64",
                                                  "-o", exe], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-3000:]
    return exe


def _run(exe, commands):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], input="\n".join(commands) + "\n", capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, (r.returncode, r.stderr[-3000:])
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr[-3000:]
    return r.stdout.split("\n")


def _kv(P):
    z = np.zeros((P, 1, 1))
    return z, z


def test_error_paths_without_a_device(driver):
    out = _run(driver, [])
    assert out[0] == "E0 -1 0"                      # null handle pointer / invalid config
    assert out[1] == "E1 -1"                        # null graph
    assert out[2] == "E2 0 0"                       # decode size queries with invalid shapes


@pytest.mark.parametrize("seed", range(12))
def test_random_call_sequences_match_oracle(driver, seed):
    rng = random.Random(seed)
    P = rng.randint(5, 40)
    W = rng.choice([-1, 1, 2, 3, 5])
    nfpb = rng.choice([1, 1, 2])
    S = rng.randint(0, 3)
    cross = rng.random() < 0.5
    ns = rng.randint(1, min(5, P))
    R = rng.randint(1, 6)
    maxf = 12
    cmds = [f"C {P} {W} {nfpb} {S} {int(cross)} {ns} {R} {maxf}"]
    ora = NaiveRingCache(CacheConfig(P=P, sliding_window_size=W, num_frame_per_block=nfpb, scale_frames=S,
                                     cross_frame_special=cross, special_row0=0, special_rows=ns,
                                     max_special_frames=R, max_frames=maxf))
    expect = []
    t = 0
    for _ in range(150):
        op = rng.choice(["key", "key", "key", "nonkey", "evict", "evict", "rollback", "reset", "stale"])
        err = False
        try:
            if op in ("key", "nonkey", "stale"):
                tt = t - 2 if op == "stale" else t
                cmds.append(f"A {tt} {int(op != 'nonkey')}")
                ora.append(tt, *_kv(P), op != "nonkey")
            elif op == "evict":
                cmds.append("E")
                ora.evict()
            elif op == "rollback":
                cmds.append("R")
                ora.rollback()
            else:
                cmds.append("X")
                ora.reset()
        except RingError:
            err = True
        if op in ("key", "nonkey") and not err:
            t += 1
        if op == "reset":
            t = 0
        expect.append((err, [tuple(p) for p in ora.visible_pages()]))
    out = _run(driver, cmds)
    lines = [l for l in out[3:] if l]
    assert lines[0] == "G -2"                       # a bookkeeping-only cache cannot capture a step
    assert lines[1] == "C 0"
    body = lines[3:]                                # after the create's own page line
    assert len(body) == 2 * len(expect)
    for i, (err, pages) in enumerate(expect):
        op, rc = body[2 * i].split()
        assert (int(rc) != 0) == err, (i, cmds[i + 1], rc)
        f = [int(x) for x in body[2 * i + 1].split()[1:]]
        got = [tuple(f[1 + 5 * j: 6 + 5 * j]) for j in range(f[0])]
        assert got == pages, (i, cmds[i + 1])
