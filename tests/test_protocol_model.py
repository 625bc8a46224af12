"""CPU model of the AG-GEMM copy / flag protocol (tests/protocol/
ag_protocol_model.cpp) under ThreadSanitizer: std::thread workgroups run the
kernels' ticket, counter and flag protocol on the library's closed-form
schedule, for the inline and side-producer transfers, both chunk orders,
several K-slab widths, split K (tiles as two K halves combined through a
stored sum and a per-tile flag) and repeated calls on one workspace. TSan
must report no race (every read of gathered rows, and of a stored half's
sum, is ordered after its publish), and must report one when the model's
publish is made relaxed (a planted mistake; also in the split-K combine
alone). A dead producer (a flag never published) must time out, set the
error word and still let every thread finish."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "protocol", "ag_protocol_model.cpp")


@pytest.fixture(scope="module")
def model(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path_factory.mktemp("protocol") / "ag_protocol_model")
    # CPU-only build with ThreadSanitizer (no GPU code is involved)
    res = subprocess.run([gxx, "-std=c++17", "-O1", "-g", "-fsanitize=thread", "-pthread", SRC, "-o", exe],
                         capture_output=True, text=True, timeout=300)
    if res.returncode != 0 and "tsan" in res.stderr.lower():
        pytest.skip("ThreadSanitizer runtime not available")
    assert res.returncode == 0, res.stderr
    return exe


def run(exe, *args, timeout=120):
    env = dict(os.environ, TSAN_OPTIONS="halt_on_error=0 exitcode=66")
    return subprocess.run([exe, *args], capture_output=True, text=True, timeout=timeout, env=env)


@pytest.mark.parametrize("args", [[], ["--inline"], ["--natural"], ["--local", "3"], ["--inline", "--local", "0"],
                                  ["--kslab", "1024"], ["--kslab", "512", "--local", "2"],
                                  ["--calls", "5", "--natural", "--inline"], ["--split"],
                                  ["--split", "--local", "0", "--calls", "5"], ["--split", "--natural"]],
                         ids=lambda a: " ".join(a) or "side")
def test_protocol_race_free(model, args):
    r = run(model, *args)
    assert "ThreadSanitizer" not in r.stderr, r.stderr[-3000:]
    assert r.returncode == 0, r.stdout + r.stderr[-2000:]
    assert r.stdout.strip().endswith("ok")


def test_planted_relaxed_publish_is_caught(model):
    r = run(model, "--relaxed", "--calls", "1")
    assert "WARNING: ThreadSanitizer: data race" in r.stderr
    assert r.returncode == 66


def test_planted_relaxed_split_publish_is_caught(model):
    # split K: the halves' combine reads the first half's sum after the
    # tile flag; a relaxed flag leaves that read unordered
    r = run(model, "--split", "--relaxed-split", "--calls", "1")
    assert "WARNING: ThreadSanitizer: data race" in r.stderr
    assert "sk_part" in r.stderr or "tile(" in r.stderr, r.stderr[-3000:]
    assert r.returncode == 66


def test_dead_producer_times_out_and_drains(model):
    # flag 25 = slab 6, K-slab 1: rank 2's chunk, a peer of local rank 1
    r = run(model, "--skip-flag", "25", "--timeout-ms", "50", "--calls", "2", timeout=120)
    assert "ThreadSanitizer" not in r.stderr, r.stderr[-3000:]
    assert r.returncode == 0, r.stdout
    assert "error word 1" in r.stdout
