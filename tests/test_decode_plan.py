"""The split decode's work decomposition, checked on the host.

`plan_decode` (transformer_attention_flash_amd/csrc/decode_plan.h) is pure host
arithmetic: from the sequence lengths it cuts every (sequence, KV head, head
block) unit's keys into key blocks and lists them as segments for the split
kernel.  tests/decode_plan_check.cpp, built here with g++ (and once more with
AddressSanitizer and UndefinedBehaviorSanitizer), runs it on seeded random
calls -- 1 to 32 sequences, GQA group sizes 1 to 32, caches of 1 to 2^30 rows,
full, ragged, empty and one-key sequences, devices of 8 to 304 CUs -- and
checks that the blocks tile each sequence exactly in split-slot order, within
the workspace's split bound, with the segment table and grid size consistent.
A run that alters one planned segment per call must be rejected every time.
"""
import shutil
import subprocess

import pytest

from pathlib import Path

ROOT = Path(__file__).resolve().parents[1]
SRC = ROOT / "tests" / "decode_plan_check.cpp"


def build(tmp_path, sanitize):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not found")
    exe = tmp_path / ("dpc_san" if sanitize else "dpc")
    flags = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined"] if sanitize else ["-O2"]
    subprocess.run([gxx, "-std=c++17", "-Wall", "-Wextra", "-Werror", *flags, "-o", str(exe), str(SRC)], check=True,
                   capture_output=True, text=True)
    return exe


def run(exe, *args):
    return subprocess.run([str(exe), *map(str, args)], capture_output=True, text=True, timeout=300)


def test_plans_tile_every_sequence(tmp_path):
    exe = build(tmp_path, sanitize=False)
    for seed in (1, 2, 3):
        r = run(exe, seed, 20000)
        assert r.returncode == 0, r.stderr
        assert r.stdout.startswith("ok 20000 calls"), r.stdout


def test_plans_under_sanitizers(tmp_path):
    try:
        exe = build(tmp_path, sanitize=True)
    except subprocess.CalledProcessError as e:
        pytest.skip(f"host sanitizers unavailable: {e.stderr[-200:]}")
    r = run(exe, 7, 5000)
    assert r.returncode == 0, r.stderr
    assert r.stdout.startswith("ok 5000 calls"), r.stdout


def test_altered_plans_are_rejected(tmp_path):
    exe = build(tmp_path, sanitize=False)
    r = run(exe, 11, 3000, "corrupt")
    assert r.returncode == 0, r.stdout + r.stderr
    assert "altered plans rejected" in r.stdout
