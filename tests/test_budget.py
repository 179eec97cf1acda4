"""Host-side pin of the prefill kernel's candidate-buffer accounting.

The kernel's streaming top-k lets all 64 lanes of a hand-off store (the
non-passing ones past the new count), so a unit needs 128 free slots in
front of it; compaction happens only at tile barriers.  tests/budget_emu.cpp
walks every buffer count reachable at a compaction point under any sequence
of hand-offs (0..64 passing keys, two per tile), flags and trims, using the
same rules the kernel compiles (sparse_attention_token_lid_amd/csrc/
lid_budget.h), and fails on any write past the capacity.  Planted mistakes in
a copy of the rules (the flag or the trim trigger one unit late, a capacity
without the trim slack) must each be caught.  (The room check before the
last unit never fires in the reachable states: the flags already keep every
buffer a tile's worth below its capacity at each barrier.)
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_attention_token_lid_amd", "csrc")
EMU = os.path.join(ROOT, "tests", "budget_emu.cpp")
K_TOPS = ["1", "2", "7", "63", "64", "65", "100", "255", "256", "257", "300", "511", "512", "513", "1000", "1024"]


def _build_and_run(include_dir, tmp_path, name):
    exe = os.path.join(tmp_path, name)
    subprocess.run(["g++", "-O2", "-std=c++17", "-I", include_dir, EMU, "-o", exe], check=True,
                   capture_output=True, text=True)
    return subprocess.run([exe, *K_TOPS], capture_output=True, text=True)


@pytest.fixture(scope="module")
def tmp_dir(tmp_path_factory):
    if shutil.which("g++") is None:
        pytest.skip("g++ not available")
    return str(tmp_path_factory.mktemp("budget"))


def test_budget_rules_never_overflow(tmp_dir):
    r = _build_and_run(CSRC, tmp_dir, "emu")
    assert r.returncode == 0, r.stdout + r.stderr
    lines = r.stdout.strip().splitlines()
    assert len(lines) == len(K_TOPS) and all(l.startswith("ok ") for l in lines)


MUTATIONS = {
    # the flag raised one unit too late: a tile's second unit can overflow
    "flag one unit late": ("return count > cap - (kUnitsPerTile + 1) * kUnitKeys;",
                           "return count > cap - kUnitsPerTile * kUnitKeys;"),
    # the trim trigger one unit looser: a flagged buffer keeps too many keys
    "trim one unit late": ("return count > K + kTrimSlack;", "return count > K + kTrimSlack + kUnitKeys;"),
    # capacity without the trim slack (2 K + 184 alone): small k_top overflow
    "capacity without slack": ("constexpr int prefill_cap(int K) {\n  return",
                               "constexpr int prefill_cap(int K) {\n  return 2 * K + 184;\n  return"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(tmp_dir, name):
    old, new = MUTATIONS[name]
    src = open(os.path.join(CSRC, "lid_budget.h")).read()
    assert old in src, name
    d = os.path.join(tmp_dir, name.replace(" ", "_"))
    os.makedirs(d, exist_ok=True)
    open(os.path.join(d, "lid_budget.h"), "w").write(src.replace(old, new))
    r = _build_and_run(d, d, "emu")
    assert r.returncode == 1 and "violation" in r.stdout, (name, r.stdout)
