"""The prefill kernels' schedule arithmetic (csrc/prefill_plan.h), checked on
the host with no GPU: the K loop's copy-wait counts against a simulation of
the order the loop issues its copies in, and the gate/up write-out roles
against full coverage of the h record at every d_ff the prefill path takes.
The header is compiled by tests/host/prefill_plan_check.cpp against the
stand-in HIP runtime under tests/host."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLANG = "/opt/rocm/llvm/bin/clang++"
K_XD, K_XCOPIES, K_WCOPIES = 3, 2, 8  # the plan's constants, restated from its description


@pytest.fixture(scope="module")
def prog(tmp_path_factory):
    if not os.path.exists(CLANG):
        pytest.skip("no host clang++")
    out = str(tmp_path_factory.mktemp("plan") / "prefill_plan_check")
    cmd = [CLANG, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-I", os.path.join(ROOT, "tests", "host"), "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "quantized_expert_ffn_softmax_amd", "csrc"),
           os.path.join(ROOT, "tests", "host", "prefill_plan_check.cpp"), "-o", out]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    return out


def _issue_order(nsb):
    """The copies in the order the K loop issues them, and what each step
    needs landed: prologue -- tiles 0 .. kXD-1, then superblock 0's weights;
    step s, after its wait and barrier -- tile s + kXD, then at a superblock's
    first step the next superblock's weights.  Step s reads tile s; step 0
    reads superblock 0's weights; step 5 S + 4 reads superblock S + 1's
    (it dequantises the next superblock's first fragments)."""
    issued = []
    for s0 in range(K_XD):
        issued += [("x", s0)] * K_XCOPIES
    issued += [("w", 0)] * K_WCOPIES
    tile_after, need_after = {}, {}
    for s in range(5 * nsb):
        last_tile = max(i for i, it in enumerate(issued) if it == ("x", s))
        needs = [last_tile]
        if s == 0:
            needs.append(max(i for i, it in enumerate(issued) if it == ("w", 0)))
        if s % 5 == 4:
            needs.append(max(i for i, it in enumerate(issued) if it == ("w", s // 5 + 1)))
        tile_after[s] = len(issued) - 1 - last_tile
        need_after[s] = len(issued) - 1 - max(needs)
        issued += [("x", s + K_XD)] * K_XCOPIES
        if s % 5 == 0:
            issued += [("w", s // 5 + 1)] * K_WCOPIES
    return tile_after, need_after


def test_copy_waits_match_the_issue_order(prog):
    out = subprocess.run([prog, "table"], check=True, capture_output=True, text=True).stdout.split("\n")
    table = {(int(a), int(b)): int(c) for a, b, c in (line.split() for line in out if line.strip())}
    tile_after, need_after = _issue_order(nsb=4)
    for s in range(20):
        first, t = s < 5, s % 5
        got = table[(1 if first else 0, t)]
        # exactly what the step reads has landed, no more: its own tile (and
        # at step 0 superblock 0's weights, the prologue's last copies); the
        # next superblock's weights, read at step 4, were issued before the
        # tile of that step
        assert got == need_after[s], (s, got, need_after[s])
        assert got == (0 if s == 0 else tile_after[s]), (s, got, tile_after[s])


def test_copy_waits_stay_in_the_counter_field(prog):
    out = subprocess.run([prog, "table"], check=True, capture_output=True, text=True).stdout
    assert all(0 <= int(line.split()[2]) < 64 for line in out.strip().split("\n"))


def test_write_out_roles_store_each_h_half_once(prog):
    r = subprocess.run([prog, "cover"], capture_output=True, text=True)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr
