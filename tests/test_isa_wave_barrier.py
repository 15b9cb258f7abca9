"""The scan's partial-wait barrier, checked on the compiled gfx950 code (CPU only).

The wide block loop of `scan_tiles_kernel` ends each block with
`s_waitcnt lgkmcnt(K); s_barrier` instead of a full wait: the wave's last K
LDS instructions, the read-back of its own states from a wave-private area,
may still be in flight.  That is correct only if, on every path into the
barrier, at least K LDS reads come after the wave's last LDS write (LDS
operations of one wave complete in order, so waiting until at most K are
outstanding then covers every write), and no scalar-memory load (which shares
the counter and completes out of order) sits among them.  The compiler
schedules those instructions, so this test compiles the kernel source with the
library's flags and walks the control flow of the assembly back from every
such barrier.  A control run on a copy whose wait count is raised to 12 must
find violations, so the walk is known to see them.
"""
import os
import re
import shutil
import subprocess

import pytest

from selective_state_space_59_amd import build

SRC = os.path.join(build.CSRC, "scan_fwd.hip")


def _read_ops():
    with open(SRC) as f:
        m = re.search(r"#define SSM_PART_READ_OPS (\d+)", f.read())
    assert m, "SSM_PART_READ_OPS not found"
    return int(m.group(1))


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    try:
        hipcc = build.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    out = str(tmp_path_factory.mktemp("isa") / "scan_fwd.s")
    flags = [f for f in build.COMMON if f not in ("-fPIC",)]
    cmd = [hipcc] + flags + ["--cuda-device-only", "-S", SRC, "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    with open(out) as f:
        return f.read().split("\n")


LABEL = re.compile(r"^(\.LBB\d+_\d+):")
BRANCH = re.compile(r"s_(?:c)?branch\w*\s+(\.LBB\d+_\d+)")


def _violations(lines, k):
    """For each `s_waitcnt lgkmcnt(k)` directly followed by `s_barrier`: the paths back
    on which an LDS write, another non-read LDS op or a scalar load comes before k LDS
    reads (an `s_waitcnt lgkmcnt(0)` ends a path as safe)."""
    labels = {m.group(1): i for i, l in enumerate(lines) for m in [LABEL.match(l)] if m}
    preds = {}
    for i, l in enumerate(lines):
        m = BRANCH.search(l.strip())
        if m and m.group(1) in labels:
            preds.setdefault(labels[m.group(1)], []).append(i)

    def walk(i, reads, seen):
        bad = []
        stack = [(i, reads)]
        while stack:
            i, reads = stack.pop()
            while True:
                i -= 1
                if i < 0:
                    bad.append("start of file")
                    break
                line = lines[i]
                t = line.strip()
                if line and not line[0].isspace() and line.endswith(":") and not LABEL.match(line) \
                        and not line.startswith("; %bb"):
                    bad.append("function entry at %d" % i)
                    break
                if LABEL.match(line) or line.startswith("; %bb."):
                    key = (i, min(reads, k))
                    if key in seen:
                        break
                    seen.add(key)
                    for p in preds.get(i, []):
                        stack.append((p + 1, reads))
                    j = i - 1
                    while j >= 0 and (not lines[j].strip() or lines[j].strip().startswith(";")):
                        j -= 1
                    if j >= 0 and not re.match(r"\s*s_(branch|endpgm|setpc)", lines[j]):
                        stack.append((i, reads))
                    break
                if t.startswith("s_waitcnt") and "lgkmcnt(0)" in t:
                    break
                if t.startswith("ds_read"):
                    reads += 1
                    if reads >= k:
                        break
                    continue
                if t.startswith("ds_") or t.startswith("s_load") or t.startswith("s_buffer_load"):
                    bad.append("line %d: %s after %d reads" % (i, t[:50], reads))
                    break
        return bad

    found, bad = 0, []
    for i, l in enumerate(lines[:-1]):
        if l.strip() == "s_waitcnt lgkmcnt(%d)" % k and lines[i + 1].strip() == "s_barrier":
            found += 1
            v = walk(i, 0, set())
            if v:
                bad.append((i, v[:2]))
    return found, bad


def test_partial_wait_barriers_follow_enough_reads(asm):
    k = _read_ops()
    found, bad = _violations(asm, k)
    print("barriers with lgkmcnt(%d): %d" % (k, found))
    assert found > 0, "no partial-wait barrier in the compiled code"
    assert not bad, bad[:3]


def test_walk_detects_a_violation(asm):
    k = _read_ops()
    big = 2 * k  # more reads than the read-back provides
    text = [l.replace("s_waitcnt lgkmcnt(%d)" % k, "s_waitcnt lgkmcnt(%d)" % big) for l in asm]
    found, bad = _violations(text, big)
    assert found > 0 and bad
