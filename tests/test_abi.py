"""Host-side tests of the C ABI (no GPU needed).

Argument checking in libssm_hip.so finishes before any HIP call, so every
error path can be driven from the CPU with placeholder device addresses that
are never dereferenced.  Also checks that the library exports every function
include/ssm.h declares and that the ctypes mirrors match the C layouts.

The whole module runs only where no GPU is visible: should an argument check
ever regress, a call would launch a kernel on the placeholder addresses, which
must never reach a real device.
"""
import ctypes
import os
import re
import subprocess
import tempfile

import pytest
import torch

from selective_state_space_59_amd import ssm

pytestmark = pytest.mark.skipif(torch.cuda.is_available(),
                                reason="placeholder device addresses must not reach a real GPU")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssm.h")

# Placeholder device addresses (256-aligned, far apart, never dereferenced).
BASE = 0x7F0000000000
STEP = 1 << 32


def addr(i, off=0):
    return BASE + i * STEP + off


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(ssm_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert set(names) == set(ssm.EXPORTED_SYMBOLS)
    L = ssm.lib()
    for n in names:
        assert hasattr(L, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", ssm.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    for n in names:
        assert re.search(r"\bT %s\b" % n, out), n


def test_abi_version_and_status_strings():
    ver = int(re.search(r"#define SSM_ABI_VERSION (\d+)", open(HEADER).read()).group(1))
    assert ssm.abi_version() == ver
    for code in range(0, 9):
        s = ssm.status_string(code)
        assert s.startswith("SSM_")
    assert "unknown" in ssm.status_string(99)


C_LAYOUT = r"""
#include <stdio.h>
#include <stddef.h>
#include "ssm.h"
#define F(T, f) printf(#T " " #f " %zu\n", offsetof(T, f));
int main(void) {
  printf("ssm_scan_args_t size %zu\n", sizeof(ssm_scan_args_t));
  printf("ssm_state_update_args_t size %zu\n", sizeof(ssm_state_update_args_t));
  printf("ssm_scan_bwd_args_t size %zu\n", sizeof(ssm_scan_bwd_args_t));
  printf("ssm_block_dims_t size %zu\n", sizeof(ssm_block_dims_t));
  printf("ssm_block_weights_t size %zu\n", sizeof(ssm_block_weights_t));
  printf("ssm_ssd_args_t size %zu\n", sizeof(ssm_ssd_args_t));
  printf("ssm_ssd_step_args_t size %zu\n", sizeof(ssm_ssd_step_args_t));
  %FIELDS%
  return 0;
}
"""


STRUCTS = (("ssm_scan_args_t", ssm.ScanArgs), ("ssm_state_update_args_t", ssm.StateUpdateArgs),
           ("ssm_scan_bwd_args_t", ssm.ScanBwdArgs), ("ssm_block_dims_t", ssm.BlockDims),
           ("ssm_block_weights_t", ssm.BlockWeights), ("ssm_ssd_args_t", ssm.SsdArgs),
           ("ssm_ssd_step_args_t", ssm.SsdStepArgs))


def test_ctypes_structs_match_c_layout():
    lines = []
    for cname, cls in STRUCTS:
        for f, _ in cls._fields_:
            lines.append("F(%s, %s)" % (cname, f))
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "layout.c")
        open(c, "w").write(C_LAYOUT.replace("%FIELDS%", "\n  ".join(lines)))
        exe = os.path.join(d, "layout")
        subprocess.run(["gcc", "-std=c11", "-I", os.path.join(ROOT, "include"), c, "-o", exe],
                       check=True)
        out = subprocess.run([exe], capture_output=True, text=True, check=True).stdout.split("\n")
    got = {}
    for line in out:
        if line:
            t, f, v = line.split()
            got[(t, f)] = int(v)
    for cname, cls in STRUCTS:
        assert got[(cname, "size")] == ctypes.sizeof(cls), cname
        for f, _ in cls._fields_:
            assert got[(cname, f)] == getattr(cls, f).offset, (cname, f)


# ----------------------------------------------------------------- scan checks
def scan_args(**kw):
    a = ssm.ScanArgs(batch=2, seqlen=8, dim=64, dstate=16, io_dtype=ssm.SSM_BF16,
                     delta_softplus=0, conv_k=0, x=addr(0), delta=addr(1), Bm=addr(2),
                     Cm=addr(3), z=addr(4), A=addr(5), Dskip=addr(6), delta_bias=None,
                     conv_w=None, conv_b=None, h0=None, y=addr(7), h_final=addr(8),
                     workspace=addr(9), workspace_bytes=1 << 30)
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def run_scan(a):
    return ssm.lib().ssm_selective_scan_fwd(ctypes.byref(a), None)


@pytest.mark.parametrize("field,value,status", [
    ("io_dtype", 7, ssm.SSM_ERR_BAD_DTYPE),
    ("batch", -1, ssm.SSM_ERR_BAD_SHAPE),
    ("seqlen", -5, ssm.SSM_ERR_BAD_SHAPE),
    ("dim", 0, ssm.SSM_ERR_BAD_SHAPE),
    ("dstate", 0, ssm.SSM_ERR_BAD_SHAPE),
    ("dstate", 17, ssm.SSM_ERR_UNSUPPORTED),
    ("conv_k", -1, ssm.SSM_ERR_BAD_SHAPE),
    ("conv_k", 5, ssm.SSM_ERR_UNSUPPORTED),
    ("conv_k", 4, ssm.SSM_ERR_NULL_ARG),          # conv_k without conv_w
    ("delta_softplus", 2, ssm.SSM_ERR_UNSUPPORTED),
    ("x", None, ssm.SSM_ERR_NULL_ARG),
    ("delta", None, ssm.SSM_ERR_NULL_ARG),
    ("Bm", None, ssm.SSM_ERR_NULL_ARG),
    ("Cm", None, ssm.SSM_ERR_NULL_ARG),
    ("A", None, ssm.SSM_ERR_NULL_ARG),
    ("y", None, ssm.SSM_ERR_NULL_ARG),
    ("x", addr(0, 1), ssm.SSM_ERR_ALIGN),        # odd address for bf16
    ("A", addr(5, 2), ssm.SSM_ERR_ALIGN),        # fp32 not 4-aligned
    ("y", addr(0, 64), ssm.SSM_ERR_ALIAS),       # y inside x
    ("h_final", addr(7, 16), ssm.SSM_ERR_ALIAS), # h_final inside y
    ("h0", addr(8), ssm.SSM_ERR_ALIAS),          # h0 == h_final
    ("conv_b", addr(10), ssm.SSM_ERR_BAD_SHAPE), # conv bias without conv
    ("batch", 1 << 56, ssm.SSM_ERR_BAD_SHAPE),   # overflow of B*L*D
])
def test_scan_rejects_bad_arguments(field, value, status):
    a = scan_args(**{field: value})
    assert run_scan(a) == status
    assert ssm.lib().ssm_last_error_message().decode() != ""


# The no-allocation scan: the same argument checks, no caller workspace, and a
# size limit checked before any HIP call.
def run_scan_noalloc(a):
    return ssm.lib().ssm_selective_scan_fwd_noalloc(ctypes.byref(a), None)


def test_noalloc_scan_rejects_a_workspace():
    assert run_scan_noalloc(scan_args()) == ssm.SSM_ERR_WORKSPACE
    assert "no workspace" in ssm.lib().ssm_last_error_message().decode()
    assert run_scan_noalloc(scan_args(workspace=None, workspace_bytes=64)) == ssm.SSM_ERR_WORKSPACE


def test_noalloc_scan_rejects_sizes_beyond_its_scratch():
    # 300000 rows of 8192 bf16 channels span more than one launch, so the carry
    # between launches needs B * D * N * 4 = 64 MiB of workspace: beyond the array.
    far = {k: addr(200 * i) for i, k in enumerate(("x", "delta", "Bm", "Cm", "z", "A", "Dskip",
                                                    "y", "h_final"))}
    a = scan_args(batch=128, seqlen=300000, dim=8192, workspace=None, workspace_bytes=0, **far)
    need = ssm.lib().ssm_selective_scan_workspace_size(ctypes.byref(a))
    assert need > ssm.NOALLOC_SCRATCH_BYTES
    assert run_scan_noalloc(a) == ssm.SSM_ERR_WORKSPACE
    msg = ssm.lib().ssm_last_error_message().decode()
    assert str(need) in msg and str(ssm.NOALLOC_SCRATCH_BYTES) in msg


@pytest.mark.parametrize("field,value,status", [
    ("io_dtype", 7, ssm.SSM_ERR_BAD_DTYPE),
    ("dstate", 17, ssm.SSM_ERR_UNSUPPORTED),
    ("x", None, ssm.SSM_ERR_NULL_ARG),
    ("y", addr(0, 64), ssm.SSM_ERR_ALIAS),
    ("x", addr(0, 1), ssm.SSM_ERR_ALIGN),
])
def test_noalloc_scan_checks_arguments_like_the_scan(field, value, status):
    a = scan_args(workspace=None, workspace_bytes=0, **{field: value})
    assert run_scan_noalloc(a) == status
    assert run_scan(scan_args(**{field: value})) == status


def test_noalloc_scan_scratch_size_matches_the_header():
    v = re.search(r"#define SSM_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", open(HEADER).read())
    assert int(v.group(1)) << int(v.group(2)) == ssm.NOALLOC_SCRATCH_BYTES


def test_noalloc_scan_without_a_device_reports_hip():
    # Valid arguments whose plan needs a workspace (a long single row is cut into
    # segments): the call gets as far as the scratch lookup, which fails here.
    a = scan_args(batch=1, seqlen=20000, dim=64, workspace=None, workspace_bytes=0)
    assert ssm.lib().ssm_selective_scan_workspace_size(ctypes.byref(a)) > 0
    assert run_scan_noalloc(a) == ssm.SSM_ERR_HIP


# Conv state (the prefill -> decode handoff): given only with the prologue,
# aligned, and overlapping nothing except its own input when updated in place.
@pytest.mark.parametrize("kw,status", [
    (dict(conv_state_in=addr(11)), ssm.SSM_ERR_BAD_SHAPE),
    (dict(conv_state_out=addr(11)), ssm.SSM_ERR_BAD_SHAPE),
    (dict(conv_k=4, conv_w=addr(10), conv_state_out=addr(0, 64)), ssm.SSM_ERR_ALIAS),
    (dict(conv_k=4, conv_w=addr(10), conv_state_out=addr(7, 64)), ssm.SSM_ERR_ALIAS),
    (dict(conv_k=4, conv_w=addr(10), conv_state_in=addr(11), conv_state_out=addr(11, 64)),
     ssm.SSM_ERR_ALIAS),
    (dict(conv_k=4, conv_w=addr(10), conv_state_in=addr(7, 32)), ssm.SSM_ERR_ALIAS),
    (dict(conv_k=4, conv_w=addr(10), conv_state_in=addr(11, 1)), ssm.SSM_ERR_ALIGN),
])
def test_scan_conv_state_checks(kw, status):
    assert run_scan(scan_args(**kw)) == status


def test_scan_conv_state_in_place_passes_the_checks():
    # Same tensor in and out is allowed: the checks pass and only the launch
    # (no device here) fails.
    a = scan_args(conv_k=4, conv_w=addr(10), conv_state_in=addr(11), conv_state_out=addr(11))
    assert run_scan(a) == ssm.SSM_ERR_HIP


def test_scan_null_args_pointer():
    assert ssm.lib().ssm_selective_scan_fwd(None, None) == ssm.SSM_ERR_NULL_ARG


def test_scan_empty_batch_is_a_noop():
    # B == 0 returns before any HIP call, so it succeeds even without a GPU.
    a = scan_args(batch=0)
    assert run_scan(a) == ssm.SSM_OK
    assert ssm.lib().ssm_last_error_message().decode() == ""


def test_scan_empty_sequence_without_final_state_is_a_noop():
    a = scan_args(seqlen=0, h_final=None)
    assert run_scan(a) == ssm.SSM_OK


def test_workspace_size_queries():
    L = ssm.lib()
    assert L.ssm_selective_scan_workspace_size(ctypes.byref(scan_args(dstate=99))) == \
        ctypes.c_size_t(-1).value
    assert L.ssm_selective_scan_workspace_size(ctypes.byref(scan_args(batch=0))) == 0
    assert L.ssm_selective_scan_workspace_size(None) == ctypes.c_size_t(-1).value
    # Valid sizes give a finite answer that only depends on sizes and flags.
    n1 = L.ssm_selective_scan_workspace_size(ctypes.byref(scan_args()))
    n2 = L.ssm_selective_scan_workspace_size(ctypes.byref(scan_args(x=addr(11))))
    assert n1 == n2 and n1 < (1 << 40)


def test_scan_workspace_checks():
    L = ssm.lib()
    a = scan_args(batch=1, seqlen=1 << 20, dim=1024)
    need = L.ssm_selective_scan_workspace_size(ctypes.byref(a))
    if need == 0:
        pytest.skip("this launch plan needs no workspace")
    a.workspace = None
    assert run_scan(a) == ssm.SSM_ERR_WORKSPACE
    a.workspace = addr(9)
    a.workspace_bytes = need - 1
    assert run_scan(a) == ssm.SSM_ERR_WORKSPACE
    a.workspace_bytes = need
    a.workspace = addr(9, 8)
    assert run_scan(a) == ssm.SSM_ERR_WORKSPACE


# Checkpoints (the forward -> backward handoff): fp32, aligned, overlapping
# nothing; with them the backward's workspace is smaller (it skips its own).
@pytest.mark.parametrize("kw,status", [
    (dict(checkpoints=addr(12, 2)), ssm.SSM_ERR_ALIGN),
    (dict(checkpoints=addr(0, 64)), ssm.SSM_ERR_ALIAS),      # inside x
    (dict(checkpoints=addr(7, 64)), ssm.SSM_ERR_ALIAS),      # inside y
    (dict(checkpoints=addr(8)), ssm.SSM_ERR_ALIAS),          # == h_final
    # inside the workspace (a long row is cut into segments, which need one)
    (dict(checkpoints=addr(9, 256), batch=1, seqlen=20000), ssm.SSM_ERR_ALIAS),
    (dict(checkpoints=addr(12), seqlen=1 << 60), ssm.SSM_ERR_BAD_SHAPE),
    # B L D and B D N fit, the 16-wide checkpoints of 2^59 channels do not
    (dict(checkpoints=addr(12), batch=1, seqlen=1, dim=1 << 59, dstate=1), ssm.SSM_ERR_BAD_SHAPE),
])
def test_scan_checkpoint_checks(kw, status):
    assert run_scan(scan_args(**kw)) == status


def test_scan_checkpoints_pass_the_checks():
    assert run_scan(scan_args(checkpoints=addr(12))) == ssm.SSM_ERR_HIP
    assert ssm.checkpoint_shape(2, 33, 64) == (3, 2, 64, 16)


# ----------------------------------------------------------------- conv checks
def run_conv(B=2, L=8, D=64, K=4, dt=ssm.SSM_BF16, x=addr(0), w=addr(1), b=addr(2), u=addr(3)):
    return ssm.lib().ssm_causal_conv1d_silu(B, L, D, K, dt, x, w, b, u, None)


@pytest.mark.parametrize("kw,status", [
    (dict(dt=5), ssm.SSM_ERR_BAD_DTYPE),
    (dict(B=-1), ssm.SSM_ERR_BAD_SHAPE),
    (dict(D=0), ssm.SSM_ERR_BAD_SHAPE),
    (dict(K=0), ssm.SSM_ERR_BAD_SHAPE),
    (dict(K=5), ssm.SSM_ERR_UNSUPPORTED),
    (dict(x=None), ssm.SSM_ERR_NULL_ARG),
    (dict(w=None), ssm.SSM_ERR_NULL_ARG),
    (dict(u=None), ssm.SSM_ERR_NULL_ARG),
    (dict(u=addr(0, 2)), ssm.SSM_ERR_ALIAS),
    (dict(x=addr(0, 1)), ssm.SSM_ERR_ALIGN),
])
def test_conv_rejects_bad_arguments(kw, status):
    assert run_conv(**kw) == status


def test_conv_empty_is_a_noop():
    assert run_conv(B=0) == ssm.SSM_OK
    assert run_conv(L=0, x=None, u=None) == ssm.SSM_OK


# --------------------------------------------------------- state-update checks
def upd_args(**kw):
    a = ssm.StateUpdateArgs(batch=4, dim=64, dstate=16, io_dtype=ssm.SSM_BF16, delta_softplus=0,
                            state=addr(0), x=addr(1), delta=addr(2), z=addr(3), Bm=addr(4),
                            Cm=addr(5), A=addr(6), Dskip=addr(7), delta_bias=None, y=addr(8))
    for k, v in kw.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("field,value,status", [
    ("io_dtype", -1, ssm.SSM_ERR_BAD_DTYPE),
    ("batch", -2, ssm.SSM_ERR_BAD_SHAPE),
    ("dim", 0, ssm.SSM_ERR_BAD_SHAPE),
    ("dstate", 0, ssm.SSM_ERR_BAD_SHAPE),
    ("dstate", 32, ssm.SSM_ERR_UNSUPPORTED),
    ("delta_softplus", 3, ssm.SSM_ERR_UNSUPPORTED),
    ("state", None, ssm.SSM_ERR_NULL_ARG),
    ("x", None, ssm.SSM_ERR_NULL_ARG),
    ("Bm", None, ssm.SSM_ERR_NULL_ARG),
    ("y", None, ssm.SSM_ERR_NULL_ARG),
    ("y", addr(1), ssm.SSM_ERR_ALIAS),
    ("y", addr(0, 128), ssm.SSM_ERR_ALIAS),
    ("x", addr(0, 64), ssm.SSM_ERR_ALIAS),       # input inside the state
    ("state", addr(0, 2), ssm.SSM_ERR_ALIGN),
])
def test_state_update_rejects_bad_arguments(field, value, status):
    a = upd_args(**{field: value})
    assert ssm.lib().ssm_state_update(ctypes.byref(a), None) == status


@pytest.mark.parametrize("kw,status", [
    (dict(conv_k=-1), ssm.SSM_ERR_BAD_SHAPE),
    (dict(conv_k=5, conv_w=addr(9)), ssm.SSM_ERR_UNSUPPORTED),
    (dict(conv_k=4), ssm.SSM_ERR_NULL_ARG),                                   # no conv_w
    (dict(conv_k=4, conv_w=addr(9)), ssm.SSM_ERR_NULL_ARG),                   # no window
    (dict(conv_state=addr(10)), ssm.SSM_ERR_BAD_SHAPE),                       # window, no conv
    (dict(conv_b=addr(10)), ssm.SSM_ERR_BAD_SHAPE),
    (dict(conv_k=4, conv_w=addr(9), conv_state=addr(0, 256)), ssm.SSM_ERR_ALIAS),  # in the state
    (dict(conv_k=4, conv_w=addr(9), conv_state=addr(8)), ssm.SSM_ERR_ALIAS),       # == y
    (dict(conv_k=4, conv_w=addr(9), conv_state=addr(9, 8)), ssm.SSM_ERR_ALIAS),    # in conv_w
    (dict(conv_k=4, conv_w=addr(9), conv_state=addr(10, 1)), ssm.SSM_ERR_ALIGN),
    (dict(conv_k=4, conv_w=addr(9, 2), conv_state=addr(10)), ssm.SSM_ERR_ALIGN),
])
def test_state_update_conv_checks(kw, status):
    a = upd_args(**kw)
    assert ssm.lib().ssm_state_update(ctypes.byref(a), None) == status


def test_state_update_width_one_conv_needs_no_window():
    a = upd_args(conv_k=1, conv_w=addr(9))
    assert ssm.lib().ssm_state_update(ctypes.byref(a), None) == ssm.SSM_ERR_HIP


def test_state_update_empty_batch_is_a_noop():
    a = upd_args(batch=0)
    assert ssm.lib().ssm_state_update(ctypes.byref(a), None) == ssm.SSM_OK


def test_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros(1, 4, 8)
    with pytest.raises(ValueError):
        ssm.selective_scan_fwd(x, x, torch.zeros(8, 4), torch.zeros(1, 4, 4), torch.zeros(1, 4, 4))


# ------------------------------------------------------------- backward checks
def bwd_args(**kw):
    a = ssm.ScanBwdArgs(batch=2, seqlen=8, dim=64, dstate=16, io_dtype=ssm.SSM_BF16,
                        delta_softplus=0, conv_k=0, x=addr(0), delta=addr(1), Bm=addr(2),
                        Cm=addr(3), z=addr(4), A=addr(5), Dskip=addr(6), dy=addr(7),
                        dx=addr(8), ddelta=addr(9), dz=addr(10), dA=addr(11), dBm=addr(12),
                        dCm=addr(13), dDskip=addr(14), workspace=addr(15), workspace_bytes=1 << 34)
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def run_bwd(a):
    return ssm.lib().ssm_selective_scan_bwd(ctypes.byref(a), None)


def _conv_bwd(**kw):
    base = dict(conv_k=4, conv_w=addr(16), dconv_w=addr(18))
    base.update(kw)
    return bwd_args(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(conv_state_in=addr(19), dconv_state_in=addr(0, 64)), ssm.SSM_ERR_ALIAS),  # grad inside x
    (dict(conv_state_in=addr(8, 2)), ssm.SSM_ERR_ALIAS),            # state inside dx
    (dict(conv_state_in=addr(19), dconv_state_in=addr(19)), ssm.SSM_ERR_ALIAS),
    (dict(conv_state_in=addr(19, 1)), ssm.SSM_ERR_ALIGN),
    (dict(conv_k=1, conv_state_in=addr(19)), ssm.SSM_ERR_BAD_SHAPE),
])
def test_bwd_conv_state_checks(kw, status):
    assert run_bwd(_conv_bwd(**kw)) == status


@pytest.mark.parametrize("N", [1, 5, 15])
def test_bwd_small_dstate_passes_the_checks_and_needs_more_workspace(N):
    """N < 16 is accepted; its workspace holds the 16-wide copies on top of the
    N = 16 workspace (the launch itself fails here: no device)."""
    a16 = bwd_args(workspace=None, workspace_bytes=0)
    aN = bwd_args(dstate=N, workspace=None, workspace_bytes=0)
    n16 = ssm.lib().ssm_selective_scan_bwd_workspace_size(ctypes.byref(a16))
    nN = ssm.lib().ssm_selective_scan_bwd_workspace_size(ctypes.byref(aN))
    assert nN > n16
    assert run_bwd(bwd_args(dstate=N)) == ssm.SSM_ERR_HIP


@pytest.mark.parametrize("field,value,status", [
    ("io_dtype", 3, ssm.SSM_ERR_BAD_DTYPE),
    ("batch", -1, ssm.SSM_ERR_BAD_SHAPE),
    ("dstate", 17, ssm.SSM_ERR_UNSUPPORTED),      # N <= 16
    ("dstate", 0, ssm.SSM_ERR_BAD_SHAPE),
    ("conv_state_in", addr(17), ssm.SSM_ERR_BAD_SHAPE),   # a conv state without conv_k > 1
    ("dconv_state_in", addr(17), ssm.SSM_ERR_BAD_SHAPE),
    ("conv_k", 4, ssm.SSM_ERR_NULL_ARG),          # conv_k without conv_w
    ("conv_k", 5, ssm.SSM_ERR_UNSUPPORTED),
    ("conv_w", addr(16), ssm.SSM_ERR_BAD_SHAPE),  # conv weights without conv_k
    ("dy", None, ssm.SSM_ERR_NULL_ARG),
    ("dx", None, ssm.SSM_ERR_NULL_ARG),
    ("dBm", None, ssm.SSM_ERR_NULL_ARG),
    ("dA", None, ssm.SSM_ERR_NULL_ARG),
    ("dz", None, ssm.SSM_ERR_NULL_ARG),           # z given
    ("dx", addr(0, 64), ssm.SSM_ERR_ALIAS),       # inside x
    ("dBm", addr(13), ssm.SSM_ERR_ALIAS),         # == dCm
    ("dA", addr(15), ssm.SSM_ERR_ALIAS),          # inside the workspace
    ("dx", addr(8, 1), ssm.SSM_ERR_ALIGN),
    ("workspace", None, ssm.SSM_ERR_WORKSPACE),
])
def test_bwd_rejects_bad_arguments(field, value, status):
    assert run_bwd(bwd_args(**{field: value})) == status


@pytest.mark.parametrize("kw,status", [
    (dict(checkpoints=addr(20, 2)), ssm.SSM_ERR_ALIGN),
    (dict(checkpoints=addr(8, 64)), ssm.SSM_ERR_ALIAS),      # inside dx
    (dict(checkpoints=addr(15, 256)), ssm.SSM_ERR_ALIAS),    # inside the workspace
])
def test_bwd_checkpoint_checks(kw, status):
    assert run_bwd(bwd_args(**kw)) == status


@pytest.mark.parametrize("N", [16, 5])
def test_bwd_with_checkpoints_needs_less_workspace(N):
    L = ssm.lib()
    plain = bwd_args(dstate=N, workspace=None, workspace_bytes=0)
    given = bwd_args(dstate=N, workspace=None, workspace_bytes=0, checkpoints=addr(20))
    n0 = L.ssm_selective_scan_bwd_workspace_size(ctypes.byref(plain))
    n1 = L.ssm_selective_scan_bwd_workspace_size(ctypes.byref(given))
    assert n1 < n0
    # the checkpoints of B=2, L=8, D=64: one block of 2 * 64 * 16 fp32 (256-rounded)
    assert n0 - n1 >= 2 * 64 * 16 * 4
    assert run_bwd(bwd_args(dstate=N, checkpoints=addr(20))) == ssm.SSM_ERR_HIP


def test_bwd_checkpoint_sizes_overflow():
    # B L D and B D N fit, but the 16-wide checkpoints of 2^59 channels do not
    a = bwd_args(seqlen=1, dim=1 << 59, dstate=1)
    assert run_bwd(a) == ssm.SSM_ERR_BAD_SHAPE
    assert ssm.lib().ssm_selective_scan_bwd_workspace_size(ctypes.byref(a)) == ctypes.c_size_t(-1).value


def test_bwd_dz_without_z_and_empty_batch():
    assert run_bwd(bwd_args(z=None)) == ssm.SSM_ERR_BAD_SHAPE
    assert run_bwd(bwd_args(batch=0)) == ssm.SSM_OK
    L = ssm.lib()
    assert L.ssm_selective_scan_bwd_workspace_size(ctypes.byref(bwd_args(dstate=17))) == \
        ctypes.c_size_t(-1).value
    assert 0 < L.ssm_selective_scan_bwd_workspace_size(ctypes.byref(bwd_args())) < (1 << 40)


# --------------------------------------------------------------- block checks
def block_dims(**kw):
    d = ssm.BlockDims(batch=2, seqlen=8, d_model=64, d_inner=128, dstate=16, dt_rank=4, conv_k=4)
    for k, v in kw.items():
        setattr(d, k, v)
    return d


@pytest.mark.parametrize("field,value,status", [
    ("batch", 0, ssm.SSM_ERR_BAD_SHAPE),
    ("seqlen", -1, ssm.SSM_ERR_BAD_SHAPE),
    ("d_model", 0, ssm.SSM_ERR_BAD_SHAPE),
    ("dt_rank", 0, ssm.SSM_ERR_BAD_SHAPE),
    ("dt_rank", 129, ssm.SSM_ERR_BAD_SHAPE),      # above d_inner
    ("dstate", 17, ssm.SSM_ERR_UNSUPPORTED),
    ("conv_k", 0, ssm.SSM_ERR_UNSUPPORTED),
    ("conv_k", 5, ssm.SSM_ERR_UNSUPPORTED),
    ("d_model", 60, ssm.SSM_ERR_UNSUPPORTED),     # not a multiple of 8
    ("d_inner", 100, ssm.SSM_ERR_UNSUPPORTED),
    ("seqlen", 1 << 29, ssm.SSM_ERR_BAD_SHAPE),   # B*L = 2^30: beyond the launch limits
])
def test_block_plan_rejects_bad_sizes(field, value, status):
    h = ctypes.c_void_p(12345)
    assert ssm.lib().ssm_block_plan_create(ctypes.byref(block_dims(**{field: value})),
                                           ctypes.byref(h)) == status
    assert not h.value


def test_block_null_arguments_and_no_device():
    L = ssm.lib()
    h = ctypes.c_void_p()
    assert L.ssm_block_plan_create(None, ctypes.byref(h)) == ssm.SSM_ERR_NULL_ARG
    assert L.ssm_block_plan_create(ctypes.byref(block_dims()), None) == ssm.SSM_ERR_NULL_ARG
    assert L.ssm_block_workspace_size(None) == 0
    L.ssm_block_plan_destroy(None)
    w = ssm.BlockWeights()
    assert L.ssm_block_fwd(None, ctypes.byref(w), addr(0), addr(1), addr(2), 1 << 30, None) == \
        ssm.SSM_ERR_NULL_ARG
    # Valid sizes: a plan where a device is present, a clean error (not an exit) where none is.
    st = L.ssm_block_plan_create(ctypes.byref(block_dims()), ctypes.byref(h))
    assert st in (ssm.SSM_OK, ssm.SSM_ERR_HIP)
    if st == ssm.SSM_OK:
        assert L.ssm_block_workspace_size(h) > 0
        L.ssm_block_plan_destroy(h)
    else:
        assert not h.value


# ----------------------------------------------------------------- SSD checks
def ssd_args(**kw):
    a = ssm.SsdArgs(batch=2, seqlen=64, nheads=4, headdim=64, ngroups=1, dstate=128,
                    io_dtype=ssm.SSM_BF16, delta_softplus=0, x=addr(0), delta=addr(1), A=addr(2),
                    Bm=addr(3), Cm=addr(4), Dskip=addr(5), z=addr(6), delta_bias=None, h0=None,
                    y=addr(7), h_final=addr(8))
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def run_ssd(a):
    return ssm.lib().ssm_ssd_fwd(ctypes.byref(a), None)


@pytest.mark.parametrize("field,value,status", [
    ("io_dtype", 5, ssm.SSM_ERR_BAD_DTYPE),
    ("io_dtype", 5, ssm.SSM_ERR_BAD_DTYPE),
    ("batch", -1, ssm.SSM_ERR_BAD_SHAPE),
    ("nheads", 0, ssm.SSM_ERR_BAD_SHAPE),
    ("ngroups", 3, ssm.SSM_ERR_BAD_SHAPE),                 # does not divide 4 heads
    ("headdim", 48, ssm.SSM_ERR_UNSUPPORTED),             # not a multiple of 32
    ("headdim", 8192, ssm.SSM_ERR_UNSUPPORTED),
    ("dstate", 100, ssm.SSM_ERR_UNSUPPORTED),
    ("dstate", 256, ssm.SSM_ERR_UNSUPPORTED),
    ("delta_softplus", 3, ssm.SSM_ERR_UNSUPPORTED),
    ("x", None, ssm.SSM_ERR_NULL_ARG),
    ("A", None, ssm.SSM_ERR_NULL_ARG),
    ("y", None, ssm.SSM_ERR_NULL_ARG),
    ("x", addr(0, 8), ssm.SSM_ERR_ALIGN),                  # needs 16 bytes
    ("delta", addr(1, 1), ssm.SSM_ERR_ALIGN),
    ("y", addr(0, 256), ssm.SSM_ERR_ALIAS),                # inside x
    ("h_final", addr(7), ssm.SSM_ERR_ALIAS),               # == y
    ("nheads", 1 << 22, ssm.SSM_ERR_UNSUPPORTED),          # batch * nheads * P / 32 > 2^23
])
def test_ssd_rejects_bad_arguments(field, value, status):
    assert run_ssd(ssd_args(**{field: value})) == status


@pytest.mark.parametrize("kw,status", [
    (dict(Bm=addr(3, 4)), ssm.SSM_ERR_ALIGN),       # fp32 B rows are read 16 bytes at a time
    (dict(h0=addr(9, 4)), ssm.SSM_ERR_ALIGN),
    (dict(x=addr(0, 2)), ssm.SSM_ERR_ALIGN),
    (dict(y=addr(0, 4)), ssm.SSM_ERR_ALIAS),         # inside x
])
def test_ssd_fp32_checks(kw, status):
    assert run_ssd(ssd_args(io_dtype=ssm.SSM_F32, **kw)) == status


def test_ssd_fp32_needs_no_workspace_and_passes_the_checks():
    L = ssm.lib()
    a = ssd_args(io_dtype=ssm.SSM_F32, batch=1, nheads=2, seqlen=4096, workspace=None)
    assert L.ssm_ssd_workspace_size(ctypes.byref(a)) == 0
    assert run_ssd(ssd_args(io_dtype=ssm.SSM_F32, x=addr(0, 4))) == ssm.SSM_ERR_HIP   # no device here


def test_ssd_workspace_checks():
    L = ssm.lib()
    # few (batch, head) pairs and a long sequence: segments, so a workspace
    a = ssd_args(batch=1, nheads=2, seqlen=4096, h_final=addr(8), workspace=None)
    need = L.ssm_ssd_workspace_size(ctypes.byref(a))
    assert 0 < need < (1 << 30)
    assert run_ssd(a) == ssm.SSM_ERR_WORKSPACE
    a.workspace, a.workspace_bytes = addr(9), need - 1
    assert run_ssd(a) == ssm.SSM_ERR_WORKSPACE
    a.workspace, a.workspace_bytes = addr(9, 16), need
    assert run_ssd(a) == ssm.SSM_ERR_WORKSPACE          # not 256-aligned
    a.workspace = addr(0)
    assert run_ssd(a) == ssm.SSM_ERR_ALIAS              # == x
    # enough (batch, head) pairs: one pass, no workspace
    assert L.ssm_ssd_workspace_size(ctypes.byref(ssd_args(batch=8, nheads=64, seqlen=4096))) == 0
    assert L.ssm_ssd_workspace_size(ctypes.byref(ssd_args(dstate=100))) == ctypes.c_size_t(-1).value


def test_ssd_empty_batch_is_a_noop():
    assert run_ssd(ssd_args(batch=0)) == ssm.SSM_OK
    assert run_ssd(ssd_args(batch=0, seqlen=0)) == ssm.SSM_OK
    assert ssm.lib().ssm_ssd_fwd(None, None) == ssm.SSM_ERR_NULL_ARG


# ------------------------------------------------------------ SSD step checks
def ssd_step_args(**kw):
    a = ssm.SsdStepArgs(batch=2, nheads=4, headdim=64, ngroups=1, dstate=128,
                        io_dtype=ssm.SSM_BF16, delta_softplus=0, state=addr(0), x=addr(1),
                        delta=addr(2), A=addr(3), Bm=addr(4), Cm=addr(5), Dskip=addr(6), z=addr(7),
                        delta_bias=None, y=addr(8))
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def run_ssd_step(a):
    return ssm.lib().ssm_ssd_step(ctypes.byref(a), None)


@pytest.mark.parametrize("field,value,status", [
    ("io_dtype", 5, ssm.SSM_ERR_BAD_DTYPE),
    ("io_dtype", ssm.SSM_F32, ssm.SSM_ERR_UNSUPPORTED),
    ("batch", -1, ssm.SSM_ERR_BAD_SHAPE),
    ("headdim", 0, ssm.SSM_ERR_BAD_SHAPE),
    ("ngroups", 3, ssm.SSM_ERR_BAD_SHAPE),
    ("dstate", 2, ssm.SSM_ERR_UNSUPPORTED),
    ("dstate", 96, ssm.SSM_ERR_UNSUPPORTED),
    ("dstate", 512, ssm.SSM_ERR_UNSUPPORTED),
    ("delta_softplus", 2, ssm.SSM_ERR_UNSUPPORTED),
    ("state", None, ssm.SSM_ERR_NULL_ARG),
    ("Cm", None, ssm.SSM_ERR_NULL_ARG),
    ("y", None, ssm.SSM_ERR_NULL_ARG),
    ("state", addr(0, 8), ssm.SSM_ERR_ALIGN),
    ("Bm", addr(4, 4), ssm.SSM_ERR_ALIGN),
    ("x", addr(1, 1), ssm.SSM_ERR_ALIGN),
    ("A", addr(3, 2), ssm.SSM_ERR_ALIGN),
    ("y", addr(1), ssm.SSM_ERR_ALIAS),                  # == x
    ("y", addr(0, 1024), ssm.SSM_ERR_ALIAS),            # inside the state
    ("x", addr(0, 64), ssm.SSM_ERR_ALIAS),              # inside the state
    ("nheads", 1 << 20, ssm.SSM_ERR_BAD_SHAPE),         # B*H*P*N/4 > 2^31
])
def test_ssd_step_rejects_bad_arguments(field, value, status):
    assert run_ssd_step(ssd_step_args(**{field: value})) == status


def test_ssd_step_empty_batch_and_null_args():
    assert run_ssd_step(ssd_step_args(batch=0, state=None, x=None)) == ssm.SSM_OK
    assert ssm.lib().ssm_ssd_step(None, None) == ssm.SSM_ERR_NULL_ARG



# ------------------------------------------------------------ measurement keys
def test_kernel_source_hash_ignores_the_checkout_path(monkeypatch):
    """The hash that keys committed counter readings to a kernel build covers the kernel's
    sources and compile flags, not where the repository sits."""
    from selective_state_space_59_amd import build as B
    srcs = ["scan_fwd.hip", "ssm_device.h"]
    ref = B.source_hash(srcs)
    monkeypatch.setattr(B, "COMMON", [f.replace(ROOT, "/elsewhere/checkout") for f in B.COMMON])
    assert B.source_hash(srcs) == ref
    monkeypatch.setattr(B, "COMMON", B.COMMON + ["-DSOMETHING"])
    assert B.source_hash(srcs) != ref
