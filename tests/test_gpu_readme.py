"""The Python example in README.md runs as written (needs an MI355X)."""
import os
import re

import pytest
import torch

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_readme_example_runs():
    text = open(os.path.join(ROOT, "README.md")).read()
    blocks = re.findall(r"```python\n(.*?)```", text, flags=re.S)
    assert blocks, "README.md has no python example"
    env = {}
    exec(compile(blocks[0], "README.md", "exec"), env)
    torch.cuda.synchronize()
    y, h, y1 = env["y"], env["h"], env["y1"]
    assert y.shape == (2, 4096, 1536) and h.shape == (2, 1536, 16) and y1.shape == (2, 1536)
    assert torch.isfinite(y.float()).all() and torch.isfinite(h).all() and torch.isfinite(y1.float()).all()
    g = env["grads"]
    assert g["dx"].shape == (2, 4096, 1536) and g["dA"].shape == (1536, 16)
    assert all(torch.isfinite(v.float()).all() for v in g.values())
    xs = env["xs"]
    assert xs.grad is not None and xs.grad.shape == xs.shape and torch.isfinite(xs.grad.float()).all()
