"""The README's Python example runs as written (shapes and finite outputs)."""

import os
import re

import pytest

README = os.path.join(os.path.dirname(os.path.dirname(__file__)), "README.md")


def _example():
    text = open(README, encoding="utf-8").read()
    blocks = re.findall(r"```python\n(.*?)```", text, re.S)
    assert len(blocks) == 1, "README holds one Python example"
    return blocks[0]


def test_readme_example_parses():
    compile(_example(), "README.md", "exec")


@pytest.mark.gpu
def test_readme_example_runs():
    import torch
    torch.manual_seed(0)          # the example draws its own inputs
    env = {}
    exec(compile(_example(), "README.md", "exec"), env)
    torch.cuda.synchronize()
    B, H, N, d = env["B"], env["H"], env["N"], env["d"]
    for name in ("o", "dq", "dk", "dv"):
        t = env[name]
        assert tuple(t.shape) == (B, H, N, d), name
        assert torch.isfinite(t.float()).all(), name
    assert tuple(env["out"].shape) == (B, env["Hq"], 128)
    assert torch.isfinite(env["out"].float()).all()
