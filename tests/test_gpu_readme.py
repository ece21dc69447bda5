"""The Python example in README.md runs as written and gives outputs of the stated shapes."""
import os
import re

import pytest

README = os.path.join(os.path.dirname(__file__), "..", "README.md")


@pytest.mark.gpu
def test_readme_example_runs():
    import torch
    text = open(README).read()
    blocks = re.findall(r"```python\n(.*?)```", text, re.S)
    assert len(blocks) == 1
    env = {}
    exec(compile(blocks[0], "README.md", "exec"), env)
    torch.cuda.synchronize()
    B, T, Hq, Hv = env["B"], env["T"], env["Hq"], env["Hv"]
    assert tuple(env["T_"].shape) == (B, T, Hv, 64) and env["T_"].dtype == torch.float32
    assert tuple(env["W"].shape) == (B, T, Hv, 128) and tuple(env["U"].shape) == (B, T, Hv, 128)
    assert tuple(env["dk"].shape) == (B, T, Hq, 128) and tuple(env["dg"].shape) == (B, T, Hv)
    assert tuple(env["o"].shape) == (B, T, Hv, 128)
    assert tuple(env["state"].shape) == (B, Hv, 128, 128)
    for name in ("T_", "W", "U", "dk", "dv", "dbeta", "dg", "o", "state"):
        assert torch.isfinite(env[name].float()).all(), name
