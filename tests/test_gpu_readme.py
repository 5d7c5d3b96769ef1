"""The Python example in README.md runs as written (bf16, the headline shape)."""

import os
import re

import pytest

pytestmark = pytest.mark.gpu

README = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "README.md")


def test_readme_example_runs():
    import torch
    code = re.search(r"```python\n(.*?)```", open(README).read(), re.S).group(1)
    scope = {}
    exec(compile(code, "README.md", "exec"), scope)
    torch.cuda.synchronize()
    for name in ("o", "dq", "dk", "dv"):
        assert torch.isfinite(scope[name].float()).all(), name
