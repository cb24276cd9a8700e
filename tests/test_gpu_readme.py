"""The README's Python example runs as written on the GPU."""
import os
import re

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_readme_python_example_runs(dev):
    text = open(os.path.join(ROOT, "README.md")).read()
    code = re.search(r"```python\n(.*?)```", text, re.S).group(1)
    scope = {}
    exec(compile(code, "README.md", "exec"), scope)
    assert scope["flags"] == 0
    assert scope["idx"].shape == (8, 1 << 16)
