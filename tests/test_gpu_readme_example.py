"""The README's Python example runs as printed (the generation path with a
folded gain, then one layer's training forward and backward)."""
import os
import re

import pytest

from tests.conftest import ROOT

pytestmark = pytest.mark.gpu


def _example() -> str:
    text = open(os.path.join(ROOT, "README.md"), encoding="utf-8").read()
    section = text[text.index("## Using it from Python"):]
    return re.search(r"```python\n(.*?)```", section, re.S).group(1)


def test_readme_example_runs():
    pytest.importorskip("yoco_shared_kv_amd")
    print("README example: generation path with a folded gain, prefill forward and backward", flush=True)
    scope: dict = {}
    exec(compile(_example(), "README.md", "exec"), scope)
    import torch
    torch.cuda.synchronize()
    assert scope["d_k"].abs().sum().item() > 0 and torch.isfinite(scope["d_q"]).all()
