import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library")


@pytest.fixture(scope="session")
def lib():
    """The built C-ABI library through its Python binding (GPU tests only)."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import diffusion_transformer_spatially_amd as dts
    dts.load()
    return dts


def pytest_terminal_summary(terminalreporter):
    """Worst-row errors of the parity assertions (the data behind the per-row bounds)."""
    try:
        from tests.gpu_util import ROW_STATS
    except Exception:  # pragma: no cover
        return
    if not ROW_STATS:
        return
    for dt in ("bf16", "f32"):
        st = sorted((s for s in ROW_STATS if s[1] == dt), key=lambda s: -s[2])
        if st:
            terminalreporter.write_line(f"worst rows ({dt}, {len(st)} assertions): " +
                                        "; ".join(f"{w}: row {r:.2e} l2 {l:.2e}" for w, _, r, l in st[:6]))
    path = os.environ.get("SAFE_ROW_STATS")
    if path:
        import json
        with open(path, "w") as f:
            json.dump(ROW_STATS, f)
