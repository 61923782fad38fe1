"""The library called from several host threads at once: tests/cabi/
threaded_first_calls.py makes every packed, joint and GGUF-layout entry
point's first call of a fresh process from racing threads, each on its own
stream, and checks each result bit for bit against the same call repeated on
the main thread."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _gpu_present():
    try:
        import torch
    except ImportError:
        return False
    return torch.cuda.device_count() > 0


if not _gpu_present():
    pytest.skip("needs a GPU", allow_module_level=True)


def test_first_calls_from_racing_threads():
    script = os.path.join(ROOT, "tests", "cabi", "threaded_first_calls.py")
    print("running", script, flush=True)
    r = subprocess.run([sys.executable, "-u", script], capture_output=True, text=True,
                       timeout=180)
    print(r.stdout[-4000:], r.stderr[-4000:], flush=True)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]
    assert "threads ok" in r.stdout
