import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


_gpu_session = {"used": False, "status": 0}


def pytest_sessionfinish(session, exitstatus):
    """Close the shared GPU context while the runtime is fully up."""
    _gpu_session["status"] = int(exitstatus)
    mod = sys.modules.get("gpu_common")
    if mod is not None and getattr(mod, "_ctx", None) is not None:
        _gpu_session["used"] = True
        try:
            import torch
            torch.cuda.synchronize()
            mod._ctx.close()
        except Exception:
            pass
        mod._ctx = None


def pytest_unconfigure(config):
    """After a session that used the GPU, end the process here with the session's status: every
    result is final and reported, and the GPU runtime's own teardown at interpreter exit is not
    part of what the tests check."""
    if _gpu_session["used"]:
        sys.stdout.flush()
        sys.stderr.flush()
        os._exit(_gpu_session["status"])
