import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")

def pytest_sessionfinish(session, exitstatus):
    """Close the shared GPU context while the runtime is fully up."""
    mod = sys.modules.get("gpu_common")
    if mod is not None and getattr(mod, "_ctx", None) is not None:
        try:
            import torch
            torch.cuda.synchronize()
            mod._ctx.close()
        except Exception:
            pass
        mod._ctx = None
