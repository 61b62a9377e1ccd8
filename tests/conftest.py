import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


# A run of the host tests against the sanitizer build of the host C++ (see
# tests/test_sanitized_host.py) points the binding at that library before any test loads it.
if os.environ.get("TV_SANITIZED_LIB"):
    import tree_attention_draft_amd._binding as _binding
    _binding.LIB_PATH = os.environ["TV_SANITIZED_LIB"]


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long CPU test")
