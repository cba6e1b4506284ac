import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    # GPU tests are selected with -m gpu and fail loudly (never skip) when no GPU or no built
    # library is present.
    config.addinivalue_line("markers", "gpu: needs an AMD GPU (MI355X) and the built HIP library")
