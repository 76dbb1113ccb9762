import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


def pytest_runtest_logstart(nodeid, location):
    # name each case on the real stderr before it runs, so a run that dies mid-test still says
    # which case it was in
    sys.__stderr__.write(f"[start] {nodeid}\n")
    sys.__stderr__.flush()
