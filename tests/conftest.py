import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running")
    # a planted oracle mistake, for the mutation test's child processes only
    if os.environ.get("AR_ORACLE_MUTANT"):
        from oracle_mutants import apply
        apply(os.environ["AR_ORACLE_MUTANT"])
