"""The oracle's pins are strong enough to catch plausible mistakes: with each
planted mistake of oracle_mutants.py compiled into the oracle (in a child
pytest process), at least one pin of test_oracle_pins.py or
test_block_oracle.py must fail."""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

from oracle_mutants import MUTANTS, apply, target

HERE = os.path.dirname(os.path.abspath(__file__))
PINS = [os.path.join(HERE, "test_oracle_pins.py"), os.path.join(HERE, "test_block_oracle.py")]


def _run_pins(mutant):
    env = dict(os.environ, AR_ORACLE_MUTANT=mutant)
    r = subprocess.run([sys.executable, "-m", "pytest", *PINS, "-x", "-q", "-p", "no:cacheprovider",
                        "-m", "not gpu"], cwd=os.path.dirname(HERE), env=env,
                       capture_output=True, text=True, timeout=600)
    return mutant, r.returncode, r.stdout[-2000:]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_applies(name):
    """Every edit still matches the oracle's source exactly once and compiles."""
    import oracle
    mod, fname = target(name)
    orig = mod.__dict__[fname]
    orig_pkg = getattr(oracle, fname, None)
    try:
        apply(name)
        assert mod.__dict__[fname] is not orig
    finally:
        mod.__dict__[fname] = orig
        if orig_pkg is not None:
            setattr(oracle, fname, orig_pkg)


def test_every_mutant_fails_a_pin():
    with ThreadPoolExecutor(max_workers=4) as ex:
        results = list(ex.map(_run_pins, sorted(MUTANTS)))
    survivors = [(m, out) for m, rc, out in results if rc == 0]
    broken = [(m, rc, out) for m, rc, out in results if rc not in (0, 1)]
    assert not broken, "pins did not run under: " + ", ".join(
        f"{m} (exit {rc}): {out[-400:]}" for m, rc, out in broken)
    assert not survivors, "no pin fails under: " + ", ".join(m for m, _ in survivors)
