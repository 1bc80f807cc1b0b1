"""Plant plausible mistakes in a copy of the KV cache model and check that
the pins catch every one (on the CPU)."""
import importlib.util
import os

import pytest

from tests import test_oracle_kv_pins as pins

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "kv_oracle.py")

MUTATIONS = {
    "window_one_short": ("lo = max(0, p - self.W + 1)", "lo = max(0, p - self.W + 2)"),
    "window_excludes_self": ("ks = self.k[layer][lo:p + 1]", "ks = self.k[layer][lo:p]"),
    "drops_one_too_many": ("drop = K - 1 - n_accepted", "drop = K - n_accepted"),
    "keeps_rejected_rows": ("drop = K - 1 - n_accepted", "drop = 0"),
    "concat_counts_window_only": ("rows = window + K - 1", "rows = window"),
}


def _load_mutant(tmp_path, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1
    path = tmp_path / "kv_mutant.py"
    path.write_text(src.replace(old, new))
    spec = importlib.util.spec_from_file_location("kv_mutant", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_kv_pins_catch_planted_mistake(name, tmp_path):
    mod = _load_mutant(tmp_path, *MUTATIONS[name])
    caught = False
    for check in pins.CHECKS:
        try:
            check(mod)
        except (AssertionError, ValueError, RuntimeError, IndexError):
            caught = True
            break
    assert caught, "pins did not catch %s" % name
