import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: full-size inputs (minutes of host work)")


def read_golden(name):
    """Parse a golden fixture: 'key: v v v' lines, repeated keys append rows;
    '#' lines are comments.  Integers may be hex (0x..)."""
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, _, rest = line.partition(":")
            vals = []
            for tok in rest.split():
                if tok.lower().startswith("0x"):
                    vals.append(int(tok, 16))
                elif any(ch in tok for ch in ".eE") and not tok.lstrip("-").isdigit():
                    vals.append(float(tok))
                else:
                    vals.append(int(tok))
            out.setdefault(key.strip(), []).append(vals)
    return out


@pytest.fixture(scope="session")
def orc():
    import oracle
    if not os.path.exists(oracle.LIB_PATH):
        oracle.build()
    return oracle
