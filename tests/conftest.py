import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def parse_golden(path):
    """Parse tests/golden/*.txt: sections of `bytes:` / `expect:` / `codebook r:` lines."""
    sections, cur = {}, None
    with open(path) as f:
        for raw in f:
            line = raw.split("#", 1)[0].strip()
            if not line:
                continue
            if line.startswith("[") and line.endswith("]"):
                cur = {"bytes": [], "expect": [], "codebook": {}}
                sections[line[1:-1]] = cur
                continue
            key, _, rest = line.partition(":")
            toks = rest.split()
            if key == "bytes":
                for t in toks:
                    v, _, n = t.partition("*")
                    cur["bytes"] += [int(v, 16)] * (int(n) if n else 1)
            elif key == "expect":
                for t in toks:
                    v, _, n = t.partition("*")
                    cur["expect"] += [float(v)] * (int(n) if n else 1)
            elif key.startswith("codebook"):
                cur["codebook"][int(key.split()[1])] = [int(t) for t in toks]
            else:
                raise ValueError(f"bad golden line: {raw!r}")
    return sections


@pytest.fixture(scope="session")
def golden_blocks():
    return parse_golden(os.path.join(ROOT, "tests", "golden", "format_blocks.txt"))
