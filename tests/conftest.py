import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long CPU test (opt-in with -m slow)")


def load_golden_cases(name):
    """Parse tests/golden/hand_worked_gemv.txt into dicts of numpy arrays."""
    import numpy as np

    path = os.path.join(ROOT, "tests", "golden", name)
    cases, cur = [], None

    def expand(tokens):
        # words / scales: "HEX" or "HEX*COUNT"
        out = []
        for t in tokens:
            if "*" in t:
                hx, cnt = t.split("*")
                out += [int(hx, 16)] * int(cnt)
            else:
                out.append(int(t, 16))
        return out

    with open(path) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            tok = line.split()
            if tok[0] == "case":
                N, K = int(tok[2]), int(tok[3])
                cur = dict(name=tok[1], N=N, K=K,
                           words=np.full((N, K // 8), 0x77777777, np.uint32),
                           scales=np.zeros((N, K // 32), np.uint16),
                           x=None, y16=np.zeros(N, np.uint16), y=np.zeros(N))
                cases.append(cur)
            elif tok[0] == "words":
                vals = expand(tok[2:])
                cur["words"][int(tok[1]), :len(vals)] = vals
            elif tok[0] == "scales":
                vals = expand(tok[2:])
                cur["scales"][int(tok[1]), :len(vals)] = vals
            elif tok[0] == "x":
                vals = []
                for t in tok[1:]:
                    cnt, hx = t.split("*")
                    vals += [int(hx, 16)] * int(cnt)
                cur["x"] = np.array(vals, np.uint16)
                assert len(cur["x"]) == cur["K"]
            elif tok[0] == "y":
                r = int(tok[1])
                cur["y16"][r] = int(tok[2], 16)
                cur["y"][r] = float(tok[3])
    return cases


def load_page_figures():
    path = os.path.join(ROOT, "tests", "golden", "page_figures.txt")
    out = {}
    with open(path) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            tok = line.split()
            out.setdefault(tok[0], []).append([float(t) for t in tok[1:]])
    return out
