"""Writes the regression anchors in this folder from the oracle alone.

Run from the repository root:  python tests/golden/make_golden.py
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402


def main():
    out = {
        "_about": "sigma schedules from oracle.schedule; regression anchors, not page values",
        "n4_li4096": [float(x) for x in oracle.schedule(4, 4096)],
        "n4_li4096_terminal": [float(x) for x in oracle.schedule(4, 4096, sigma_terminal=0.02)],
        "n50_li4096": [float(x) for x in oracle.schedule(50, 4096)],
        "n4_li1024": [float(x) for x in oracle.schedule(4, 1024)],
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "schedule_anchor.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print("wrote", path)


if __name__ == "__main__":
    main()
