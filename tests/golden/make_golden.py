"""Writes the stored expected values under tests/golden/.

Calls only ``oracle/`` and plain Python arithmetic.  Run from the repo root:
    python tests/golden/make_golden.py
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from oracle import QUINTIC, CUBIC, scalar_map  # noqa: E402


def main():
    out = {
        "_about": (
            "Action of the NS iteration on one singular value, phi^(s)(sigma) with "
            "phi(sigma) = a*sigma + b*sigma^3 + c*sigma^5 (DMuon technical summary, "
            "gist.science ko, §2.2; polynomial form is the plainest reading). "
            "Written by tests/golden/make_golden.py from oracle.scalar_map."),
        "quintic": list(QUINTIC),
        "quintic_phi5_of_1": scalar_map(1.0, QUINTIC, 5),
        "quintic_phi1_of_1": scalar_map(1.0, QUINTIC, 1),
        "cubic": list(CUBIC),
        "cubic_phi30_of_0.05": scalar_map(0.05, CUBIC, 30),
    }
    with open(os.path.join(HERE, "scalar_map.json"), "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")


if __name__ == "__main__":
    main()
