"""Writes qstar_table.txt: q*(m, f) for m = 0..16 at the f values the workloads use.

The values come from the brute-force definition in the oracle (argmin over every
F of max(F*(65536-f), (m-F)*f), lowest F on ties) and nothing else.
Run: python tests/golden/make_qstar_table.py
"""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from oracle.qstar import qstar_bruteforce  # noqa: E402

F_VALUES = (0, 1, 16384, 26214, 32768, 45875, 49152, 65535, 65536)


def main():
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "qstar_table.txt")
    with open(path, "w") as fh:
        fh.write("# q*(m, f) by brute force over F (oracle.qstar.qstar_bruteforce); rows m = 0..16\n")
        fh.write("# m " + " ".join(str(f) for f in F_VALUES) + "\n")
        for m in range(17):
            fh.write(str(m) + " " + " ".join(str(qstar_bruteforce(m, f)) for f in F_VALUES) + "\n")


if __name__ == "__main__":
    main()
