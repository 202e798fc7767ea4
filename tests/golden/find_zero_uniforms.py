"""Find Philox counters whose node uniforms are exactly zero.

Writes ``zero_uniforms.txt`` beside this file. A uniform is zero when the top
24 bits of its Philox word are all zero (probability 2^-24), which is the only
way a draw can land exactly on the boundary of a zero-probability token, so
these counters pin the strict inequalities of the acceptance test and of the
inverse-CDF draw. Uses only the oracle's own Philox4x64-10.

Counters searched: (offset, 0, i, 0) under key (seed, 0) for offset = 0, 1, ...;
node i = 1 for the acceptance word (the root is never tested), i = 0 for the
resampling word.
"""

import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__)))))
import oracle  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "zero_uniforms.txt")


def search(seed: int, node: int, word: int, chunk: int = 1 << 20, limit: int = 1 << 28) -> int:
    for start in range(0, limit, chunk):
        ctr = np.zeros((chunk, 4), np.uint64)
        ctr[:, 0] = np.arange(start, start + chunk, dtype=np.uint64)
        ctr[:, 2] = node
        w = oracle.philox4x64_10(ctr, (seed, 0))
        hit = np.nonzero((w[:, word] >> np.uint64(40)) == 0)[0]
        if hit.size:
            return start + int(hit[0])
    raise RuntimeError("no zero uniform found")


def main():
    seed = 0
    acc = search(seed, 1, 0)
    res = search(seed, 0, 1)
    with open(OUT, "w") as f:
        f.write("# Philox4x64-10 counters (offset, 0, node, 0) under key (seed, 0) whose word\n")
        f.write("# has zero top 24 bits, i.e. a node uniform of exactly 0. Written by\n")
        f.write("# find_zero_uniforms.py with the oracle's Philox.\n")
        f.write("# kind seed offset node   (acceptance: word 0; resample: word 1; b = 0)\n")
        f.write(f"acceptance {seed} {acc} 1\n")
        f.write(f"resample {seed} {res} 0\n")
    print(open(OUT).read())


if __name__ == "__main__":
    main()
