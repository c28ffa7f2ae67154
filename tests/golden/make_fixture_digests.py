"""Writes fixture_digests.json: SHA-256 of the seeded input bytes of small
workloads, so a change in the generator (or a platform difference in its math
library) shows up as a failing test. Calls only ``fixtures``.

Run from the repository root:  python -m tests.golden.make_fixture_digests
"""
import json
import os

import fixtures as fx

HERE = os.path.dirname(os.path.abspath(__file__))


def current_digests():
    W = fx.WORKLOADS
    cases = {
        "C1": W["C1"],
        "C2-L3000": fx.shrink(W["C2"], 3000),
        "C3-L2500-B2": fx.shrink(W["C3"], 2500, B=2),
        "C4-L4160-B1": fx.shrink(W["C4"], 4160, B=1),
    }
    out = {name: fx.digest(*fx.make_attn(w)) for name, w in cases.items()}
    c5 = fx.shrink(W["C5"], 5000)
    out["C5-L5000-indexer"] = fx.digest(*fx.make_indexer(c5))
    out["C5-L5000-attn"] = fx.digest(*fx.make_attn(c5))
    return out


if __name__ == "__main__":
    with open(os.path.join(HERE, "fixture_digests.json"), "w") as f:
        json.dump(current_digests(), f, indent=1, sort_keys=True)
        f.write("\n")
