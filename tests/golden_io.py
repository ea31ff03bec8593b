"""Reader for the hand-built fixtures under tests/golden/."""
from __future__ import annotations

import os

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
TYPE_IDS = {"Q4_0": 0, "Q8_0": 1, "Q4_K": 2, "Q6_K": 3, "Q5_0": 4, "Q5_K": 5}


def load(fname: str) -> list[dict]:
    blocks, cur = [], None
    with open(os.path.join(GOLDEN, fname)) as f:
        for raw in f:
            line = raw.strip()
            if not line or line.startswith("#"):
                continue
            key, _, val = line.partition(":")
            key, val = key.strip(), val.strip()
            if key == "name":
                cur = {"name": val}
                blocks.append(cur)
            elif key == "type":
                cur["type"] = TYPE_IDS[val]
            elif key == "hex":
                cur["bytes"] = bytes.fromhex(val)
            elif key in ("expect", "sc", "m", "q_by_g", "q_by_h"):
                cur[key] = [float(v) for v in val.split()]
            elif key in ("rowsum", "q_const"):
                cur[key] = float(val)
            elif key == "spot":
                cur["spot"] = {int(a): float(b) for a, b in (p.split("=") for p in val.split())}
            else:
                raise ValueError("unknown key %r in %s" % (key, fname))
    return blocks
