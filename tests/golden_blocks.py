"""Reader for tests/golden/q4k_blocks.txt (hand-derived Q4_K blocks)."""
import os

import numpy as np

PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                    "q4k_blocks.txt")


def load(path=PATH):
    blocks = []
    cur = None
    with open(path) as f:
        for raw in f:
            line = raw.split("#", 1)[0].strip()
            if not line:
                continue
            key, _, rest = line.partition(" ")
            toks = rest.split()
            if key == "block":
                cur = {"name": toks[0], "q": {}, "w": {}, "wbits": {}}
            elif key == "d":
                cur["d"] = int(toks[0], 16)
            elif key == "dmin":
                cur["dmin"] = int(toks[0], 16)
            elif key == "scales":
                cur["scales"] = bytes(int(t, 16) for t in toks)
            elif key == "qs":
                if toks[0] == "range":
                    cur["qs"] = bytes(range(128))
                else:
                    cur["qs"] = bytes([int(toks[1], 16)] * 128)
            elif key in ("sc", "m"):
                cur[key] = [int(t) for t in toks]
            elif key == "q":
                cur["q"].update({int(a): int(b) for a, b in (t.split(":") for t in toks)})
            elif key == "w":
                cur["w"].update({int(a): float(b) for a, b in (t.split(":") for t in toks)})
            elif key == "wbits":
                cur["wbits"].update({int(a): int(b, 16) for a, b in (t.split(":") for t in toks)})
            elif key == "end":
                raw_block = (cur["d"].to_bytes(2, "little") + cur["dmin"].to_bytes(2, "little")
                             + cur["scales"] + cur["qs"])
                assert len(raw_block) == 144, cur["name"]
                cur["bytes"] = np.frombuffer(raw_block, np.uint8).copy()
                blocks.append(cur)
                cur = None
            else:
                raise ValueError(f"unknown golden line: {raw!r}")
    return blocks
