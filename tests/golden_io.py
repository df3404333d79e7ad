"""Reader for the hand-built block fixtures in tests/golden/ (format described in the file)."""
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
BLOCK_BYTES = {"q4_k": 144, "q6_k": 210, "q8_0": 34, "q5_k": 176, "q4_0": 18}
BLOCK_WEIGHTS = {"q4_k": 256, "q6_k": 256, "q8_0": 32, "q5_k": 256, "q4_0": 32}


def _value(tok: str) -> float:
    if tok.lstrip("-").startswith("0x"):
        return float.fromhex(tok)
    return float(tok)


def load_blocks(name: str = "kquant_blocks.txt"):
    """List of dicts: name, type, block (uint8 array), expect (float64 array, weights order)."""
    out = []
    cur = None
    with open(os.path.join(GOLDEN, name)) as f:
        for raw in f:
            line = raw.split("#", 1)[0].strip()
            if not line:
                continue
            parts = line.split()
            op = parts[0]
            if op == "block":
                cur = {"name": parts[1], "type": None, "bytes": None, "expect": []}
            elif op == "type":
                cur["type"] = parts[1]
                cur["bytes"] = np.zeros(BLOCK_BYTES[parts[1]], np.uint8)
            elif op == "set":
                off = int(parts[1])
                vals = [int(h, 16) for h in parts[2:]]
                cur["bytes"][off:off + len(vals)] = vals
            elif op == "fill":
                off, cnt, val = int(parts[1]), int(parts[2]), int(parts[3], 16)
                cur["bytes"][off:off + cnt] = val
            elif op == "expect_runs":
                run = int(parts[1])
                for tok in parts[2:]:
                    cur["expect"].extend([_value(tok)] * run)
            elif op == "end":
                exp = np.array(cur["expect"], np.float64)
                assert exp.size == BLOCK_WEIGHTS[cur["type"]], cur["name"]
                out.append({"name": cur["name"], "type": cur["type"], "block": cur["bytes"],
                            "expect": exp})
                cur = None
            else:
                raise ValueError(f"unknown directive {op!r}")
    return out
