"""Reader of the golden fixtures: `key = python literal` lines, `#` comments."""
import ast
import os

HERE = os.path.dirname(os.path.abspath(__file__))


def load(name):
    out = {}
    with open(os.path.join(HERE, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, val = line.split("=", 1)
            out[key.strip()] = ast.literal_eval(val.strip())
    return out
