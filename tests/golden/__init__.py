"""Loader for the small text fixtures in this folder."""
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))


def load(name):
    """Parse a fixture: '[name d0 d1 ...]' headers followed by whitespace-separated values;
    '#' starts a comment.  Returns {name: float64 array of that shape}."""
    arrays, cur, shape, vals = {}, None, None, []
    with open(os.path.join(HERE, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            if line.startswith("["):
                if cur is not None:
                    arrays[cur] = np.array(vals, dtype=np.float64).reshape(shape)
                parts = line.strip("[]").split()
                cur, shape, vals = parts[0], tuple(int(p) for p in parts[1:]), []
            else:
                vals.extend(float(v) for v in line.split())
    if cur is not None:
        arrays[cur] = np.array(vals, dtype=np.float64).reshape(shape)
    return arrays
