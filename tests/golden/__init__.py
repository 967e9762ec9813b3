"""Hand-worked block fixtures (hex text, '#' comment lines state the fields and closed forms)."""
import os

import numpy as np

_DIR = os.path.dirname(os.path.abspath(__file__))


def load_block(name: str) -> np.ndarray:
    data = []
    with open(os.path.join(_DIR, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            data.extend(int(tok, 16) for tok in line.split())
    return np.array(data, dtype=np.uint8)
