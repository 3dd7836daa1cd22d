"""Readers for the hand-derived text fixtures in this folder."""
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))


def overwrite_recall(name: str = "overwrite_recall_onehot.txt"):
    """Return dict(keys, queries, v, o_expected, S_expected) from a recall fixture."""
    keys, queries, vs, os_, srows = [], [], [], [], {}
    with open(os.path.join(HERE, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            head, *rest = [p.strip() for p in line.split("|")]
            h = head.split()
            if h[0] == "S":
                srows[int(h[1])] = [float(x) for x in rest[0].split()]
                continue
            keys.append(int(h[1]))
            queries.append(int(h[2]))
            vs.append([float(x) for x in rest[0].split()])
            os_.append([float(x) for x in rest[1].split()])
    S = np.array([srows[i] for i in sorted(srows)], dtype=np.float64)
    return dict(keys=np.array(keys), queries=np.array(queries), v=np.array(vs, dtype=np.float64),
                o_expected=np.array(os_, dtype=np.float64), S_expected=S)
