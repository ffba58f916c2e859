"""Reader of the hand-worked fixtures under ``tests/golden/``."""
import collections
import os

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def single_voxel_taps():
    """{(theta_degrees, u_offset): {channel: weight}} from
    ``golden/single_voxel_taps.txt`` (channels not listed are 0)."""
    out = collections.defaultdict(dict)
    with open(os.path.join(HERE, "single_voxel_taps.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            th, off, ch, w = line.split()
            out[(float(th), float(off))][int(ch)] = float(w)
    return dict(out)
