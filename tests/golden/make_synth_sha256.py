"""Writes tests/golden/synth_sha256.txt: SHA-256 of the seeded generator's
outputs for fixed (config, layer, shape, format) keys, so that a change to the
generator (or to the numpy random streams it draws from) is caught.  Calls only
the generator (hxq_synth), with its on-disk cache off.

Usage: python tests/golden/make_synth_sha256.py
"""

import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))
os.environ["HXQ_SYNTH_CACHE"] = ""

from hxq_synth import gen  # noqa: E402

# (label, generator call): the 256 x 256 u8 layer of the single-layer
# configuration, a small pk12 layer (2D k-means of 6144 pairs into 4096 entries), a small u8
# layer with the pk12 configuration's sidecar density, activations, and a
# random parity layer
CASES = [
    ("config0_layer0_u8_256x256", lambda: gen.config_layers(0)[0]),
    ("cfg3_layer0_pk12_96x128", lambda: gen.synth_layer(3, 0, 96, 128, "pk12", 2000)),
    ("cfg2_layer1_u8_48x96_den2000", lambda: gen.synth_layer(2, 1, 48, 96, "u8", 2000)),
    ("random_layer_7_pk12_40x64", lambda: gen.random_layer(7, 40, 64, "pk12", nnz=30, duplicates=True)),
]
X_CASES = [("synth_x_cfg1_layer4_8x2048", lambda: gen.synth_x(1, 4, 8, 2048))]


def digests():
    import hashlib

    import numpy as np

    out = []
    for label, fn in CASES:
        lay = fn()
        for field, h in sorted(lay.sha256().items()):
            out.append((label, field, h))
    for label, fn in X_CASES:
        out.append((label, "x", hashlib.sha256(np.ascontiguousarray(fn()).tobytes()).hexdigest()))
    return out


if __name__ == "__main__":
    path = os.path.join(HERE, "synth_sha256.txt")
    with open(path, "w") as f:
        f.write("# SHA-256 of seeded generator outputs (written by make_synth_sha256.py)\n")
        f.write("# label field sha256\n")
        for row in digests():
            f.write("%s %s %s\n" % row)
    print("wrote", path)
