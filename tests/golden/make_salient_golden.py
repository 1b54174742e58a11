"""Writes the oracle's expected mixed-precision (fp16 salient channels)
results for the full-size search workload (W[11008, 4096], calibration
X[65536, 4096], G = 128, round(K / 100) = 41 salient channels) into
salient_7b_mlp_wmult1.json: the chosen channels, the plain quantizer's
output loss and the mixed layer's.

Calls only the oracle and the seeded input generators: the stored values are
the oracle's (exact Gram route), never the GPU's.

    python tests/golden/make_salient_golden.py
"""

from __future__ import annotations

import base64
import hashlib
import json
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import synth  # noqa: E402


def digest(*arrays) -> str:
    h = hashlib.sha256()
    for a in arrays:
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()


def main() -> None:
    t0 = time.time()
    lay = synth.search_layer(w_mult=1.0)
    w, x = lay["w"], lay["x"]
    K = w.shape[1]
    n = oracle.salient_count(K)
    idx = oracle.salient_channels(oracle.activation_absmean(x), n)
    g = oracle.gram(x)
    w64 = np.asarray(w).astype(np.float64)
    losses = []
    for sel in (idx[:0], idx):
        d = oracle.mixed_weight(w, 128, sel) - w64
        losses.append(float(np.sum((d @ g) * d)))
    rec = {
        "what": "oracle mixed-precision loss (Gram route) on the 7B MLP-shaped search workload",
        "shape": {"N": int(w.shape[0]), "K": int(K), "T": int(x.shape[0]), "group_size": 128},
        "inputs_sha256": digest(w, x),
        "n_salient": n,
        "idx_i64_b64": base64.b64encode(idx.astype("<i8").tobytes()).decode(),
        "loss_rtn": losses[0],
        "loss_salient": losses[1],
        "oracle_seconds": round(time.time() - t0, 1),
    }
    path = os.path.join(HERE, "salient_7b_mlp_wmult1.json")
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
    print(path, rec["loss_rtn"], rec["loss_salient"], rec["oracle_seconds"], "s")


if __name__ == "__main__":
    main()
