"""Writes the oracle's expected scale-search results for the full-size search
workload (W[11008, 4096], calibration X[65536, 4096] = 128 x 512 tokens,
alpha_i = i/20, G = 128) into search_7b_mlp_*.json.

Calls only the oracle and the seeded input generators: the stored values are
the oracle's (exact Gram route), never the GPU's.

    python tests/golden/make_search_golden.py [w_mult ...]
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


def golden_path(w_mult: float) -> str:
    return os.path.join(HERE, f"search_7b_mlp_wmult{int(w_mult)}.json")


def main(w_mults) -> None:
    for w_mult in w_mults:
        t0 = time.time()
        lay = synth.search_layer(w_mult=w_mult)
        w, x = lay["w"], lay["x"]
        alphas = oracle.alpha_grid(synth.SEARCH_N_ALPHA)
        losses, best, s = oracle.scale_search(w, x, 128, alphas=alphas, use_gram=True)
        m = oracle.activation_absmean(x)
        rec = {
            "what": "oracle scale search (Gram route) on the 7B MLP-shaped search workload",
            "shape": {"N": int(w.shape[0]), "K": int(w.shape[1]), "T": int(x.shape[0]), "group_size": 128},
            "w_mult": w_mult,
            "inputs_sha256": digest(w, x),
            "alphas": alphas.tolist(),
            "losses": losses.tolist(),
            "best_index": best,
            "m_f64_b64": base64.b64encode(m.astype("<f8").tobytes()).decode(),
            "best_scales_f32_b64": base64.b64encode(s.astype("<f4").tobytes()).decode(),
            "oracle_seconds": round(time.time() - t0, 1),
        }
        with open(golden_path(w_mult), "w") as f:
            json.dump(rec, f, indent=1)
        print(golden_path(w_mult), "best", best, "in", rec["oracle_seconds"], "s", flush=True)


if __name__ == "__main__":
    main([float(a) for a in sys.argv[1:]] or [1.0, 10.0])
