"""Writes the oracle regression fixtures in this folder. Calls only ``oracle/`` and numpy.

Run from the repository root:  python tests/golden/make_golden.py

The fixture freezes the oracle's output for one tiny seeded case (two heads of D=32,
70 tokens, window 32, key bits 2 and value bits 4), so that any later change to the
oracle's arithmetic shows up as a failing test and has to be justified by a passage of
the pages ("Changelog" v0.8.0 KIVI, v0.42.0 fused decode + attention, v0.30.0 lo/scale).
"""
import json
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__)))))
from oracle import kivi  # noqa: E402

HERE = os.path.dirname(os.path.abspath(__file__))


def case():
    rng = np.random.default_rng(2024)
    H, S, D = 2, 70, 32
    K = rng.standard_normal((H, S, D)).astype(np.float32)
    K[:, :, 3] *= 10
    K = K.astype(np.float16)
    V = rng.standard_normal((H, S, D)).astype(np.float16)
    q = (rng.standard_normal((1, H, D)) / np.sqrt(D)).astype(np.float16)
    return K, V, q


def compute(K, V, q):
    seqs = []
    for h in range(K.shape[0]):
        s = kivi.KiviSequence(K.shape[2], 2, 4, 32, 32)
        s.prefill(K[h], V[h])
        seqs.append(s)
    out = kivi.decode_attend(q, [seqs])
    return seqs, out


def main():
    K, V, q = case()
    seqs, out = compute(K, V, q)
    rec = {
        "inputs_fp16_bits": {"K": K.view(np.uint16).tolist(), "V": V.view(np.uint16).tolist(),
                             "q": q.view(np.uint16).tolist()},
        "heads": [{
            "n_q": s.n_q, "n_r": s.n_r,
            "key_codes": s.kc.tolist(), "key_scale_bits": s.ks.view(np.uint16).tolist(),
            "key_zero_bits": s.kz.view(np.uint16).tolist(),
            "value_codes": s.vc.tolist(), "value_scale_bits": s.vs.view(np.uint16).tolist(),
            "value_zero_bits": s.vz.view(np.uint16).tolist(),
        } for s in seqs],
        "out_fp64_hex": [[float(x).hex() for x in row] for row in out[0]],
    }
    with open(os.path.join(HERE, "oracle_tiny_d32.json"), "w") as f:
        json.dump(rec, f, separators=(",", ":"))


if __name__ == "__main__":
    main()
