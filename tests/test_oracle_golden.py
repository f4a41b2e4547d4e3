"""The oracle still reproduces its frozen fixture (tests/golden/oracle_tiny_d32.json)."""
import json
import os

import numpy as np

from tests.golden.make_golden import compute

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_oracle_matches_frozen_fixture():
    with open(os.path.join(HERE, "oracle_tiny_d32.json")) as f:
        rec = json.load(f)
    inp = rec["inputs_fp16_bits"]
    K = np.array(inp["K"], np.uint16).view(np.float16)
    V = np.array(inp["V"], np.uint16).view(np.float16)
    q = np.array(inp["q"], np.uint16).view(np.float16)
    seqs, out = compute(K, V, q)
    for s, h in zip(seqs, rec["heads"]):
        assert (s.n_q, s.n_r) == (h["n_q"], h["n_r"])
        assert s.kc.tolist() == h["key_codes"] and s.vc.tolist() == h["value_codes"]
        assert s.ks.view(np.uint16).tolist() == h["key_scale_bits"]
        assert s.kz.view(np.uint16).tolist() == h["key_zero_bits"]
        assert s.vs.view(np.uint16).tolist() == h["value_scale_bits"]
        assert s.vz.view(np.uint16).tolist() == h["value_zero_bits"]
    expect = np.array([[float.fromhex(x) for x in row] for row in rec["out_fp64_hex"]])
    # float64 attention: BLAS summation order may differ between machines
    assert np.max(np.abs(out[0] - expect)) < 1e-13
