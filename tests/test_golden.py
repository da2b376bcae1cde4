"""The oracle still reproduces the stored regression fixtures."""

import json
import os

import numpy as np

from oracle import lmhead, philox, verify

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load(name):
    with open(os.path.join(HERE, name)) as f:
        return json.load(f)


def test_small_cases_reproduce():
    for c in load("oracle_small_cases.json"):
        ld = np.array(c["draft"], dtype=np.float32)
        lt = np.array(c["target"], dtype=np.float32)
        tok = np.array(c["tokens"], dtype=np.int32)
        temps = np.array(c["temperature"])
        if c["kind"] == "single":
            r = verify.spec_verify_single(ld, lt, tok, temps, c["seed"], c["offset"])
        else:
            lf = np.array(c["final"], dtype=np.float32)
            r = verify.spec_verify_hier(ld, lt, lf, tok, temps, c["seed"], c["offset"], 4)
        for key, val in c["expect"].items():
            assert r[key].tolist() == val


def test_philox_blocks_reproduce():
    for row in load("oracle_philox_blocks.json"):
        j, b, s, off = row["counter"]
        w = philox.block_words(np.uint64(j), b, s, off, row["seed"])
        assert [int(np.asarray(x)) for x in w] == row["words"]


def test_lmhead_cases_reproduce():
    for c in load("oracle_lmhead_cases.json"):
        r = lmhead.spec_verify_lmhead_single(
            np.array(c["h_draft"], dtype=np.uint16), np.array(c["h_target"], dtype=np.uint16),
            np.array(c["w"], dtype=np.uint16), np.array(c["tokens"], dtype=np.int32),
            np.array(c["temperature"]), c["seed"], c["offset"])
        for key, val in c["expect"].items():
            assert r[key].tolist() == val
