"""Writes the regression fixtures in this folder.  Calls only ``oracle/``
(inputs come from a seeded NumPy generator written out in full).

The pages print no worked numeric example (no logits, probabilities or
tokens), so these fixtures are not the pages' values: they freeze the oracle's
output on small fixed inputs so that any later change to its arithmetic shows
up in ``tests/test_golden.py`` and has to be justified.

Run:  python tests/golden/make_golden.py
"""

import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from oracle import lmhead, philox, verify  # noqa: E402


def small_cases():
    rng = np.random.default_rng(20251001)
    cases = []
    for idx, (B, k, V, kind) in enumerate([(3, 4, 37, "single"), (4, 3, 50, "hier"),
                                           (2, 5, 23, "single")]):
        temps = [1.0, 0.7, 0.0, 1.3][:B]
        ld = np.round(rng.normal(0, 2, (B, k, V)), 2).astype(np.float32)
        lt = np.round(0.8 * rng.normal(0, 2, (B, k + 1, V)), 2).astype(np.float32)
        lt[:, :k] += np.round(0.6 * ld, 2)
        lf = np.round(0.7 * lt + rng.normal(0, 1, lt.shape), 2).astype(np.float32)
        tokens = rng.integers(0, V, (B, k)).astype(np.int32)
        tokens[:, 0] = ld[:, 0].argmax(-1)
        seed, offset = 1000 + idx, 3 * idx
        case = dict(kind=kind, B=B, k=k, V=V, temperature=temps, seed=seed, offset=offset,
                    draft=ld.tolist(), target=lt.tolist(), tokens=tokens.tolist())
        if kind == "single":
            r = verify.spec_verify_single(ld, lt, tokens, np.array(temps), seed, offset)
            case["expect"] = dict(accept_len=r["accept_len"].tolist(),
                                  out_tokens=r["out_tokens"].tolist())
        else:
            case["final"] = lf.tolist()
            r = verify.spec_verify_hier(ld, lt, lf, tokens, np.array(temps), seed, offset, 4)
            case["expect"] = dict(accept_len_inter=r["accept_len_inter"].tolist(),
                                  accept_len_final=r["accept_len_final"].tolist(),
                                  out_tokens=r["out_tokens"].tolist())
        cases.append(case)
    return cases


def philox_blocks():
    rows = []
    for (j, b, s, off, seed) in [(0, 0, 0, 0, 0), (1, 0, 0, 0, 0), (7, 255, 1, 49, 0),
                                 (63, 65535, 0, 999, 0xDEADBEEF12345678), (3, 17, 1, 2**31, 42)]:
        w = philox.block_words(np.uint64(j), b, s, off, seed)
        rows.append(dict(counter=[j, b, s, off], seed=seed,
                         words=[int(np.asarray(x)) for x in w]))
    return rows


def lmhead_cases():
    """Small LM-head verify cases: hidden states and head as bf16 bit patterns."""
    rng = np.random.default_rng(20251002)
    cases = []
    for idx, (B, k, d, V) in enumerate([(3, 4, 32, 41), (2, 2, 48, 29)]):
        def bits(x):
            return (np.asarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)
        hd = bits(rng.normal(0, 1, (B, k, d)))
        ht = bits(rng.normal(0, 1, (B, k + 1, d)))
        w = bits(rng.normal(0, 0.3, (V, d)))
        tokens = rng.integers(0, V, (B, k)).astype(np.int32)
        temps = [1.0, 0.0, 0.8][:B]
        seed, offset = 77 + idx, idx
        r = lmhead.spec_verify_lmhead_single(hd, ht, w, tokens, np.array(temps), seed, offset)
        cases.append(dict(B=B, k=k, d=d, V=V, temperature=temps, seed=seed, offset=offset,
                          h_draft=hd.tolist(), h_target=ht.tolist(), w=w.tolist(),
                          tokens=tokens.tolist(),
                          expect=dict(accept_len=r["accept_len"].tolist(),
                                      out_tokens=r["out_tokens"].tolist())))
    return cases


if __name__ == "__main__":
    with open(os.path.join(HERE, "oracle_lmhead_cases.json"), "w") as f:
        json.dump(lmhead_cases(), f)
    with open(os.path.join(HERE, "oracle_small_cases.json"), "w") as f:
        json.dump(small_cases(), f)
    with open(os.path.join(HERE, "oracle_philox_blocks.json"), "w") as f:
        json.dump(philox_blocks(), f, indent=1)
    print("written")
