"""Plain, slow, CPU reference ("oracle") for batched lossless token verification.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call, link or
execute this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, headers, tables
or helpers with the HIP library under ``lossless_token_verification_amd/``, and
it imports nothing from there (nor from the input generators).

Everything is NumPy float64 (or exact ``fractions.Fraction`` object arrays where
a test wants the exact law), one sequence at a time, in the order the method is
described:

* the pages: "Technische Zusammenfassung: HiSpec: Hierarchische spekulatives
  Decodieren fuer LLMs" (gist.science, paper 2510.01336), section 2 "Methodik:
  HiSpec" -- "Kernmechanismus" (exits L_d, L_i, L_f) and "Wichtige technische
  Innovationen" (bullets "Verlustfreie Garantie", "Dynamische
  Verifizierungsrichtlinie", "Wiederverwendung von KV-Cache ...",
  "Unterstuetzung fuer Batch-Inferenz");
* "Speculative Speculative Decoding" (gist.science, paper 2603.03251),
  Technische Zusammenfassung section 2 item 1 (bonus token) and section 3.B
  (residual distribution proportional to target minus draft);
* the acceptance rule itself, which the pages invoke ("lossless speculative
  decoding proof") but never write out, is the standard speculative-sampling
  rule (Leviathan, Kalman, Matias 2023; Chen et al. 2023): accept x with
  probability min(1, p(x)/q(x)), else resample from norm(max(0, p - q)), and
  draw a bonus token from p when every draft is accepted.

Modules
-------
philox     Philox4x32-10 (and the 4x64 instantiation used to pin the round
           structure), from Salmon, Moraes, Dror, Shaw, SC'11.
numerics   bf16/fp32 decode and the per-row target/draft distributions.
rule       the accept test, the inverse-CDF draw, one verification chain.
verify     batched single-stage and hierarchical (L_d -> L_i -> L_f) verify.
blocktable paged-KV block-table / length rollback.
lmhead     logits of a linear LM head (hidden . W^T, float64) fed to the
           single-stage verify.
byproducts row entropies and the verification-outcome export (acceptance
           probability and largest residual tokens per tested position).
tentative  cross-call tentative buffering: intermediate rounds append to a
           per-sequence pending state, a flush verifies it against the final
           exit.

Parity status: every function here is pinned by a CPU test (tests/test_oracle_*)
except the 4x32 *constants* of Philox, which no library in the CPU container
exposes; their round structure is pinned through the 4x64 instantiation
against ``numpy.random.Philox`` and the constants are the published ones.
"""

from . import philox, numerics, rule, verify, blocktable, byproducts, tentative  # noqa: F401
