"""CPU oracle for parallel constrained decoding (PCD) -- test infrastructure.

A plain, slow, fp64 NumPy implementation of what the device path computes.  It
exists to check the HIP library; it is not part of the product.  Only the test
suite, the smoke check and the benchmark's CPU-baseline leg may import it.  It
shares no code with the HIP path: both only read the seeded inputs of
``pcd_inputs``.

Pages cited (by title and section):
  [Scratch]   "How TypeSafe's Jev Might Work: Parallel Constrained Decoding from
              Scratch" (faritgaleev.com)
  [TechRef]   "Parallel Constrained Decoding: A Technical Reference" (shivam2003.com)
  [FirstPr]   "Parallel Constrained Decoding, From First Principles"
              (ai.thesatyajit.com)
  [README]    "Parallel Constrained Decoding" engine README (stig.sh/stephanj)

Modules:
  decoder  -- the textbook decoder (RMSNorm, rotate-half RoPE, GQA attention,
              SwiGLU) with an explicit KV context; pinned against an independent
              library implementation and against closed forms.
  plan     -- canonical per-field trie, readout nodes, branch-token layout.
  pcd      -- prefill, one batched branch pass, full-vocabulary readout,
              combine (candidate softmax, candidate mass, argmax, margin);
              from-scratch re-evaluation and brute-force greedy references.
"""
from . import decoder, plan, pcd  # noqa: F401
