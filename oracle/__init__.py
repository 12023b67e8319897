"""CPU oracle for one Medusa decoding step -- TEST INFRASTRUCTURE ONLY.

Plain, slow, obviously correct NumPy float64 code that defines what the step
computes.  Only the test suite, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it; the GPU product path never
calls it and shares no code with it.

Sources, cited by page title and section (the pages are public web text):

* [MH-heads]  "Medusa Heads" glossary (Ultralytics; Arabic and Portuguese
  editions carry the same text), section on how the heads predict later tokens,
  including its PyTorch sketch of three heads and its printed result.
* [MH-tree]   same page, section on tree attention and acceptance.
* [SD-k+1]    "Giai ma dau co: doan truoc roi kiem mot luot" (interactive
  e-book on speculative decoding), section on why a round always yields
  accepted + 1 tokens.
* [SD-E]      same e-book, section on the expected tokens per round (closed
  form and its special cases table).
* [SD-default], [SD-gamma], [SD-peak]  same e-book, sections re-reading the
  default numbers, on guessing further, and on where the peak moves.
* [SD-flags]  same e-book, section on the round-by-round table driven by an
  acceptance-flag string.

Every function below states the passage it follows.  Where the pages are silent
the reading taken is named in the docstring.

The tree-verify pass through a Llama-shaped decoder (``decoder.py``) follows
the same section: the verify pass is the base model's forward pass over all
candidates with the ancestor mask.

Parity status: every function here is pinned by a ``-m "not gpu"`` test against
something other than itself (printed values, closed forms, special cases,
brute force, or an independent implementation: the decoder against Hugging
Face transformers' Llama run causally on every branch); see
tests/test_oracle_*.py.
"""
from .medusa import *  # noqa: F401,F403
from .cost import *    # noqa: F401,F403
from .decoder import *  # noqa: F401,F403
from .generate import *  # noqa: F401,F403
from .typical import *  # noqa: F401,F403
from .specsample import *  # noqa: F401,F403
