"""Plain fp64 CPU oracle for the tensor-parallel transformer-shard path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product package imports, calls or
links this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may use it.  It shares no code with the
HIP library; the two meet only through the seeded input generators in
``synth/``, which hold none of the method's arithmetic.

Every function is the plain definition from the pages, written out in fp64
with numpy (and ``scipy.special.erf`` for GELU).  Page names used in the
citations:

* "5-megatron" -- formulaic.cloudchewie.com, docs/large-language-models/
  distributed-training/5-megatron (Megatron walkthrough with code).
* "Megtron张量/模型并行" -- amentiraz.github.io (tensor-parallel theory:
  row/column splits, MLP, attention by heads, embedding, cross entropy).
* "notion 310f8c09" -- www.baty7811.com/blog/notion-310f8c09... (PP/DP/TP
  notes, tensor-parallel recap).
* "zwxr 246059" -- www.zwxr.cn/news/246059 (Megatron's gradient
  synchronisation across parallel modes; its section 4.3 sums the LayerNorm
  gradients of sequence-parallel regions over the tensor-parallel group).

Parity status of each function is listed in ``PINS`` below; a function with
no independent pin says "parity unpinned".
"""

from .tp_oracle import *  # noqa: F401,F403
from .tp_oracle import PINS  # noqa: F401
