"""CPU oracle of the MoE-layer forward and backward passes (numpy, fp64).

TEST INFRASTRUCTURE ONLY.  This package is imported, called or executed only by
``tests/``, by ``__graft_entry__.smoke()`` (to check the GPU result) and by the
CPU-baseline leg of ``bench.py``.  The product path (the C-ABI library and its
Python binding) never imports it and has no CPU fallback.

It shares no code with the GPU path.  It follows the pages it cites:

* "Mixture-of-Kittens: MoE Megakernel for NVL72s" (the MoK paper): §2.1 MoE
  equation, Algorithm 1 (pull-based dispatch schedule), §3.1 "Scheduling",
  §3.3 "Ring-Aware Forward Replay", §3.4 "Determinism", "MXFP8 Support" and
  "Router Weight Gradient Computation", §4.1 (benchmark protocol and FLOP
  count);
* the MoK blog post (repost titled "Cursor 开源 MoK：面向 NVL72 的 MoE 训练"),
  section "Overlapping computation and communication in MoE" (SiLU gate,
  normalised gates g_i = s_i / sum_j s_j).

Every function is pinned by ``tests/test_oracle_*.py`` to something other than
itself (brute force, closed forms, library routines, invariants).
"""

from . import backward, bf16, mx, moe  # noqa: F401
