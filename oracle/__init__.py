"""CPU oracle for 3D window attention (SeedVR2 NaDiT windows).

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import this package:
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` use it.  It shares no code with the HIP library: it is a plain,
slow, obviously correct restatement of what the method computes, written from
the page "Window-Aligned Sequence Parallelism (SeedVR2)" (vLLM-Omni design
notes), in Python integers, IEEE doubles and NumPy fp64.

Modules
-------
plan       window sizes, axis segments, window boxes and the integer tables
           (section "Window layouts").
permute    entry gather, exit scatter and layout-to-layout transition
           (sections "Motivation", "Window layouts", "Plan A redistribution").
attention  per-window softmax attention in fp64, and the brute-force twin that
           runs full attention under a same-window mask (section "Motivation",
           "SeedVR2 integration").
pack       several requests' plans packed into one varlen call with alignment
           tails (page "vLLM-Omni diffusion runtime", section 4.2).
sp_plan    the single-GPU tables of window-aligned sequence parallelism: LPT
           assignment and Plan A redistribution, with the exchange simulated
           on fake ranks (sections "Planner", "Plan A redistribution").
rope       window-local 3D rotary position embedding of queries and keys
           (section "Reference quirks reproduced on purpose").
text_attention
           [video window, replicated text] segments and the text stream's
           mean over windows (sections "SeedVR2 integration", "Text stream").
"""
from . import plan, permute, attention, pack, sp_plan, rope, text_attention  # noqa: F401
