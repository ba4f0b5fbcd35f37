"""Oracle for the MiniMax-H3 DiT denoiser hot path -- TEST INFRASTRUCTURE ONLY.

A plain, slow, float64 CPU statement of what the denoiser computes, written from the
public pages that describe the h3.c / h3-metal engine.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may import or
call anything in this package.  It shares no code with the HIP path and imports nothing
from it: every input arrives as a NumPy array handed over by the caller.

Citation keys used in the docstrings of this package:

  P1  news.ditty.ir, "h3: native MiniMax-H3 on Apple Silicon" (Persian news summary):
      introduction and key-points list.
  P2  aihot.vn, "H3-metal: running MiniMax-H3 directly on Apple Silicon" (Vietnamese
      tutorial): sections 1-5 of the tutorial ("§2 first fast video", "§4 presets",
      "§5 resolution and duration").
  P3  dothoosh.com, "How h3.c cuts MiniMax-H3 video inference to 3.5 seconds on M5"
      (Persian article): sections "speed architecture", "DiT fusions and memory",
      "aggressive levers", "the int8 path", "memory and resolution limits",
      "temporal shapes and prompting".
  P4  wqu.guru, "h3-metal: native MiniMax-H3 inference for Apple Silicon" (Chinese README
      translation): tutorial sections 1-4 and the speed/quality preset table.
  P5  iitog.ru, "H3-metal: native inference of the MiniMax-H3 video model on Apple
      Silicon" (Russian summary): measurements and key facts.

The pages print no equations for the transformer block.  Where they are silent the
oracle takes one plain reading and says so in the docstring ("Reading: ...").
Functions without an independent pin say "parity unpinned" in their docstring.

Modules:
  host  -- integer host logic: frame alignment, token grid, sigma schedule, fresh
           evaluations, layer thinning, token-pair plan (all exact).
  dit   -- float64 arithmetic of one fresh evaluation and of the Euler loop.
"""
