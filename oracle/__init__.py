"""Plain CPU oracle for the TurboQuant KV-cache hot path.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
execute anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it, to check and to time the
HIP library. It shares no code with the library and imports nothing from it.

What it computes, in the order the pages describe it:

* ``config``     -- the ``TurboQuantConfig`` arithmetic (presets, slot sizes).
* ``rotation``   -- per-layer seeded random signs and the Walsh-Hadamard
                    rotation that precedes scalar quantization of keys.
* ``lloyd_max``  -- the Lloyd-Max centroid table for rotated coordinates.
* ``codec``      -- key / value encode into ``[key_packed | value_packed]``
                    slots, the paged pool addressing, and dequantization.
* ``attention``  -- decode attention over the dequantized cache plus the exact
                    ring buffer, by its plain definition in float64, and the
                    rotated-query form used by the fused kernel.

Sources (cited by page title and section throughout):

* vLLM API page "vllm.model_executor.layers.quantization.turboquant"
  (the ``TurboQuantConfig`` dataclass, its docstring and properties).
* prhub summary of vLLM PR #39931, "TurboQuant supports hybrid models and
  fixes page-size alignment" (the page-size snippet from ``interface.py``).
* hnwysp.cn article on the stand-alone ``turboquant`` project's full_tq
  zero-allocation mode (sections on the write path and on the fused
  decode kernel).

Parity status per function is listed in each module header. Every function
here is pinned by a test in ``tests/test_oracle_*.py`` against something other
than itself (printed values, textbook tables, library routines, closed forms,
brute force); none is "parity unpinned" except where a module header says so.
"""

from . import config, rotation, lloyd_max, codec, attention  # noqa: F401
