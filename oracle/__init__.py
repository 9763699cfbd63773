"""CPU oracle for the NVFP4 paged-KV hot path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
link this package: only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, tables or
constants with the HIP library and imports nothing from it.

What it computes, and where the pages define it:

* ``nvfp4``    -- the NVFP4 format (E2M1 values, an E4M3 scale per block of
  16 values, an FP32 tensor-level scale) and the page codec built on it
  ("Accelerating Long-Context and Agentic Inference with NVFP4 KV Cache",
  introduction and Figure 1; "KV Cache Compression in TensorRT LLM",
  NVFP4 Cold-Page Compression / How It Works and Figure 6).
* ``attention`` -- single-token decode attention over the exactly
  dequantized paged K/V ("Accelerating Long-Context ...", Path 3: Decode and
  NVFP4 KV Decode Attention Kernel Implementation / Figure 3).

Arithmetic is fp64 throughout; every rounding the method performs is done
once, from a value that fp64 holds exactly or provably on the right side of
every rounding boundary (see ``nvfp4`` for the argument).  Every function is
pinned by ``-m "not gpu"`` tests against values fixed by the pages or by
mathematics (exhaustive tables, exact-rational brute force, closed forms,
a library attention routine).  No function here is "parity unpinned".
"""

from . import nvfp4, attention  # noqa: F401
