"""CPU oracle for the tensor-parallel transformer-layer shard (TEST INFRASTRUCTURE).

Plain, slow, float64 numpy code that defines what the HIP path must compute.
Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU-baseline
leg may import it; the product library never does, and nothing here touches
the GPU path's code.

Page citations use these short names:

* podcast page -- xiaoyuzhoufm.com episode "Megatron-LM's parallelism" (the
  Outline list and the "Key concepts" glossary);
* overview page -- zzmblog.top "Megatron: a training framework for large
  models" (sections 1-6);
* guide page -- rkmt.cn "From Transformer splitting to communication
  optimisation" (sections 1.1-4.3).

Pins (tests/test_oracle_*.py) tie every function here to something other than
itself: library routines (torch LayerNorm, SDPA, MultiheadAttention, GeLU,
cross_entropy, math.erf), brute-force loops, closed forms, invariants and
central finite differences. Parity unpinned by the pages (fixed by reading):
the exact-erf GeLU form and LayerNorm epsilon 1e-5 (the pages name neither).
"""
from .layer import *  # noqa: F401,F403
from .layer import __all__  # noqa: F401
from .step import step_reference  # noqa: F401,E402
from . import compare  # noqa: F401,E402
