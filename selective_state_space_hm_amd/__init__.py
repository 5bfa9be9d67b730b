"""MI355X (gfx950) native causal, normalized Hedgehog linear attention.

The computation runs in libhm.so (HIP kernels behind the C ABI of include/hm.h);
`hm` is its thin ctypes binding and `inputs` the seeded synthetic workloads.
"""
from .hm import (hm_featurize, hm_linattn_fwd, hm_linattn_fwd_plan,  # noqa: F401
                 hm_linattn_step, state_numel)
