"""Ring-attention share on AMD MI355X (gfx950).

`ra` is the binding of the C ABI in include/ra.h (libra.so, built by
`python -m long_context_exact_ra_amd.build`); `synth` draws seeded inputs.
The binding loads the library on first use and raises if it is missing.
"""
from . import ra, synth  # noqa: F401
from .ra import (RaError, causal_pairs, causal_share_backward,  # noqa: F401
                 causal_share_forward, finalize, fp8_tiles, quantize_fp8,
                 share_forward_fp8,
                 kv_head, ring_block, ring_schedule, share_backward, share_forward,
                 state_init, step)
