"""fp64 CPU oracle and integer cache model: TEST INFRASTRUCTURE.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg import
this package.  It shares no code with block_diffusion_draft_fc_amd/ and imports
nothing from it; the product path never reaches it.
"""
from . import cache_model, dflash_oracle  # noqa: F401
