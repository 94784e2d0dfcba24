"""CPU oracle for MLA attention over a latent KV cache.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, links or runs
anything under this directory; only the tests, the package smoke check and the
CPU-baseline leg of the benchmark do.  The oracle shares no code with the HIP
path: it receives plain float64/integer arrays and returns plain arrays.
"""
from .mla_oracle import *  # noqa: F401,F403
