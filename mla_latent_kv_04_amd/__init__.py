"""MI355X (gfx950) Multi-head Latent Attention over a paged latent KV cache.

The compute path is the HIP library built from csrc/ (C ABI in include/mla.h);
this package only marshals arguments to it.  Importing the package does not
require a GPU; calling an entry point requires the built library and a GPU.
"""
from ._binding import (MLAError, MLA_BF16, MLA_F32, exported_symbols, lib_path, load,  # noqa: F401
                       mla_absorb_q, mla_combine_planned, mla_decode_paged,
                       mla_decode_paged_planned, mla_kv_append, mla_out_proj, mla_plan_decode,
                       mla_rope_theta, mla_split_plan, mla_splitkv_combine, status_string)

__all__ = ["MLAError", "MLA_BF16", "MLA_F32", "exported_symbols", "lib_path", "load",
           "mla_absorb_q", "mla_combine_planned", "mla_decode_paged", "mla_decode_paged_planned",
           "mla_kv_append", "mla_out_proj", "mla_plan_decode", "mla_rope_theta", "mla_split_plan",
           "mla_splitkv_combine", "status_string"]
