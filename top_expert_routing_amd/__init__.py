"""libmoe bindings: one MoE layer's expert path on MI355X (gfx950) HIP kernels.

The calls mirror the C ABI in include/libmoe.h.  torch supplies device
memory and streams only; all computation runs in libmoe.so.  Importing this
package does not load the library; the first call does, and raises ImportError
if libmoe.so has not been built.
"""
from ._lib import MoeError, load, EXPORTS  # noqa: F401
from .api import (router, gate, gate_record, stage_to_host, permute, grouped_ffn, grouped_ffn_noalloc,  # noqa: F401
                  grouped_ffn_combine, ffn_combine_workspace_bytes,
                  NOALLOC_SCRATCH_BYTES, grouped_ffn_packed, pack_weights, grouped_ffn_fp8w, quantize_fp8_rows,
                  pack_fp8_codes, combine, stats, prob_signature, MoeLayer,
                  permute_workspace_bytes, ffn_workspace_bytes, ffn_fp8w_workspace_bytes, stats_workspace_bytes)
