"""MI355X-native fused causal attention kernels (Threshold Rectified Attention
forward and backward, Threshold Differential Attention forward, the NSA
selection-branch forward (query-outer and block-outer) and backward) behind a C-ABI HIP
library, ``libattn.so``.

The Python functions here only marshal arguments into the C ABI declared in
``include/attn.h``; every step of the computation runs in the HIP kernels.
The library is loaded on first use and the call raises if it is missing.
"""
from ._lib import (AttnError, attn_status_str, library_path, load_library, nsa_sel_bwd,
                   nsa_sel_bwd_workspace_bytes, nsa_sel_fsa_workspace_bytes, nsa_sel_fwd,
                   nsa_sel_fwd_fsa, tda_fwd, tda_fwd_noalloc, tda_noalloc_scratch_bytes,
                   tda_workspace_bytes,
                   tra_bwd, tra_fwd, tra_fwd_f32)

__all__ = ["AttnError", "attn_status_str", "library_path", "load_library", "nsa_sel_bwd",
           "nsa_sel_bwd_workspace_bytes", "nsa_sel_fsa_workspace_bytes", "nsa_sel_fwd",
           "nsa_sel_fwd_fsa", "tda_fwd", "tda_fwd_noalloc", "tda_noalloc_scratch_bytes",
           "tda_workspace_bytes",
           "tra_bwd", "tra_fwd", "tra_fwd_f32"]
