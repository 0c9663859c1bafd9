"""Vocabulary-sharded LM-head cross-entropy and masked embedding for MI355X.

The compute path is libvce.so (hand-written HIP kernels for gfx950, C ABI in
include/vce.h); this package is its ctypes binding plus step sequencing.
Importing it raises ImportError when the library has not been built.
"""

from ._lib import (  # noqa: F401
    ACC_DH, ACC_DW, LIB_PATH, REDUCE_MEAN, REDUCE_SUM, VCE_BF16, VCE_F32, BadTargetError, VceError,
    lib, read_scalar, strerror,
    vce_argmax, vce_argmax_noalloc, vce_argmax_workspace_bytes, vce_bwd, vce_bwd_workspace_bytes, vce_fwd,
    vce_fwd_workspace_bytes, vce_remap, vemb_bwd,
    vemb_bwd_workspace_bytes, vemb_fwd, vngram_fwd, vss_candidates, vss_candidates_workspace_bytes,
    vss_scatter, vss_scatter_replace,
)
from .steps import (  # noqa: F401
    Workspaces, ce_step, from_bits, ngram_bwd, ot_h_step, sampled_step, tied_step,
)
