"""N:M activation pruning fused with its linear layer, for MI355X (gfx950).

The compute runs in ``libspa.so`` (hand-written HIP kernels behind a C ABI,
declared in ``include/spa.h``); this package is its thin Python binding.
"""
from ._binding import (  # noqa: F401
    EXPORTS,
    EtaCalibration,
    Fp8Weight,
    PreparedCall,
    PreparedWeight,
    PruneConfig,
    SpaError,
    decode_meta,
    encode_meta,
    eta_lookup,
    lib,
    meta_row_bytes,
    prepare_amber,
    prepare_weight,
    prefill_layout,
    prepare_weight_fp8,
    prune_nm,
    sparse_linear_decode,
    sparse_linear_decode_static,
    sparse_linear_prefill,
    sparse_linear_prefill_fp8,
    sparse_ffn_relu2_prefill,
    workspace,
    workspace_bytes,
)
