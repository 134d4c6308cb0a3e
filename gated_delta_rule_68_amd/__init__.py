"""MI355X (gfx950) KDA / GDN gated delta-rule mixer: a C-ABI HIP library
(``libkda.so``, declared in include/kda.h) and its thin Python binding."""
from ._lib import (  # noqa: F401
    ARM_NAMES, EXPORTS, KDA_DTYPE_BF16, KDA_DTYPE_F32, KDA_GATE_SIGMOID, KDA_GATE_SOFTPLUS,
    KDA_MODE_AUTO, KDA_MODE_CHUNKED, KDA_MODE_SEGMENTED, gdn_decode_gated, gdn_prefill_gated, kda_decode_gated,
    kda_prefill_gated, gdn_rollback_gated, kda_rollback_gated, KDA_GATE_GIVEN, gdn_prefill_gqa,
    gdn_decode_gqa, gdn_rollback_gqa, gqa_workspace_bytes, prefill_varlen, varlen_workspace_bytes,
    KDA_MODE_SEQUENTIAL, KdaError, gdn_decode, gdn_prefill, gdn_rollback, kda_decode, kda_prefill,
    kda_rollback, lib, prefill_arm, kda_prefill_noalloc, KDA_NOALLOC_SCRATCH_BYTES, rollback_workspace_bytes, status_string, workspace_bytes,
)
