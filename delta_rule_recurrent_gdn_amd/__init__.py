"""Gated Delta Rule-2 (GDN-2) operator for AMD Instinct MI355X (gfx950).

The computation lives in hand-written HIP kernels behind the C ABI of
include/gdn2.h (libgdn2.so, built in-tree by ``delta_rule_recurrent_gdn_amd.build``).
This package only marshals torch tensors and streams into that ABI.
"""

from .ops import gdn2_bwd_chunked, gdn2_decode_step, gdn2_fwd_chunked, gdn2_workspace_bytes  # noqa: F401
from .ops import gdn2_fwd_chunked_noalloc  # noqa: F401
from .ops import (gdn2_bwd_varlen, gdn2_decode_step_slots, gdn2_fwd_varlen,  # noqa: F401
                  gdn2_varlen_max_chunks)
from .ops import gdn2_bwd_chunked_records, gdn2_fwd_chunked_train, gdn2_records_bytes  # noqa: F401
from .ops import gdn2_bwd_varlen_records, gdn2_fwd_varlen_train, gdn2_varlen_records_bytes  # noqa: F401

__all__ = ["gdn2_fwd_chunked", "gdn2_decode_step", "gdn2_bwd_chunked", "gdn2_workspace_bytes", "gdn2_fwd_varlen",
           "gdn2_bwd_varlen", "gdn2_decode_step_slots", "gdn2_varlen_max_chunks",
           "gdn2_fwd_chunked_train", "gdn2_bwd_chunked_records", "gdn2_records_bytes",
           "gdn2_fwd_varlen_train", "gdn2_bwd_varlen_records", "gdn2_varlen_records_bytes",
           "gdn2_fwd_chunked_noalloc"]
