"""kvfix: cross-context KV-cache correction on AMD MI355X (gfx950).

The product is the C-ABI library libkvfix.so (include/kvfix.h) built from
csrc/ by cross_context_kv_amd.build; `kvfix` is its thin Python binding.
Calls raise ImportError when the library has not been built: there is no
CPU fallback.
"""
from . import kvfix  # noqa: F401
from .kvfix import (  # noqa: F401
    Diff,
    KvfixError,
    Plane,
    kvfix_apply,
    kvfix_diff_decode,
    kvfix_diff_decode_workspace,
    kvfix_diff_encode,
    kvfix_diff_encode_workspace,
    kvfix_fit_mean,
    kvfix_fit_mean_workspace,
    kvfix_rope_shift,
    kvfix_score,
    kvfix_score_draft,
    kvfix_score_draft_workspace,
    kvfix_select_topb,
)

__version__ = "0.1.0"
