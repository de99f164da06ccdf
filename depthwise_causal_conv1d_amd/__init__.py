"""libsconv: paged depthwise causal short convolution for AMD MI355X (gfx950).

The compute lives in hand-written HIP kernels behind a C ABI
(``include/sconv.h``, built into ``libsconv.so``); this package is the thin
torch binding over it.  The library is loaded on first use (or by
``load()``); every op fails loudly, with ImportError, if it has not been
built.  Importing the package itself never touches the library, so its
build module runs even where an older library lies next to it.
"""
from ._lib import LibsconvError, load
from .ops import (
    causal_conv1d_update,
    causal_conv1d_update_tokens,
    causal_conv1d_varlen_fwd,
    gather_intermediate_conv_window,
    gather_intermediate_ssm_state,
    sconv_fused_insert_conv,
    sconv_fused_insert_conv_gather,
    sconv_fused_insert_conv_qsl,
    sconv_fused_insert_conv_streams,
    sconv_fused_plan,
    sconv_init,
    sconv_seq_metadata,
)


__all__ = [
    "LibsconvError",
    "causal_conv1d_update",
    "causal_conv1d_update_tokens",
    "causal_conv1d_varlen_fwd",
    "gather_intermediate_conv_window",
    "gather_intermediate_ssm_state",
    "sconv_fused_insert_conv",
    "sconv_fused_insert_conv_gather",
    "sconv_fused_insert_conv_qsl",
    "sconv_fused_insert_conv_streams",
    "sconv_fused_plan",
    "sconv_init",
    "sconv_seq_metadata",
]
