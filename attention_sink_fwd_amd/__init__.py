"""Sink attention (causal GQA with one learnable sink logit per query head)
for AMD Instinct MI355X: HIP kernels behind a C ABI (libsinkattn.so), with a
thin torch binding.  See include/sink_attn.h for the contract."""
from .binding import (  # noqa: F401
    make_params,
    sink_attention,
    sink_attn_bwd,
    sink_attn_bwd_fused,
    sink_attn_bwd_noalloc,
    sink_attn_bwd_workspace_size,
    sink_attn_fwd,
    sink_attn_fwd_paged,
    token_logps,
    token_logps_bwd,
    token_logps_fwd,
)
from ._lib import LIB_PATH, SinkAttnError, load  # noqa: F401
