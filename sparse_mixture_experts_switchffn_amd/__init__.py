"""SwitchFFN forward pass for one MI355X (gfx950): hand-written HIP behind a C-ABI.

The layer -- fp32 router with top-1 routing, capacity-limited in-order
dispatch, grouped expert FFNs on the matrix cores, gate-scaled combine on the
residual path and the load-balancing aux loss -- lives in libswitchffn.so
(include/switch_ffn.h).  This package is its thin Python binding.
"""
from .binding import (  # noqa: F401
    SFFN_BF16,
    SFFN_EDTYPE,
    SFFN_EHIP,
    SFFN_ESCRATCH,
    SFFN_EINVAL,
    SFFN_EUNSUPPORTED,
    SFFN_EWORKSPACE,
    SFFN_FP32,
    SFFN_NO_RESIDUAL,
    SFFN_REROUTE_OVERFLOW,
    SFFN_GEGLU,
    SFFN_OK,
    LIB_PATH,
    header_functions,
    lib,
    switch_ffn_backward,
    switch_ffn_backward_num_stages,
    switch_ffn_backward_stage_name,
    switch_ffn_backward_workspace_bytes,
    switch_ffn_capacity,
    switch_ffn_forward,
    switch_ffn_forward_ex,
    switch_ffn_forward_noalloc,
    switch_ffn_forward_topk,
    switch_ffn_noalloc_scratch_bytes,
    switch_ffn_num_stages,
    switch_ffn_stage_name,
    switch_ffn_status_string,
    switch_ffn_workspace_bytes,
    switch_ffn_workspace_bytes_topk,
)
