"""CRISP sparse prefill attention on MI355X (gfx950).

The compute path is the HIP library libcrisp.so (C ABI in include/crisp.h);
`binding` marshals torch tensors into it, `synth` draws seeded inputs.
"""
from . import synth  # noqa: F401
from .binding import (  # noqa: F401
    CrispBuffers, CrispError, crisp_abi_version, crisp_dense_attn, crisp_list_capacity, crisp_prefill, crisp_proxy,
    crisp_proxy_scratch_bytes, crisp_route, crisp_select, crisp_select_gamma, crisp_select_workspace_bytes,
    crisp_sparse_attn, make_cfg, make_dims, NF_MEAN, NF_MEDIAN, ROUTE_AUTO, ROUTE_FORCE_PE, ROUTE_FORCE_VS, ROUTE_PE,
    ROUTE_VS,
)
