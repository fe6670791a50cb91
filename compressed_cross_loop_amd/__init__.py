"""MI355X (gfx950) decode attention over a compressed cross-loop KV latent
cache: Looped Latent Attention (reconstruct on read; absorbed LLA-D) and
Hybrid Latent Attention (absorbed read + exact window).

The compute path is the C-ABI library liblla.so (hand-written HIP kernels);
`binding` marshals torch tensors and streams into it.
"""
from . import binding  # noqa: F401
from .binding import (  # noqa: F401
    LlaError, hla_decode_windowed, lla_abi_version, lla_bytes_per_token, lla_decode_absorbed,
    lla_decode_plan_splits, lla_decode_reconstruct, lla_decode_workspace_bytes,
    lla_status_string, lla_write_latents, lla_write_workspace_bytes)
