"""Python binding of the MI355X segment-routed multi-adapter LoRA delta library.

Argument marshalling only: every step runs in liblora_sgmv.so (host C++ for
packing and routing, HIP kernels for shrink and expand).  There is no
fallback: if the library is not built, importing the device functions raises.

Host functions take and return numpy arrays.  Device functions take torch
tensors that live on the GPU and launch on torch's current stream (or the
stream passed in).
"""

from ._lib import (  # noqa: F401
    CACHE_LRU,
    CACHE_NO_EVICT,
    LoraSlotCache,
    lora_reset_slot,
    lora_write_slot,
    DTYPE_BF16,
    DTYPE_F32,
    FAMILY_DOWN,
    FAMILY_GATE_UP,
    FAMILY_O,
    FAMILY_QKV,
    PATH_AUTO,
    PATH_FUSED,
    PATH_MFMA,
    PATH_VALU,
    MAX_HOST_GROUPS,
    LoraDims,
    LoraOptions,
    LoraRouting,
    LoraError,
    a_tiled_shape,
    family_shape,
    library_path,
    lora_abi_version,
    lora_build_routing,
    lora_build_token_routing,
    lora_family_shape,
    lora_pack_adapter,
    lora_pack_family,
    lora_pack_bias,
    lora_sgmv_delta,
    lora_sgmv_delta_noalloc,
    lora_sgmv_noalloc_scratch_bytes,
    lora_sgmv_expand,
    lora_sgmv_shrink,
    lora_sgmv_workspace_bytes,
    lora_status_string,
    packed_to_torch,
    tile_a,
    untile_a,
)
