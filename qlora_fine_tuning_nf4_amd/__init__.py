"""MI355X-native QLoRA NF4 quantized-linear hot path.

Weight formats: NF4 (double-quantized or single-level scales; bf16 or fp16
compute), asymmetric uint4 and Q8_0 blocks.  The product is the C-ABI HIP
library ``libqlora_nf4.so`` (declared in
``include/qlora_nf4.h``); ``binding`` is its thin ctypes binding, with the same
entry-point names.  Build in-tree with ``python -m qlora_fine_tuning_nf4_amd.build``.
"""
from .binding import (  # noqa: F401
    FORMATS, QLORA_BF16, QLORA_F16, QLORA_F32, QLORA_FMT_NF4, QLORA_FMT_Q8_0, QLORA_FMT_U4_ASYM,
    FwdGroup, NF4Weight, QLoRAError,
    device_codebook, lib, qlora_dequantize, qlora_group_init, qlora_group_table_bytes,
    qlora_linear_bwd, qlora_linear_fwd, qlora_linear_fwd_grouped, qlora_merge, qlora_nf4_bytes,
    qlora_nf4_block_bytes, qlora_nf4_codebook, qlora_nf4_single_bytes, qlora_quantize, qlora_strerror,
    qlora_weight_bytes, qlora_workspace_bytes,
)
