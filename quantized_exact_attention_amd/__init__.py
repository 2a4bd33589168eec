"""MI355X (gfx950) SageAttention2-style quantized exact attention forward.

INT8 QK^T on matrix cores with int32 accumulation, online softmax with FP8
(OCP E4M3FN) probabilities, FP8 PV with two-level accumulation, BF16 output.
The computation runs in the HIP library ``lib/libsage_attn.so`` (C ABI in
``include/sage_attn.h``); this package only marshals arguments.

    from quantized_exact_attention_amd import sage_quant_prep, sage_attn_fwd
    quant = sage_quant_prep(q, k, v)        # bf16 [B,H,N,D] CUDA tensors
    out = sage_attn_fwd(quant)              # bf16 [B,H,Nq,D]
"""

from .sage import (SageError, SageQuant, sage_attention, sage_attn_fwd, sage_attn_fwd_capture,
                   sage_buffer_bytes, sage_quant_prep)

__all__ = ["SageError", "SageQuant", "sage_attention", "sage_attn_fwd", "sage_attn_fwd_capture",
           "sage_buffer_bytes", "sage_quant_prep"]
