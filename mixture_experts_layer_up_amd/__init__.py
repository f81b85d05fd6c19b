"""MI355X-native bf16 routed MoE-LoRA layer.

The compute path is the HIP library ``libmoe_lora.so`` (C ABI declared in
``include/moe_lora.h``); :mod:`.binding` marshals torch tensors into it.
Submodules are imported lazily so that the input generator can be used on a
machine without a GPU.
"""

__all__ = ["binding", "synth", "build"]
