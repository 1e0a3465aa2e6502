"""Routed multi-LoRA projection on MI355X (gfx950): y = W x + s_slot * B_slot (A_slot x).

The compute path is the HIP library ``_lib/liblora_mi355x.so`` (C ABI declared
in ``include/lora_mi355x.h``); ``binding`` marshals torch tensors into it.
``workloads`` holds the seeded synthetic input generators.
"""
