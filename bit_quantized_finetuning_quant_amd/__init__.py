"""QLoRA linear layer for MI355X (gfx950): NF4 storage with FP8 double quantization,
BF16 dequantization fused into MFMA matrix products, LoRA adapters, and the backward
pass into the adapters.  The compute lives in a C-ABI HIP library
(``libqlora_gfx950.so``); ``qlora`` is its thin ctypes binding."""
