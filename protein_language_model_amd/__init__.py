"""MI355X-native varlen RoPE attention (forward + backward) for ESM-2-style
protein language model training.

The compute lives in a HIP/C library (libesm_attn.so, C ABI declared in
include/esm_attn.h); `protein_language_model_amd.esm_attn` is its thin Python
binding. `protein_language_model_amd.workloads` holds the seeded synthetic
inputs. Importing this package loads nothing.
"""
