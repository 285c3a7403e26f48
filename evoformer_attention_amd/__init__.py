"""MI355X (gfx950) biased, gated attention for the Evoformer: a C-ABI HIP
library (libevoattn.so) and a thin torch-tensor binding over it.

Importing the package loads nothing; the library is loaded on first use by
evoformer_attention_amd.ops, which raises if it is missing."""
__all__ = ["ops", "synth", "metrics"]
