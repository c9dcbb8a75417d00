"""MI355X (gfx950) Mamba-2 mixer core: causal conv1d + SiLU, chunked SSD scan,
grouped gated RMSNorm and single-token decode, as hand-written HIP kernels
behind a C ABI (include/ssd_mi355x.h). ``ops`` holds the thin torch binding.
"""
__all__ = ["ops", "synth"]
