"""vegas_attn on MI355X: the attention hot path of one Vegas decode iteration.

Verify attention with the two-row logit export, score aggregation, exact
top-k selection and sparse draft attention, as hand-written HIP kernels for
gfx950 behind the C-ABI in include/vegas_attn.h.  This package holds the
ctypes binding (`_binding`), device-side plumbing for running a workload
(`runner`), the seeded input generator (`synth`) and the build script
(`build`).  Submodules load lazily so that `synth` imports without the GPU
library.
"""
__all__ = ["_binding", "runner", "synth", "build"]
