"""Per-row MoE route on one MI355X (gfx950): latent down projection
(7168 -> 3584, BF16, one rounding), FP32 router logits over 896 experts and the
standalone top-16, as hand-written HIP kernels behind a C ABI (libroute.so).

`latent_projection_top_amd.route` is the Python binding; importing it loads the
library and fails loudly if it is not built.
"""
