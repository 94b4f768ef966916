"""CPU oracle of the per-row MoE route (latent down projection, FP32 router,
standalone top-16). TEST INFRASTRUCTURE: only tests, the smoke entry point and
the benchmark's CPU-baseline leg may import it; the product path never does."""
from .route_oracle import (  # noqa: F401
    bf16_bits_to_f64, round_f64_to_bf16_bits, latent_exact, latent_abs_terms,
    latent_ref, two_round_latent_ref, logits_exact, logits_abs_terms, logits_ref, topk16_ref,
    topk16_sharded_ref, route_weights_ref, route_ref, route_ref_widened, route_detail_widened,
    widen_weights,
)
