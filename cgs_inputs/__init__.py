"""Seeded synthetic inputs shaped like the rMuscle workloads.

This module is shared by the CPU oracle's tests and by the HIP path's tests and
benchmark.  It draws random numbers and encodes them as bf16 bit patterns; it
holds none of the selective-FFN arithmetic (no scores, no FFN, no masks, no
normalisation).  Every array is produced on the host with
``numpy.random.default_rng(SeedSequence([seed, layer, role]))`` so that each
side receives byte-identical inputs.

Shapes follow rMuscle (Zhou et al.), "rMuscle: Robotic Muscle Memory for
Efficient Vision-Language-Action Model Inference":
  * three camera views x 256 patches = 768 visual tokens, VLM FFN d=2048,
    ff=16384, 17 FFN layers (§4.2, asynchronous online reconstruction);
  * action expert H=4096 neurons (Fig. 9 uses top-k=2048 at rho_n=0.5),
    d=1024, 50 action tokens, 18 layers.
"""
from .gen import (  # noqa: F401
    ROLE,
    rng,
    f32_to_bf16_bits,
    ffn_weights,
    ffn_weight_pool,
    ctx_layer_inputs,
    act_tokens,
    synthetic_h_ref,
    timestep_embedding,
    random_bf16,
)
