"""Seeded synthetic inputs shared by the CPU oracle and the HIP path.

This package holds no arithmetic of the attention method itself: it only draws
random video-latent Q/K/V tensors, audio-to-video norm maps and upstream
gradients with the structure the Prism pages describe (static background,
directional content variation, compact sounding regions), and rounds them to
bfloat16.
"""

from .generator import (CONFIGS, Workload, WorkloadConfig, a2v_output, bf16_bits_to_f32, bf16_round,  # noqa: F401
                        generate)
