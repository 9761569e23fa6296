"""Seeded synthetic inputs shared by the oracle tests, the GPU tests and the
benchmark.  Holds no arithmetic of the verify step itself."""

from .synth import (BF16, CONFIG_ORDER, CONFIGS, F32, Config, Workload,
                    batch_temperatures, f32_to_bf16_bits, make_workload,
                    uniforms)

__all__ = ["BF16", "CONFIG_ORDER", "CONFIGS", "F32", "Config", "Workload",
           "batch_temperatures", "f32_to_bf16_bits", "make_workload",
           "uniforms"]
