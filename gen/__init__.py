"""Seeded synthetic workloads shared by the oracle tests and the GPU path.

Holds only random draws and array layout, none of the method's arithmetic.
"""
from .configs import (DecodeConfig, PrefillConfig, NAMED, BY_ID, TINY_DECODE, DECODE_32K,
                      DECODE_128K_TOPP, DECODE_64K_HEADSPLIT, PREFILL_64K, SMALL_DECODE_TOPK,
                      SMALL_DECODE_TOPP, SMALL_DECODE_HEADSPLIT, SMALL_TINY_RAGGED, SMALL_PREFILL,
                      DECODE_128K_PERGROUP, SMALL_DECODE_PERGROUP, PREFILL_64K_IMPORTANCE, SMALL_PREFILL_IMPORTANCE,
                      DECODE_128K_TOPP_Q4, SMALL_DECODE_TOPP_Q4)
from .synth import (make, make_decode, make_decode_index, make_prefill, f32_to_bf16_bits, bf16_bits_to_f32, as_f32,
                    rng_for, analytic_boost, solved_boost, decode_boost)

__all__ = [n for n in dir() if not n.startswith("_")]
