"""Seeded synthetic inputs (no method arithmetic) shared by the oracle and the HIP path."""
from .gen import (  # noqa: F401
    BF16, FP8, Workload, Inputs, workload, seed_of, make_inputs, decode_picks, rng,
    to_bf16_bits, to_e4m3fn_bits,
)
