"""Seeded synthetic inputs shared by the oracle-side tests, the GPU tests and the
benchmark.  This package draws random numbers and rounds them to the storage
dtype; it holds none of the TT / TTM arithmetic."""

from .workloads import (  # noqa: F401
    BASE_SEED,
    LayerSpec,
    TTMSpec,
    bf16_bits,
    fp8_bits,
    fp8_decode,
    bf16_round,
    config_layers,
    make_tt_layer,
    make_ttm,
    CONFIG_TOKENS,
    CONFIG_ZERO_FRAC,
    CONFIG_DTYPE,
    make_link_diagonals,
    zipf_ids,
)
