"""MI355X-native exact long-sequence attention forward (gfx950 HIP kernels behind a C ABI).

The HIP library is loaded on first use by ``exact_long_sequence_amd.attnio``; calls
raise if it has not been built.  ``exact_long_sequence_amd.inputs`` holds the seeded
synthetic input generators and touches no GPU code.
"""

__all__ = ["attnio", "inputs"]
