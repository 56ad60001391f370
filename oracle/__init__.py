"""CPU oracle for Level-of-Detail attention.  TEST INFRASTRUCTURE ONLY.

Only ``tests/``, the smoke check and the benchmark's CPU-baseline leg may import
this package.  The GPU library never loads it and shares no code with it.
"""
from .oracle import (Config, attend, build_all, build_library, build_stream, canonical_dot,
                     decode, dense, dense_rows, kmeans, prefill_rows, round_bf16, streams)

__all__ = ["Config", "attend", "build_all", "build_library", "build_stream", "canonical_dot",
           "decode", "dense", "dense_rows", "kmeans", "prefill_rows", "round_bf16", "streams"]
