"""CPU oracle for the hybrid Gated-DeltaNet + attention decoder forward pass.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call, link or
run this package: only the test suite, the package smoke check and the
benchmark's CPU-baseline leg use it.  It shares no code with the GPU library; the
only common module is ``workloads`` (seeded shapes and random draws).

The oracle is a plain, single-threaded, float64 forward pass written token by
token from the definitions (``ops``), plus a whole-model driver (``model``).  It
follows the launch page "OS Megakernel that match M5 Max Tok/w at 2x the
Throughput on RTX 3090" (sections "Why nobody had done this yet?" for the layer
mix and "We wrote a single CUDA kernel ..." for BF16 weights with FP32
accumulation and the fused attention) for what the path computes.  Where the
pages are silent the readings used are written next to each function.
"""
from .ops import *  # noqa: F401,F403
from .model import OracleModel, Contract, EXACT, C1, C2  # noqa: F401
