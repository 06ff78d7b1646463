"""CPU oracle for the LowRAM decode path — TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the CPU-baseline leg of the benchmark
may import this package.  The product path (the HIP library and its Python
binding) never imports it, and it imports nothing from the product.

Method: "LowRAM: Low-Rank Keys and Amortised Values for Composable KV Cache
Compression at Test-Time" (arXiv:2611.07025).  Every function cites the page
and section whose statement it follows.
"""
from .lowram_oracle import *  # noqa: F401,F403
