"""Plain, slow, fp64 CPU oracle of the fused MoE layer.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute anything in this package: only the test suite, the smoke check and the
CPU-baseline leg of the benchmark use it.  It shares no code, tables or
helpers with the HIP implementation; the two meet only at the seeded input
generator (``workloads``), which holds none of the layer's arithmetic.

Sources.  The layer it computes is the one described on the page
"DeepSeek悄悄更新：Mega MoE、FP4 Indexer来了" (机器之心), section "Mega MoE 是什么？":
tokens are dispatched to experts, go through a first linear map, a SwiGLU
activation, a second linear map, and are combined back per token.  The gating,
routing and quantisation steps follow the "Tile Kernels" section of the page
"DeepSeek 模型更新解读 Tile Kernels 与 DeepEP V2 新特性" (youleyou): top-k
expert selection with scores, token-to-expert mapping with expand/reduce and
weight normalisation, and per-token / per-block FP8 and FP4 quantisation fused
with SwiGLU.  Where the pages are silent the readings taken are listed in the
module docstring of ``oracle.moe_oracle``.

Parity status per function is stated in each docstring; every function is
pinned by a test in ``tests/test_oracle_pins.py`` or ``tests/test_formats.py``.
"""

from . import formats, moe_oracle  # noqa: F401
