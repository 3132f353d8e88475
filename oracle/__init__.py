"""CPU oracle for the SVDQuant W4A4 + low-rank linear layer and the INT8 KV-cache quantizer.

TEST INFRASTRUCTURE ONLY. This package is a plain, slow, obviously-correct NumPy statement of
what the GPU path must compute. Only the tests, the smoke check and the benchmark's CPU
baseline may import it; the product library never does, and it shares no code with the HIP
kernels (the only module both sides use is ``synthetic``, which draws random inputs).

Arithmetic: fp64 everywhere, except where the method fixes a rounding (fp32 smoothing and
quotients, fp16 scales, bf16 low-rank factors), which is emulated exactly with NumPy's IEEE
float32 / float16 types and an explicit bf16 rounding.

Sources (web pages; cited below by the short name on the left):
  VARC  "VAR-Compressor：在边缘GPU上实现80亿参数视觉自回归模型的高效量化部署" (zingnex.cn forum)
  FLUX4 "AI图像生成4-bit量化技术解析与应用" (intelliparadigm.com)
  W4A8  "W4A8量化技术在边缘计算中的实践与优化" (mhpn.cn)
  SVDQ  "SVDQuant是什么？一文让你看懂SVDQuant的技术原理、主要功能、应用场景" (zhuoshang.net)
  DCMP  "DeepCompressor：MIT 团队开源的大模型与 Diffusion 模型压缩工具箱" (pomoai.com)

Parity pins: every function here is pinned by tests in ``tests/test_oracle_*.py`` against
closed forms, brute force, library routines or invariants; none is "parity unpinned".
"""
from . import kv_int8, numerics, svdquant  # noqa: F401
