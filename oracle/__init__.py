"""CPU oracle for the W8A8_DYNAMIC path. TEST INFRASTRUCTURE ONLY.

This package is a plain, slow, obviously correct NumPy restatement of what the
W8A8_DYNAMIC linear and MoE paths compute. Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may import
or call it. The HIP library never uses it, and it shares no code, constants or
helpers with the HIP library.

Sources (web pages, cited by title and section):
  * "DeepSeek-V4 W8A8 执行链从量化权重到 Ascend INT8 算子": §一 (the per-token /
    per-channel symmetric INT8 recipe), §二 (dense path: dynamic quant, INT8
    matmul, BF16 output), §三 (MoE path: group_list, W13 -> SwiGLU -> requant ->
    W2).
  * "Qwen3.8-FP8 on Ascend 950: Why Weights Become MXFP8 at Load Time": Deep Dive
    1-5 (block-FP8 resolve, MX re-quantization, runtime MX matmul).
  * [MXFP8] Deep Dive 6 for the MoE form of the MX variant (``oracle/mx_moe_ref.py``).
  * "超大 MoE 的低比特推理：INT4、FP4 与量化感知训练" for the W4A16 weight variant
    (``oracle/w4a16_ref.py``).
  * [DSV4] again for the static W8A8 scheme (``oracle/static_ref.py``) and for
    the INT8 dispatch and combine around the MoE chain (``oracle/moe_io_ref.py``).

Parity status per function is listed in ``oracle/w8a8_ref.py``'s header.
"""

from . import mx_ref as mx  # noqa: F401
from . import static_ref as static  # noqa: F401
from . import moe_io_ref as moe_io  # noqa: F401
from . import mx_moe_ref as mx_moe  # noqa: F401
from . import w4a16_ref as w4a16  # noqa: F401
from .w8a8_ref import *  # noqa: F401,F403
from .w8a8_ref import __all__  # noqa: F401
