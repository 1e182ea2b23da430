"""Plain, slow, obviously-correct CPU oracle for the DeepSeek-V4 CSA/HCA attention forward.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call, link or
execute anything under ``oracle/``: only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library (no kernels, headers, tables, constants or pre/post-processing); it reads
NumPy arrays and returns NumPy arrays.

Arithmetic is float64 throughout, except where the method fixes a decision in a
narrower precision (rounding to bf16 / fp8 / fp4 storage, and the fp32 scale
computations of the quantizers), which is done exactly as the storage format
defines it.

Sources (cited by page title and section; the pages are web copies of the
DeepSeek-V4 technical report and notes on it):

* [V4-CN]  "DeepSeek-V4中文翻译（翻译模型：Opus4.7）", blog.uika.cn -- a Chinese
  translation of the report.  The authority for the definitions: §2.3.1 (CSA
  compression equations, lightning indexer score, shared-KV MQA), §2.3.2 (HCA
  compression), §2.3.3 (partial RoPE + inverse RoPE, sliding window, attention
  sink), §2.3.4 (mixed FP8/BF16 KV storage, FP4 indexer), §3.4 (MXFP4 QK path).
* [NOTES]  "DeepSeek-V4：把百万 token 上下文从额度变成架构问题",
  awesome.papernotes.org -- "关键设计 1" (CSA equations, per-dimension weights,
  the csa() sketch) and "关键设计 2" (HCA equation, the hca() sketch), and the
  visible-set model N_CSA / N_HCA.
* [SUMMARY] "DeepSeek-V4: 突破百万 token 上下文效率瓶颈的开源大模型",
  liyaozong1991.github.io -- §2.2.1-§2.2.4.

Parity status of every function is listed in ``oracle/csa_oracle.py`` and
``oracle/quant.py`` headers; all are pinned by ``tests/test_oracle_*.py``.
"""

from . import quant  # noqa: F401
from . import csa_oracle  # noqa: F401
