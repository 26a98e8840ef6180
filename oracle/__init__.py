"""fp64 CPU oracle for the quantized, paged GQA decode-attention path.

TEST INFRASTRUCTURE ONLY. Nothing in the product package imports, links or
runs this package. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may use it. It shares no code, table or
constant generator with the HIP library; the two meet only through the seeded
inputs of ``kvsynth`` and through bytes compared in the tests.

Sources (the web pages this method is described on):

* Strata page: the hotelren.com article "KV 沉进内存、显存减半：Strata 让
  12 GB 显卡跑满 262K 上下文". Sections used: "KV 从显存搬进内存之后发生了什么"
  (pinned-host KV, residency table, CLOCK, zero-copy page-in, bitwise-equal
  results), "4-bit KV 缓存：先旋转，再压到 4-bit" (256-point Walsh-Hadamard
  rotation of Q, K and V; q4_0 blocks; output restored by H), "三种 KV 格式横向
  对比" (int8 / q4_0 / k8v4 and their byte sizes).
* VRAM wiki page: the anozoder.com wiki page "qwen38-27b-quant-vram-2026"
  (Qwen3.8-27B quantization and VRAM). Sections "一、为什么 256K 上下文的显存
  这么吓人" (KV-size formula; 24 Q heads / 4 KV heads / head_dim 256; 16
  full-attention layers) and "二、核心组合表" (KV at 256K: 17.2 / 9.1 / 4.8 GB).
* KV-offload news page: the rebasdaily.com topic page on Qwen3.8-Flash-Next KV
  offload, section "缓存为何不能直接搬走？" (every decoded token re-reads the
  whole KV of each full-attention layer; 2,048 B per token per layer).

Modules:

* ``hadamard``   - the normalized 256-point Walsh-Hadamard matrix and the
                   exact rotation.
* ``records``    - fp16 rounding, the int8 and q4_0 vector records.
* ``layout``     - the paged pool byte layout (packer and unpacker).
* ``attention``  - fp64 GQA decode attention on dequantized values.
* ``residency``  - the CLOCK (second-chance) residency table.
* ``accounting`` - byte accounting of the formats and the KV-size formula.

Parity status: every function here is pinned by tests in
``tests/test_oracle_pins.py`` and ``tests/test_oracle_residency.py``. The
exact constant convention of q4_0 (signed maximum mapped to -8, offset 8,
round half up) is a reading: the pages print no worked example of a q4_0
block, so only the invariants and the byte size pin it (see ``records``).
"""

from . import accounting, attention, hadamard, layout, records, residency  # noqa: F401
from .records import FMT_INT8, FMT_Q4_0, FMT_K8V4, FORMATS  # noqa: F401
