"""CPU oracle for the QLoRA linear layer (NF4 base weight + LoRA adapter).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in this package.
The product path (``nf4_bit_quantized_amd``) never imports it, and this package
imports nothing from the product path: the two share no code, tables or
constant generators.  The only module both sides use is ``workloads`` (seeded
synthetic inputs, which holds none of the method's arithmetic).

It is a plain, slow, obviously-correct numpy implementation of what the pages
describe, step by step and in the pages' order:

* ``oracle.nf4``  -- the 16-level tables, blockwise absmax quantization to
  4-bit indices, nibble packing, double quantization of the scales, dequant.
* ``oracle.lora`` -- the two-branch forward, the frozen-base backward, merge.
* ``oracle.bf16`` -- the oracle's own bfloat16 round-to-nearest-even.
* ``oracle.optim`` -- the AdamW update of the adapter parameters.

Page keys used in citations (titles of the pages the method is read from):

* [QLoRA-入门到精通]  "QLoRA技术从入门到精通" (bjdmk.com.cn developer community)
* [LoRA-QLoRA-工程]    "LoRA 与 QLoRA：把大模型微调拆成可负担的工程" (gwbblog.top)
* [X长文]              "【X 长文】LoRA 与 QLoRA：用一块 GPU 微调大模型" (aihot.news)
* [QLoRA-量化微调]     "7、QLoRA 量化微调" (aibook.faruheaisha.me)

Pinning status of each function is listed in its docstring; every function here
is pinned by at least one ``-m "not gpu"`` test against something other than
itself, except where the docstring says "parity unpinned".
"""

from . import bf16, lora, nf4, optim  # noqa: F401
from .nf4 import (  # noqa: F401
    nf4_levels,
    uniform_levels,
    quantize,
    dequantize,
    storage_bits_per_weight,
    Quantized,
)
from .lora import forward, backward, merged_weight  # noqa: F401
