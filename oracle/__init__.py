"""CPU oracle for causal prefill attention (BF16 and FP8 e4m3 inputs).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from this package.  The
product path (the HIP library and its Python binding) never imports, links or
runs it, and shares no code with it.

Page legend used in the citations below:

* [P1] "Zyphra ZYFA: 1.76x FP8 FlashAttention Speedup on AMD MI355X"
  (kongchang.com)
* [P2] "Zyphra Says Its AMD MI355X Attention Kernel Is 1.76x Faster"
  (fourweekmba.com)
* [P3] "Zyphra 开源 ZYFA：面向 AMD MI355X 的 FP8 FlashAttention，最高提速 1.76 倍"
  (attain.fans, a rendering of a MarkTechPost article)

Modules:

* ``attention`` -- exact causal softmax attention in fp64 (the plain
  definition that tiled online-softmax attention reproduces, [P1] "Why prefill
  attention deserves dedicated optimization"; the pages' own accuracy yardstick
  is fp64 attention, [P3] "ZYFA 的 FP8 注意力有多准确？"), also for a chunk of
  queries after a key prefix, with the log-sum-exp of each row.
* ``e4m3`` -- the OCP FP8 e4m3fn code: decode and round-to-nearest-even
  saturating encode ([P1] "ZYFA's performance and accuracy data" describes the
  format; [P3] "ZYFA 如何工作？" uses its integer ordering).
* ``hadamard`` -- the Sylvester Hadamard rotation of Q and K along the head
  dimension (one H_128 at d = 128, three H_64 blocks at d = 192) ([P3] "ZYFA 的
  FP8 注意力有多准确？", [P2] "Accuracy and Code").
* ``quantize`` -- per-(batch, head) amax/448 FP8 quantization, and per-64-position
  block quantization with power-of-two scales ([P1] "ZYFA's performance and
  accuracy data" names scaling granularity).

Every function is pinned by a ``-m "not gpu"`` test against something other than
itself (library routines, closed forms, invariants, brute force).
"""

from .attention import attn_chunk_ref_rows, attn_ref, attn_ref_rows, causal_weights_ref  # noqa: F401
from .e4m3 import e4m3_decode, e4m3_encode_rne_sat  # noqa: F401
from .hadamard import (  # noqa: F401
    fwht128_f32,
    fwht_f32,
    hadamard_norm_f32,
    hadamard_rotate_f32,
    sylvester_hadamard,
)
from .quantize import (  # noqa: F401
    block_exponent,
    dequantize_block64_ref,
    dequantize_ref,
    quantize_block64_ref,
    quantize_ref,
)
