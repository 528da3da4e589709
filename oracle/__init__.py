"""CPU oracle for sparse-V decode attention over a block-quantized KV cache.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import or call this
package: only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` use it. It shares no code with the HIP library (no kernels, headers,
tables or constant generators); the only module both sides use is ``synth``,
which draws the fp32 inputs and holds none of the method's arithmetic.

Sources (cited by page title and section; the pages are the only authority):

* "Пропуск 90% работы по деквантизации ускорил декодирование LLM на 22,8%"
  (tproger.ru news item on Tom Turney's *sparse V dequantization*), referred to
  below as **[SV]**. Sections used: "Решение — не ускорять, а пропускать" (the
  rule: weights come from K before V is touched; skip V dequantization and
  accumulation entirely when the attention weight is below 1e-6), "Почему это
  работает для любой квантизации" (formats q8_0, q4_0, turbo3; turbo3 uses a
  LUT codebook with a norm), "14 попыток, которые провалились" (8-entry LUT
  dequant = index extraction, sign, multiply by norm), and the FAQ (a skipped
  position contributes under a millionth of the maximum; K must be dequantized
  for every position).
* "FP8 MLA KV compression projection" (kernelindex.com), referred to as
  **[MLA]**: the 576-wide latent (kv_lora_rank 512 + qk_rope_head_dim 64),
  fp8 with BlockWise1x128 scaling, qk_nope_head_dim 128.

Modules: ``formats`` (fp64 pack/unpack of q8_0, q4_0, LUT3, FP8-B128),
``lloyd_max`` (the 8-level Lloyd-Max quantizer of N(0,1) that fills the LUT),
``attend`` (dequantize-then-attend with the skip rule, masks and statistics),
``mp`` (an mpmath brute force for tiny contexts), ``kskip`` (how many key rows
a provable score bound could leave out: the FAQ's future-work K-side skip).

Parity status: every function here is pinned by ``tests/test_oracle_*.py``
(closed forms, invariants, a library routine or a textbook table). The pages
print no worked numerical example, so no pin compares against a number taken
from them directly.
"""
