"""Plain, slow CPU oracle of the QLoRA NF4 quantized-linear path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run anything in this package.
The product path (the HIP library and its Python binding) never imports it, and
it imports nothing from the product path: the two share no code, no tables and
no constant generators.  Inputs reach both sides from ``synth.py``.

Modules
-------
nf4     -- the NF4 codebook, blockwise absmax NF4 encoding with double
           quantization of the block scales, dequantization, storage sizes.
linear  -- the LoRA-augmented linear layer forward and backward in float64.
affine  -- the affine (scale + zero-point) integer quantizer of the worked
           INT8 example; used only as a pinned unit.
merge   -- folding the trained adapter into the base weight (binary32 rank-order
           sum, bf16 rounding) before requantization.
formats -- the alternate block formats of the base weight: asymmetric 4-bit
           min/max blocks of 64 (fp32 scale and zero-point) and Q8_0 blocks of
           32 (int8 values, fp16 scale), with their storage order.

Pages cited (by address and section):
  [kwkr]  kwkr.cn/news/627310            (quantized vs. non-quantized)
  [rkmt]  news.rkmt.cn/news/4821         (QLoRA double / block-wise quantization)
  [zky]   zky001.github.io/llm-training-guide/docs/post-training/qlora
          (section 5.8, "QLoRA: 4-bit base + 16-bit sticky notes")
  [lqnn]  www.lqnn.cn/news/228537        (course notes: quantization + LoRA)
  [cf1]   www.cf-1.com/news/5705389      (LoRA training on a quantized base)
"""
