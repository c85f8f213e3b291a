"""CPU oracle for KIVI / FP8 KV-cache quantization and decode attention.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or
execute this package: only the tests, the smoke check and the benchmark's
cpu_baseline leg use it. It shares no code, header, table or constant with the
HIP library; the two meet only through the seeded inputs of `synth` and
through the documented device layouts, which this package re-implements on its
own from their written definition.

Sources (web pages, cited by title and section):
  [KIVI-page]  "4.4 KV Cache 量化：KIVI 2-bit 与 FP8 KV Cache" (aiinfraguide)
  [Tutorial]   "大模型量化从0到1（十三）：KV Cache 量化" (aiot.csdn.net)
  [Interview]  "KV Cache 量化是什么？它如何降低长上下文推理显存？" (offer.aigcbaba)
  [FP8-page]   "LLM推理加速KV Cache量化压缩实战方案" (yunthe.com)

Precision: quantization statistics, scales, zero-points and codes are computed
in fp32 with each operation correctly rounded (the bit-exact contract);
attention is computed in fp64 over the fp32 dequantized values.

Modules:
  bytes_model — the byte formula and per-step byte accounting
  kivi        — KIVI group quantization, dequantization, bit packing, split
  fp8         — E4M3 value table, encoder, per-tensor scale
  attention   — fp64 single-query decode attention with GQA
  cache       — the cache state machine (prefill / append / flush / decode)
"""
from . import attention, bytes_model, cache, fp8, kivi  # noqa: F401
