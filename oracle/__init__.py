"""CPU oracle for the MoE-layer hot path: plain, slow, obviously correct.

TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import or call anything here; the product
path (the HIP library and its Python binding) never does, and shares no code
with it. The oracle is written from the operator pages:

* "MegaMoE" (gitcode mc2/mega_moe README), section "A8W8-FP quantization
  scenario" (four stages: gather + MX quantization, GMM1 + activation + MX
  requantization, GMM2, weighted combine plus shared experts) and "Activation
  function formulas" (SiLU / swiglu);
* "moe_token_permute" (CANN ops-transformer article), sections
  功能说明 (stable argsort, inverse, gather by index // topK), 返回值说明
  (output shapes, num_out_tokens rule) and 约束说明;
* "MoeInitRoutingV3" README, 计算公式 steps 1-6 (keyValueSort, inverse
  scatter, histogram, quantized gather, availableIdxNum) and 参数说明
  (active expert range, rowIdxType, expertTokensNumType).

Floating point is float64 throughout unless a step fixes another precision;
where a reading of the pages had to be chosen it is named in the function's
docstring. Every function has pins in tests/test_oracle_*.py (worked examples,
closed forms, invariants, brute force) except where its docstring says
"parity unpinned".
"""

from . import mxfp, routing, moe  # noqa: F401
