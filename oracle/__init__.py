"""Plain fp64 CPU oracle for paged-KV e4m3 decode attention.

TEST INFRASTRUCTURE ONLY. This package is the slow, obviously-correct
definition that the HIP path is checked against. Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it. The product package (``paged_kv_fp8_amd``) never imports, calls or
links anything here, and nothing here imports the product package: the two
share no code. Inputs reach both sides from the seeded generators in
``paged_kv_fp8_amd.workloads``, which hold none of the method's arithmetic.

Sources (the pages, cited by title and section):
  [T5]   "mjolnir-kernel 0.1.0 wheel: mjolnir/t5_decode.py" (PyPI diff page):
         module docstring (tensor contract, query packing, causal tail,
         split-KV plan, workspace), ``plan_split_kv``, the softmax/epilogue
         of ``decode``, ``reduction``, ``emulate_decode`` (its exact branch),
         ``quantize_q_fp8``.
  [VLLM] "vLLM PR #62633: swap-AB CuTe DSL decode attention for DeepSeek-V4.1"
         (Kernel design; Validation: fp64 reference tests).
  [MSA]  "MiniMax MSA fmha_sm100/cute README", section "Paged FP8 Decode".

Modules
  formats   OCP e4m3 and bf16 decoding (256-entry table from the definition).
  attention decode attention as the plain dequantise -> softmax(QK^T*s) -> V
            definition, GQA / causal tail / block mode / MLA latent record.
  merge     LSE merge of split partials (the split-KV combine rule).
  plan      the occupancy-pinned split-KV planner (integer algorithm).
  brute     pure-Python loop version of the attention for tiny inputs.
  sparse    decode over per-token slot lists (window + top-k) with a sink.
  producers e4m3 encoding (round to nearest even, saturating), the query
            quantisation and the paged KV-cache write (e4m3 and latent).

Pin status of each function is recorded in its docstring; every function
here is pinned by a ``-m "not gpu"`` test in ``tests/test_oracle.py`` or
``tests/test_plan_oracle.py``.
"""
