"""CPU oracle of the Beam routed-MoE block — TEST INFRASTRUCTURE ONLY.

Plain, slow, float64 numpy code that computes what the block computes, written from the pages
that describe the method. Only the tests, the smoke check and the benchmark's CPU-baseline leg
may import it; the GPU library never calls it, and it shares no code with the HIP path (the two
meet only in the seeded input generator, `synthgen`, which holds none of the method's arithmetic).

Sources, cited by tag and section throughout:
  [S]  "SGLang 原生支持 Reflection 的 Beam 并驱动其生产 API" (SGLang day-0 post for Beam)
  [V]  "vLLM 实现 Reflection Beam 501B MoE 模型 Day 0 支持" (vLLM day-0 post for Beam)
  [H]  "Reflection 发布 501B 开源模型 Beam，Apache 2.0 许可" (translated HF launch post)
  [N]  "Reflection Beam 技术笔记：501B MoE 如何把「大容量」和「可部署」拧在一起" (third-party notes)

What is computed (all float64 unless a step fixes another precision):
  router    logits = x . W_r^T, s = sigmoid(logits), b = s + bias           [V] §MoE and residual stream;
                                                                              [S] §Dense Layers and Grouped MoE Routing
  selection group score = sum of the two largest b in the group; keep the best Gk groups;
            top-K experts by b over the union of kept groups; ties -> lower index   [H] §专家混合; [V] ibid.
  weights   w_k = scale * s_k / sum_j s_j (bias not included)               [V] ibid.; [H] §专家混合
  experts   SwiGLU: h = silu(gate . x) * (up . x), y = down . h              [H] §专家混合; [N] §1
            with the bf16 rounding points of the BF16 kernels ([S] §BF16 MoE Kernel Optimization):
            gate/up outputs -> bf16, activation product -> bf16; FP32 routing weight applied to the
            down output before any rounding; FP8 variant quantises x per token and h per row.
  combine   out = sum_k w_k * y_k, fixed k order, no shared expert           [V] ibid.; [H] §专家混合

Modules: codecs (bf16 / e4m3 codecs, activation quantisation), router (logits, scores, group-limited
selection, weights, cut margins), experts (expert MLP under each numerics contract, combine).
Every function is pinned by the CPU tests in tests/test_oracle_*.py against brute force, closed
forms, exact rational arithmetic or library routines — none against this code itself.
"""
from . import codecs, experts, router  # noqa: F401
