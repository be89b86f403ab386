"""CPU oracle for balanced expert-parallel MoE dispatch.

TEST INFRASTRUCTURE, NOT PART OF THE LIBRARY. Only the tests, the smoke check and
the benchmark's CPU-baseline leg may import this package. The GPU library never
calls it and shares no code with it: the only code both sides use is the seeded
input generator ``redundant_expert_balancing_amd.synth``, which holds none of the
method's arithmetic.

The oracle is plain, slow and written to be checked by eye: Python loops over
ranks, experts and slots, numpy only for storage and for library steps (bincount,
matmul), float64 for every floating-point value.

Sources (cited below by the short name in brackets):

[noticiai]  noticiai.com.br, "Moonshot AI libera MoonEP: biblioteca de codigo
            aberto para balanceamento perfeito em modelos MoE"
[spaxe]     spaxe.top, "Moonshot AI Open-Sources MoonEP: A Perfectly Balanced
            Expert Parallelism Library for MoE Training" (no headings; cited by
            paragraph number, 1-based)
[maestro]   ai-maestro.online, "Moonshot AI open-sources MoonEP, a perfectly
            balanced expert parallelism library"
[hamidun]   news.hamidun.com, "Moonshot AI otkryla kod MoonEP"

Modules:
  plan   -- the redundant-expert plan (which rank serves which token-slot).
            Parity unpinned against the pages for the choice among valid plans:
            the pages fix no planning algorithm, so this is a stated rule; every
            property the pages do fix is pinned by tests.
  moe    -- dense and plan-based forward / backward of one expert projection,
            the permute, combine and reduce_grad steps, bfloat16 rounding.
  check  -- an invariant checker that accepts any valid plan without knowing
            the rule.
  ffn    -- the full expert FFN on the same plan (gate/up projection, SwiGLU,
            down projection), dense and plan-based, forward and backward, with
            the layer's rounding points; column-selective helpers for sampled
            checks at full size. The activation is a reading: the pages name
            the intermediate size H' but no activation.
"""
