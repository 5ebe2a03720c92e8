"""CPU oracle of the DFlash drafter step.  TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The HIP library never calls it, it shares
no code with the HIP library, and it imports nothing from the
``block_diffusion_drafter_gemm_amd`` package.  Its inputs come from
``dflash_synth`` (seeded draws only) or from its own computations.

It is plain numpy in float64.  Where the drafter stores a tensor in bf16 (or
fp32 in the tiny configuration), the oracle rounds its float64 value to that
type at the same point (round to nearest, ties to even), so the two sides
differ only by accumulation order.

Sources, cited by page title and section:

* [FN]  "DFlash — 블록 확산 드래프터로 6배 빨라지는 투기적 디코딩" (LLM field
  notes appendix): §1 standard speculative decoding, §2 the one-pass drafter
  cycle, the acceptance-length box and KV injection, §3.1 shared embedding /
  LM head, §6 non-causal in-block attention, §7 one-step masked prediction.
* [INS] "한 번에 초안을 생성하는 DFlash …" (molayo insight article): the
  paragraph on fusing multi-layer target features with a lightweight projection
  and injecting them into every drafter layer's Key/Value.
* [SUM] "기술 요약: DFlash – 플래시 추측적 디코딩을 위한 블록 확산" (gist.science
  summary of arXiv 2602.06036): §2.2 inference design (feature extraction, KV
  injection, parallel block diffusion), §2.3 shared frozen embedding / LM head.
* [PKR] "DFlash 소개" (discuss.pytorch.kr): the BERT-style masked prediction
  paragraph and the ``spec_generate`` usage example.

Modules: ``numerics`` (storage rounding), ``drafter`` (inject, draft block,
LM head, accept length), ``target`` (tiny target, greedy and speculative
decoding, the causal block verify under the storage rounding contract), ``sampling`` (Philox4x32-10 draws, Gumbel-max sampling and the
speculative-sampling accept rule at temperature > 0).
"""
from .numerics import round_bf16, round_f32, round_storage, bf16_bits, from_storage  # noqa: F401
from . import drafter, sampling, target  # noqa: F401
