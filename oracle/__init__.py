"""CPU oracle for the routed-expert FFN step over an HBM slot cache.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, obviously-correct
CPU restatement of what the method computes.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import or run it.  It shares no code with the HIP library (it imports nothing
from ``expert_ffn_serving_amd``); both sides take their inputs from ``synth``.

Sources (the four pages, cited by title and section):
  [FT-deep]   "FreeToken 딥다이브 — 게이밍 PC 한 대로 284B 모델을 돌리는 엔진" (fiv.co.kr)
  [FT-blog]   "FreeToken:让消费级电脑跑起 284B MoE，一次把整机当成推理集群的系统设计"
  [NVMe-8GB]  "NVMe에서 전문가(experts)를 스트리밍하여 8GB GPU에서 133GB MoE 모델 구동하기 (11 토큰/초)"
  [Edge0]     "SSD 가중치층으로 35B MoE를 라우팅 예측으로 24GB 데스크톱에서 서빙한다" (onedev.kr)

Modules:
  formats  number formats (bf16, int4-g32, e2m1, e4m3) and the record layout decoder
  qstar    the Q16 bandwidth-matched split rule and its brute-force definition
  router   fixed-order fp32 router logits, top-k, softmax weights
  ffn      SwiGLU expert and top-k-weighted combine (fp64)
  policy   slot cache state machine: ensure / split / install (integer, step by step)
  engine   a decode layer and a prefill layer put together from the above
  cffn     binding of ffn_ref.c, the same expert FFN as plain C loops (large shapes)

Parity pins: every function is checked in tests/test_oracle_*.py against
closed forms, brute force, invariants or values printed on the pages.
"""
