"""Plain fp64 CPU oracle for one training step of nanochat's dense GPT.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or
execute anything under ``oracle/``; only ``tests/``, the smoke check in
``__graft_entry__.py`` and the ``cpu_baseline`` leg of ``bench.py`` use it.
It shares no code with the HIP path: it has its own config, its own
parameter layout, its own random generator and its own arithmetic.

Pages cited in this package (titles as printed on them):
  [release]  followin.io news article on Karpathy's nanochat release
             (zh-Hant, via AI前線/36氪); the model's architecture bullet list
             sits in its section "純手寫 8000 行代碼，“Agent 幫不上忙”".
  [summary]  aibars.net, "nanochat 專案詳細介紹".
  [tutorial] wmrh.cn tutorial (zh-CN), numbered sections 1-6.
  [harness]  vnrom.net, "nanochat: khung thử nghiệm đơn giản nhất để huấn
             luyện mô hình AI".
  [blog]     hsin-life.com, "你不知道的nanochat：輕量級端到端訓練如何挑戰
             OpenAI霸主地位".
"""
from .model import (OracleConfig, layout, param_count, unpack, forward_loss,
                    forward_backward, rmsnorm, rmsnorm_bwd, rope_tables,
                    rope, rope_bwd, causal_mqa, causal_mqa_bwd, softcap_ce_rows,
                    row_forward)
from .rng import splitmix64_stream, init_params
from .eval import bits_per_byte, bits_per_byte_from_losses

__all__ = [
    "OracleConfig", "layout", "param_count", "unpack", "forward_loss",
    "forward_backward", "rmsnorm", "rmsnorm_bwd", "rope_tables", "rope",
    "rope_bwd", "causal_mqa", "causal_mqa_bwd", "softcap_ce_rows", "row_forward", "splitmix64_stream", "init_params",
    "bits_per_byte", "bits_per_byte_from_losses",
]
