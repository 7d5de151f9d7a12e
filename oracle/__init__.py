"""CPU oracle of SpecFold's folded multi-branch verification layer.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls, links or
executes this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may use it.  It shares no code with the HIP
path (``sparse_layer_rho_amd``); the only code both sides use is the seeded input
generator in ``synth``.

It is a plain, slow, step-by-step float64 NumPy restatement of what the pages say
the layer computes.  Pages cited (by title and section, as the pages label them):

* [SpecFold summary] "SpecFold: Folding Multi-Branch Redundancy for Faster
  Speculative Decoding in Diffusion Language Models", paperlayer.ai source-linked
  summary of arXiv 2610.04875v2 (sections §1-§5, Appendix A-D, Figures, Tables).
* [SpecFold review (ko)] "SpecFold가 확산 언어모델 추측 디코딩의 분기 중복을 접어
  속도를 높인다", onedev.kr/papers/830 (sections "무엇인가", "어떻게 동작하나",
  "무엇과 다른가", "어떻게 쓰나", "전제와 한계").

Every function here is pinned by a ``-m "not gpu"`` test to something other than
itself (closed forms, brute force, library routines, invariants); there is no
"parity unpinned" function in this package.
"""

from .layer import (  # noqa: F401
    attention_block,
    compact,
    dense_branch_layer,
    ffn_rows,
    gate,
    qkv_rows,
    resolve,
    rms_norm,
    rope,
    silu,
    stack,
    verify_layer,
)
from .tables import verify_layer_tables  # noqa: F401
from .correction import folded_attention_by_correction  # noqa: F401
from .head import embed, final_norm, greedy_tokens, lm_head_logits, verify_head  # noqa: F401,E402
