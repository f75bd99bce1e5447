"""Float64 CPU oracle for block-sparse causal prefill attention with mean correction.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this package.  The
library in ``block_sparse_long_scores_amd`` never imports it, and it imports
nothing from the library: the only code the two sides share is the seeded
input generator in ``synth``, which holds none of the method's arithmetic.

Every function is plain NumPy in float64, written to be checked against the
pages by eye.  The pages are cited by title and section:

* [ABS]  "FlashPrefill V2: block-sparse prefill attention for long-context LLM
  serving" -- the abstract (chatpaper.ai page; English and Traditional-Chinese
  text of the same abstract).
* [EXP]  "128K 长上下文还在等'读秒开聊'？arXiv 2608.19758 把预填充加速拉到 47×
  的工程真相" (papers.ananclaw.com explainer): §1.1 (prefill is O(N^2)
  softmax(QK^T)V), §2.1 (algorithm layer: V1 keeps the threshold-selected keys
  of each query block, V2 adds the mean-correction term of the Out_q^V2
  formula), §2.2 (PackGQA), §2.3 (FP8 E4M3 with scale calibration, paged KV,
  continuous batching).
* [SCR]  "FlashPrefill V2 短脚本镜像" (papers.ananclaw.com script page): §4
  storyboard scene-4 (the same Out_q^V2 formula).
* [NEWS] the 163.com article and the iitog.ru article (key facts): mean
  correction suppresses approximation error; pattern discovery plus max-based
  dynamic thresholding come from FlashPrefill V1.

Pins: every function here is checked in ``tests/test_oracle.py`` against
brute force, closed forms, invariants or a library routine.  The
sparse-vs-dense *quality* figures are reported, not pinned: the pages print
no error numbers ("parity unpinned" for that report only).
"""

from .attention import (  # noqa: F401
    Geometry,
    geometry,
    pool,
    block_scores,
    select,
    attend,
    dense_attention,
    sparse_prefill,
    correction_split,
    sparsity,
    score_band_mask,
)
from .e4m3 import e4m3_decode, e4m3_encode, dequantize  # noqa: F401
