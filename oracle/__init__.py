"""FP64 CPU oracle for the CSA hot path: indexer -> causal top-k -> gather ->
sink-softmax attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import this
package; only the tests, the smoke check and the benchmark's CPU-baseline leg
use it.  It shares no code with the HIP library (its own E4M3/BF16 decoders,
its own indexing), and it is plain and slow on purpose so that a reader can
check it against the pages by eye.

Sources (cited by page title and section):
  [Audit]   "DSV4 Audit -- Decode Repetition + Precision / Tensor-Core Plan"
            (both revisions): A3 (visible range of compressed blocks, SWA /
            compressed overlap), A4 (inverse RoPE of the attention output
            at the query position), B1 (FP8_E4M3 nope dims + BF16 rope dims),
            B2 (indexer scoring einsum 'tnd,cd->tnc', weighted-ReLU MQA
            logits, top-k with no global lock; the FP4 variant of its QK).
  [Roadmap] "ROADMAP -- Stage E and the path to a runnable model": E1 (paged
            FP8 cache with block table and stored inverse scale; gathers of
            selected / all compressed entries and of the SWA window), E4
            (attention returns (o, lse)), E7 (top-k over indexer scores; FP4
            indexer scoring).
  [README]  "DSV4 Inference Kernel": Architecture (CSA m=4, HCA m'=128, a
            512-d latent shared by all 128 heads, sink weights merging the
            sparse and SWA branches), KV cache management (SWA window state,
            paged compressed cache).

Readings taken where the pages are silent are listed in each function's
docstring.  Every function here is pinned by the `not gpu` tests in
tests/test_oracle_*.py against closed forms, library routines, invariants and
pure-Python brute force on tiny inputs.
"""
from .codecs import e4m3_decode, bf16_decode, e2m1_decode, e8m0_decode, mxfp4_decode  # noqa: F401
from .csa import (  # noqa: F401
    n_visible, index_scores, topk_select, key_rows, attend, run_decode_path,
    run_attention, merge_by_lse, dequant_entries, entry_rows, inverse_rope, index_scores_mxfp4,
    index_scores_unquantised,
)
