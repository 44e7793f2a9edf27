"""fp64 CPU oracle for exact attention.

TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check in
``__graft_entry__.smoke`` and the CPU-baseline leg of ``bench.py`` may import
this package. The library (``exact_io_aware_07_amd``) never imports it and
shares no code with it; the two meet only at the seeded input generator.
"""
from .attention import (attn_bwd64, attn_bwd64_magnitudes, attn_bwd64_sampled, attn_fwd64,  # noqa: F401
                        attn_probs64, visible_mask)
from .brute import (brute_head_allowed, brute_head_forward, brute_head_grad_fd,  # noqa: F401
                    brute_head_part, brute_loss, brute_loss_allowed)
from .memory import score_matrix_bytes  # noqa: F401
from .split import attn_part64, merge64  # noqa: F401
from .gqa import attn_bwd64_gqa, attn_fwd64_gqa  # noqa: F401
from .sparse import (attn_bwd64_sparse, attn_bwd64_sparse_sampled, attn_fwd64_sparse,  # noqa: F401
                     sparse_visible)
from .fp8 import (E4M3_MAX, attn_fwd64_fp8, e4m3_decode, e4m3_encode, fp8_quantize,  # noqa: F401
                  fp8_quantize_rows, fwht32, mfma_loss_bound)
