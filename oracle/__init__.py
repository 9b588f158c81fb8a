"""CPU oracle for the HiLS attention hot path (test infrastructure).

Only tests/, the smoke check in __graft_entry__ and the CPU-baseline leg of
bench.py may import anything here. The product library never does, and the
oracle never imports the product library.
"""
from .hils_oracle import (hils_forward, hils_backward, hils_decode, hils_route, row_forward,
                          surrogate_scores, rank_chunks,
                          row_backward, select_topk, n_distant, window_start, qcal, f64,
                          logsumexp, softmax)
