"""CPU oracle for exact attention: TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import or call anything in this package.  The GPU library and
its Python binding never import it, and it imports nothing from them.

Contents
--------
``attention_ref``  plain fp64 standard attention: materialises the score
                   matrix S and the probability matrix P (per block of query
                   rows, over every key), then O = P V and the row logsumexp.
``twopass_ref``    the same definition written as explicit Python loops (a
                   max pass, then an exp/sum/weighted-sum pass), tiny inputs.
``online_emul``    the tiled method itself in fp64: query and key/value blocks,
                   a running max and running sum per row, rescaling of the
                   partial output, one division at the end.
``attention_kvcache_ref``  the same attention for a few query rows against a
                   key/value cache of per-batch length (rows aligned to the
                   end of the cache), as in decoding; and for a packed batch
                   of sequences of different lengths (each sequence its own
                   cache case).
``attention_bwd_ref``  fp64 gradients dQ, dK, dV of the forward above for an
                   upstream gradient dO (chain rule through O = P V and the
                   row softmax; P rebuilt per block of rows), with optional
                   absolute-value products for error bounds; and the same
                   for packed sequences of different lengths (each
                   sequence's queries aligned to the end of its keys).

What is computed (all three): for batch b, query head h with key/value head
h_kv = h // (Hq // Hkv), and query row i,
    s_ij = scale * <q[b,h,i,:], k[b,h_kv,j,:]>,  s_ij = -inf where masked,
    p_ij = exp(s_ij - max_j s_ij) / sum_j exp(s_ij - max_j s_ij),
    o[b,h,i,:] = sum_j p_ij v[b,h_kv,j,:],
    lse[b,h,i] = log sum_j exp(s_ij)            (natural log),
with (i, j) masked when (causal and j > i) or (window_left >= 0 and
j < i - window_left).

Sources: the Flash Attention page (heepie.pages.dev), "AS-IS" standard
attention diagram (S = QK^T, P = softmax(S), O = PV) and the tiling section
(blocks rescaled by normalisation factors and summed give the exact result);
the Hacker News answer on GQA and sliding windows (softmax(QK^T)V, a window
only changes the mask, GQA only changes how K/V heads are formed); the
FlashAttention quiz, question 4 (online softmax with running rescaling).
The scale factor, the causal/window conventions, the GQA head grouping and the
logsumexp output are readings of points the pages leave open; each is listed
with its justification in the design notes at the repository root.

Every function here is pinned by tests in ``tests/test_oracle.py`` against
closed forms, invariants, hand-worked fixtures and an independent library
routine (torch's CPU scaled-dot-product attention in float64); the gradients
are pinned in ``tests/test_oracle_bwd.py`` against central finite differences
of the forward oracle, torch's float64 autograd, and closed forms (the
packed form against central finite differences of the packed forward oracle
and against the fixed-length gradients sequence by sequence); the cache
form in ``tests/test_oracle_kvcache.py`` against the last rows of the full
forward oracle, a loop-by-loop brute force, and closed forms.
"""
from .attention_ref import attention_fwd, masked, kv_head_of  # noqa: F401
from .twopass_ref import attention_twopass  # noqa: F401
from .online_emul import attention_online  # noqa: F401
from .attention_bwd_ref import attention_bwd, attention_bwd_varlen  # noqa: F401
from .attention_kvcache_ref import attention_fwd_kvcache, attention_fwd_varlen  # noqa: F401
