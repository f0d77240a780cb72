"""CPU oracle for the weight-informed activation-sparse linear (fp64, numpy).

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports this package:
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may call it. It shares no code with the HIP library; both sides
take their inputs from ``workloads``.

Every function restates, in plain slow code, what the pages define:

* WINA article (arXiv:2505.19427, lsdiaocha.cn), section 一 (weight-aware
  activation): the gate keeps input j when |x_j * c_j| is among the K largest
  entries of |x (.) c|, c being the column-wise L2 norm of W.
* Spark Transformer article, section 2.2 (statistical top-k operator): fit a
  Gaussian to the vector (mean, population variance) and keep the entries
  above mu + sigma * Phi^-1(1 - s).
* Spark Transformer article, section 3.1 (sparse matrix multiplication, the
  index-list product): y accumulates x_j times the weight vector of input j
  over the active indices only.

* Spark Transformer article, section 2.1 (the FFN scores, selects and
  computes only the selected part): the sparse FFN chain gate/up -> h =
  bf16(SiLU(g) u) -> down, each projection with its own gate
  (``oracle.ffn``).

* Double Sparsity article, section 在线前向计算 (online forward): decode
  attention over the tokens whose label-channel scores are the k largest
  (``oracle.double_sparse``).

Parity status of each function is listed in ``oracle.sparse_linear``,
``oracle.ffn`` and ``oracle.double_sparse``.
"""
from .sparse_linear import (  # noqa: F401
    as_f64,
    column_norms,
    scores,
    topk_gate,
    stat_moments,
    stat_threshold,
    stat_gate,
    normal_quantile,
    active_indices,
    sparse_product,
    sparse_product_rows,
    gate,
    forward,
)
from .ffn import silu, bf16_round, silu_mul, ffn_chain  # noqa: F401,E402
from . import double_sparse  # noqa: F401,E402
from . import ffn  # noqa: F401,E402
