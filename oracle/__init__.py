"""CPU oracle for the tree-verification step.  TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously correct reference of what the verification step
computes, in float64:
  * ``mask``      - the ancestor-or-self tree mask and node depths;
  * ``attention`` - tree attention over a paged prefix plus tree ancestors;
  * ``sampling``  - softmax of target/draft logits, Philox4x64-10 uniforms and
                    the root-down rejection-sampling walk (plain C, fp64);
  * ``commit``    - the KV commit of the accepted path (copying and in place);
  * ``expand``    - top-k (or sampled without replacement) draft tokens,
                    log-probabilities and entropy per row;
  * ``select``    - the budget-constrained top-M subtree by cumulative log q,
                    and entropy-ranked branching widths;
  * ``topology``  - the budget's best tree topology by dynamic programming
                    under acceptance by sibling rank;
  * ``cost``      - the speedup model and the per-position overhead fit;
  * ``step``      - the four composed.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import, call, link or execute anything in this package. The
GPU library never does, and this package shares no code with it.

Functions pinned only by properties that the pages do not fix are marked
"parity unpinned" in their docstrings; at present there are none.
"""

from .mask import tree_mask, ancestor_matrix  # noqa: F401
from .attention import tree_attention, bf16_bits_to_f64  # noqa: F401
from .sampling import (softmax, philox4x64_10, node_uniforms,  # noqa: F401
                       verify_walk, verify_greedy, WalkResult)
from .commit import kv_commit, kv_commit_inplace  # noqa: F401
from .expand import expand_topk, expand_sample, gumbel_keys  # noqa: F401
from .select import select_topm, widths_by_entropy  # noqa: F401
from .topology import topology, tree_value  # noqa: F401
from . import cost  # noqa: F401
from .step import verify_step_ref  # noqa: F401
