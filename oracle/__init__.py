"""fp64 CPU oracle for packed variable-length causal attention.

TEST INFRASTRUCTURE ONLY.  This package is the slow, plain, obviously correct
reference that the HIP library is checked against.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it.  It imports nothing from the HIP library and shares no code,
constants or helpers with it; the two meet only at the seeded input generators
in ``workloads``.

Modules
  attention  per-document softmax attention (forward) and its analytic
             gradient (backward), plus row-sampled versions for large batches
  merge      combination of partial (O, LSE) results over key chunks
  permute    the Ulysses sequence<->head layout change of one GPU's shard,
             with the kv-head split (replication when Hkv < P) of GQA
  schedule   cu_seqlens validation, the tile work lists and the pair counts,
             and the packed-chunk attention-pattern map
  sp_groups  batch-aware sequence-parallel groups and token shards
  router     the NSP planner: SP tree, per-GPU cost model, beam-search routing

Every function cites the passage of the pages it follows (page title and
section / equation / figure).  Where the pages are silent, the reading taken is
named in the docstring.
"""
from . import attention, merge, permute, router, schedule, sp_groups  # noqa: F401
from .attention import (attn_fwd, attn_bwd, attn_fwd_rows, attn_bwd_dq_rows,  # noqa: F401
                        attn_bwd_dkv_rows)
from .merge import lse_merge  # noqa: F401
from .permute import seq2head, head2seq  # noqa: F401
