"""CPU oracle for query-union sparse-attention prefill.

TEST INFRASTRUCTURE.  Only the test suite, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run anything in this
package.  The product path (``query_union_kv_amd``) never does, and this
package never imports the product path: the two share no code.  Inputs come
from the ``workloads`` generators.

What it computes, in plain slow form (numpy fp64, pure-Python integer code):

* ``numerics``   bf16 and OCP fp8-e4m3fn decoding from their definitions.
* ``prep``       per-(query, KV head) page bitsets, the bounded greedy
                 affinity grouping, per-group page-union tables with member
                 masks, the page-visit / masked-slot statistics of
                 PageWeaver Fig. 2 and Fig. 6, and the page-major work items
                 of the direct KV-page union.
* ``attention``  causal softmax attention of every query over exactly its
                 own pages (route A: per-query gather, the definition), the
                 same through group unions with member and causal masks
                 (route B: how the method reaches it) and through the direct
                 KV-page union with per-page partials merged by lse (route C),
                 plus a pure-Python brute force for tiny inputs.
* ``kvcache``    writing a chunk's bf16 keys and values into the paged cache,
                 with per-(KV head, page) fp8 e4m3fn quantisation.

Pins (tests marked ``not gpu``): the Fig. 2 worked example, brute force on
tiny inputs, dense equivalence with a library attention, closed forms,
set-algebra identities, grouping invariance, the fp8/bf16 library casts, the
e4m3fn format's error bound and the workload generator's own quantisation.
The grouping rule's details beyond what Fig. 1/2 state (window, score, seed
and tie-break) are readings, not pinned by the pages beyond Fig. 2: the
heuristic's choices on the synthetic workloads are "parity unpinned" by the
pages and are checked by invariants, hand traces and a brute-force argmax
check instead.
"""
from . import numerics, prep, attention, kvcache  # noqa: F401
