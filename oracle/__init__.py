"""CPU oracle for Forest Cascade Attention -- TEST INFRASTRUCTURE ONLY.

Plain, slow, fp64 definitions of what the decode path computes.  Only the
tests, the smoke check and the benchmark's CPU-baseline leg may import this
package; the library never does, and it shares no code with the HIP path.

What it defines (citations are to the ZoRRo Inference & Forest Cascade
Attention page, section "Overview"/"Core Mechanism", unless stated):

* ``attention``  -- standard per-request softmax attention over a paged cache,
  no cascade: Forest Cascade Attention is stated to be mathematically
  equivalent to it.  Also the partial (o, max, denominator) triple of a token
  subset and the exact log-sum-exp merge of such triples, used to pin the
  split/merge identity.
* ``grouping``   -- discovery of request groups that share a cache prefix, as a
  dictionary trie over physical block IDs, in canonical order.
* ``accounting`` -- logical and unique KV bytes of a batch.

Pins (see tests/): brute-force softmax on tiny inputs, closed forms,
invariants (split/merge, block order, relabelling, request permutation, GQA
replication), a layout pin with coded values, the construction truth of every
seeded forest, brute-force set grouping on random tiny forests, and the
worked numbers printed on the PagedAttention vs. RadixAttention page.
"""

from . import accounting, attention, grouping  # noqa: F401
