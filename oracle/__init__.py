"""fp64 CPU oracle for one device's share of a Ring Attention forward pass.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product path
(``ring_attention_block_step_amd`` and its HIP library) never imports, calls or
links it, and this package imports nothing from the product path.

Everything here is plain NumPy in float64, written from the method's definition
on the pages:

* "Ring Attention" (aarnphm.xyz), the recurrence for S, m, z, y and O over the
  ring order b(u, s) = (u - s) mod p;
* "Ring Attention: distributed attention across devices" (aicomputerinstitute),
  section "Building block: the online-softmax trick" and the section
  "Worked example: tracing the ring by hand";
* "Ring Attention" (darshanfofadiya.com), section 4.4 "Online Softmax Across KV
  Blocks" and section 4.8.1 "Skipping Fully-Masked Blocks";
* the transformer-math page on Ring Attention (aicassindra.com), sections "The
  mechanism, compressed", "Causal masking wastes half the ring" and "The ring is
  a prefill algorithm" (the rescale-and-add merge of partial triples, and the
  decode split that keeps key/value shards stationary) and "The backward pass
  costs a second ring" (the backward ring with scores rebuilt from the saved
  statistics);
* "Ring Attention" (darshanfofadiya.com) 4.8.3 (the zigzag assignment) and
  4.9.4.4 (pass-Q decode).

Every function is pinned by ``tests/test_oracle.py`` against values the pages
print, closed forms, brute force on tiny inputs and invariants.  No function
here is "parity unpinned".
"""

from .ring_oracle import (  # noqa: F401
    NEG_INF,
    allowed_mask,
    allowed_pair_count,
    backward_dense,
    backward_sampled,
    decode_partial,
    dense_attention,
    empty_state,
    finish,
    merge_partials,
    online_fold,
    ring_backward,
    ring_forward,
    shard_positions,
)
