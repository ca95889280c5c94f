"""FlowCache per-step hot path on MI355X (gfx950).

Two parts, both exported by the C-ABI library ``libflowcache.so`` built from
``csrc/``:

* joint importance-redundancy KV-cache compression (``fc_kv_compress``);
* chunkwise relative-L1 reuse decision (``fc_chunk_rel_l1_decide``).

``kv_cache_compression_fc_amd.binding`` is the thin Python binding (argument
marshalling only); importing it loads the library and fails loudly when the
library is missing.  ``kv_cache_compression_fc_amd.synth`` draws the seeded
synthetic inputs.
"""
