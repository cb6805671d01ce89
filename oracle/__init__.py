"""CPU oracle for the mixed-precision KV-cache hot path.

TEST INFRASTRUCTURE ONLY. Nothing in the product path (the libkvq library and
its Python binding) may import, call or link anything under this directory;
only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` use it.

The oracle is a plain, slow restatement of what the source pages define,
written in float64 numpy plus exact Python integers/Fractions wherever a
result has to be bit-exact (codes, scales, offsets, packed bytes, masks). It
shares no code with the HIP path. Every function cites the page and section it
follows; the pages are:

* MixKVQ (ACL 2026) summary, papercache.org - query-aware 3-tier Key channels
* QJL (AAAI 2025) summary, papercache.org - 1-bit JL sign sketch of Keys
* PN-Mix reproduction notes, daiwk.github.io - RoPE-pair precision mask, H3/L1
* "KIVI quantization axes" blog, charlestar.github.io - grouping axes, RNE,
  packing order, residual state machine, global softmax, storage formula
* InnerQ digest, shd-paper.top - sink/recent windows, folding K scales into q

Parity-pin status of each function is stated in its docstring; functions whose
result no page fixes independently say "parity unpinned".
"""
