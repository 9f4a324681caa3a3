"""CPU fp64 oracle for the gated delta-rule recurrent decode step.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, calls or
links anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with
the HIP library (no kernels, headers, helpers, tables or constants) and does
not import it; the two meet only on the seeded inputs made by
``recurrent_state_decode_amd.workloads``.

Everything here is plain NumPy in float64 (or ``fractions.Fraction``), slow
and written to be checked by eye against the pages it cites:

* ``activations`` -- L2 normalisation, softplus gate, sigmoid beta
  (max.nn.state_space.kda_decode, description and Parameters;
  flashinfer.gdn_paged.gated_delta_rule_decode_paged, signature).
* ``recurrence``  -- the sequential per-token step, with one decay per head
  (GDN) or one per key row (KDA) (Circuit.LLM.Mixer, "Delta rule" and
  "Gated memory").
* ``e4m3``        -- OCP FP8 E4M3 decode table, round-to-nearest-even with
  saturation, and the per-[K, block_v]-tile amax quantise/dequantise
  (modelopt ... linear_attention.config, LinearAttentionConfig).
* ``paging``      -- slot/page resolution for the pooled and CSR-paged pools
  (flashinfer.gdn_paged.gated_delta_rule_decode_paged, description,
  Parameters and Notes; max.nn.state_space.kda_decode, Parameters).
* ``decode``      -- the three decode front-ends built from the above.
* ``chunked``, ``unrolled``, ``exact`` -- independent cross-check forms
  (chunked WY scan, explicit transition products, exact rationals).  They
  import nothing from ``recurrence`` and are compared against it in tests.

Parity status of each function is stated in its docstring; a function with
no independent pin says "parity unpinned".
"""
