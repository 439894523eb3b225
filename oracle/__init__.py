"""CPU oracle of the gated delta rule path -- TEST INFRASTRUCTURE ONLY.

Plain, slow, float64 numpy implementations of what the HIP library computes,
written from the gated delta rule as the Agnes-3.0-Flash pages describe it
(the update rule in words on the gpts24 page, "gated DeltaNet" paragraph; the
gate formulas and the recurrent call on the yfxerp page, section 1.2) and the
formula S_t = S_{t-1} exp(g_t) (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
o_t = S_t q_t.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports, links or calls anything here; the two share
no code except the seeded input generators.

Modules
  gdr   -- token-serial recurrence (the definition), fp64 chunk-form model
           (equivalence pin only), decode step
  conv  -- causal conv + SiLU (fp64, and the fixed-order fp32 evaluation that
           defines bit-exactness), gates, gated RMSNorm, bf16 rounding

No function here is "parity unpinned": each is checked by the tests in
``tests/test_oracle_*.py`` against closed forms, special cases, invariants or
brute force.
"""
