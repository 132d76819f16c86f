"""CPU oracle for weight-absorbed MLA decode.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import, call or execute anything
in this package.  The GPU library (``mla_latent_kv_03_amd``) never imports it and
shares no code, table or helper with it.

Everything here is plain float64 NumPy (or pure Python for the brute-force
forms), written from the MLA pages' definitions, slow and obviously correct.

Modules
-------
mla_ref      : RoPE, the non-absorbed (plain) and absorbed forms, split partials,
               the log-sum-exp combine, the split-table partition rule and the
               paged append reference.
fp8          : OCP FP8 E4M3 ("fn") decode table and round-to-nearest-even,
               saturating encoder, plus the per-token amax quantizer.
bruteforce   : pure-Python scalar loops for tiny inputs.
cache_cost   : the per-token KV-cache cost formula and the MLA row size.

Pins (what each function is checked against) are listed in each module header.
No function here is "parity unpinned": every one has at least one pin that does
not re-derive it from its own code.
"""
