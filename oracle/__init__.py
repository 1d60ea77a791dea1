"""CPU oracle for block-sparse video attention -- TEST INFRASTRUCTURE ONLY.

This package is the plain, slow, obviously-correct statement of what the
block-sparse attention path computes.  It exists to check the HIP library and
is used only by ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline
leg of ``bench.py``.  The product path (the ``libvsa`` shared library and its
Python binding) never imports, calls or links anything in here, and nothing in
here imports the product path.

Modules
  vsa_oracle  fp64 numpy definition: tile order, routing, window rule, CSR,
              tile-major permute, masked softmax attention, split merge.
  brute       pure-Python loops for tiny grids (an independent second writing
              of the same definition, used to pin ``vsa_oracle``).
  fit_dense_count  script that fits the routed count of the HunyuanVideo-shaped
              call to a retained density of about 10%.

Parity pins: every function of ``vsa_oracle`` is pinned by a CPU test against a
closed form, a textbook routine or brute force (see ``tests/test_oracle_*``).
"""
