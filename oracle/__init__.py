"""CPU oracle for STAR-KV decode attention over a low-rank, quantised KV cache.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run anything in this package.
The product path (``rank_kv_cache_starkv_amd`` and ``libstarkv``) never calls it
and shares no code with it; the two meet only through the seeded inputs of
``rank_kv_cache_starkv_amd.inputs`` and through their outputs, which the tests
compare.

Modules:

* ``starkv_oracle`` -- the method step by step (rank selection, factor build,
  calibration, latent projection, quantisation, the cache byte format,
  reconstruct-then-attend, latent-space attention, split-K merge), NumPy fp64
  except where a step is defined in fp32/fp16/bf16.
* ``accounting`` -- closed-form bit and byte accounting of the compressed cache.
* ``brute`` -- a pure-Python brute force (exact rationals, ``math.fsum``) for
  tiny inputs.

Parity status: every function is pinned by ``tests/test_oracle_pins.py``
(closed forms, library routines, invariants, brute force) except the
end-to-end values of *quantised* attention, which the pages do not fix
numerically: those are "parity unpinned" beyond the invariants that hold for
them (quantiser round-trip bounds, pack/unpack, reorder, merge, brute force on
tiny inputs).
"""
