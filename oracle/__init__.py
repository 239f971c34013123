"""Reference (oracle) implementation of paged-KV attention: TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import or run anything in this package.  The library's product path never touches it, and this
package imports nothing from the library or its Python binding.

* ``oracle.attention`` - numpy float64 definition: explicit block-table gather, then masked
  softmax attention per q-head; pool append (scatter) and block copy as plain integer indexing.
* ``oracle.quant``     - the int8 pool: per-(token, KV head) absmax quantisation in fp32, the int8
  storage layout, and attention on the dequantized values (float64, via ``oracle.attention``).
* ``oracle.sparse``    - sink + window sparse attention: each row past a length threshold reads
  only the sequence's first positions and its latest ones (a key mask on ``oracle.attention``).
* ``oracle.hoststore`` - the host page store for parked blocks: page bytes, the 128-bit content
  hash that identifies equal pages, and a store model that dedups by comparing bytes.
* ``oracle.brute``     - pure-Python brute force for tiny inputs (``math.fsum``, log-sum-exp
  normalisation, element-wise scatter by the storage formula, a quantiser rounding each
  operation to float32) used to pin ``oracle.attention``, ``oracle.quant``, ``oracle.sparse`` and
  ``oracle.hoststore``.

Every function is pinned by a ``-m "not gpu"`` test against something other than itself
(brute force, closed forms, invariants).  Nothing here is "parity unpinned".
"""
from . import attention, brute, hoststore, quant, sparse  # noqa: F401
