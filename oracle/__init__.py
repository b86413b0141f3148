"""CPU oracle for paged-KV decode attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the C-ABI library
and its Python binding) never calls it and shares no code with it.

Everything here is plain fp64 NumPy written from the defining passages of
the pages (cited per function).  ``oracle.octave`` holds the quantized
packed-cache codec and attention over it.  See ``oracle.attention`` for the parity
status of each function; every function is pinned by ``tests/test_oracle*.py``
against closed forms, brute force, a library routine or hand-computed
fixtures under ``tests/golden/``.
"""

from .attention import (  # noqa: F401
    HND,
    NHD,
    decode_attention,
    decode_attention_varlen,
    gather_kv,
    key_bounds,
    merge_states,
    query_maps,
    segment_state,
    split_decode_attention,
)
