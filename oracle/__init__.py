"""CPU oracle of the performer step -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check of ``__graft_entry__`` and the CPU-baseline
leg of ``bench.py`` may import this package.  The GPU library never calls it
and shares no code, header, table or helper with it.

Every function is the plain definition of what the performer step computes,
in float64 (float32 where the method fixes a float32 decision, e.g. the fp8
quantiser's product).  See ``oracle/performer.py`` for the citations.
``oracle/fp8c.py`` (with ``oracle/fp8_cache.c``) is the fp8 quantiser and
decoder once more in plain C, fast enough for the long fp8 history; it is
pinned bit for bit to ``performer.py``'s and to torch's float8 cast.
"""
from .performer import (  # noqa: F401
    visibility_mask,
    attention_dense,
    attention_over_cache,
    attention_incremental,
    PagedCache,
    PagedCacheFP8,
    e4m3_decode,
    e4m3_encode,
    quantize_rows,
    velocity,
    euler_solve,
    performer_unit,
)
