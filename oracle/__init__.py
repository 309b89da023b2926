"""CPU oracle for the asymmetric quantized KV cache.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The HIP library
under ``asymmetric_quantized_kv_amd/`` never imports it, and this package never
imports the library: the two share no code.
"""
from .kvq_oracle import *  # noqa: F401,F403
