"""CPU oracle for the paged QK-norm + RoPE + grouped-query attention step.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. The GPU library
(``qk_norm_rope_amd``) never imports it and it imports nothing from there.
"""
from .qknr_oracle import *  # noqa: F401,F403
