"""CPU oracle for the S3R hot path.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import this package:
only tests/, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of bench.py
use it. It shares no code with the HIP library (no kernels, headers, helpers or
constant tables) and never imports it.
"""
from .s3r_oracle import *  # noqa: F401,F403
from .s3r_oracle import __all__  # noqa: F401
