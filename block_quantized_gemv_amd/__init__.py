"""q4_K x q8_0 decode GEMV for AMD MI355X (gfx950).

The compute lives in the HIP library libmq.so (C ABI in include/mq.h);
``binding`` is its thin ctypes front end over torch device memory and
streams.  ``synth`` draws the seeded synthetic inputs and ``workloads``
holds the benchmark shapes.
"""
from . import synth, workloads  # noqa: F401
