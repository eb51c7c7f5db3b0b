"""libncattn: nanochat's attention hot path as hand-written gfx950 HIP kernels.

The compute lives in the C-ABI shared library ``libncattn.so`` built from
``csrc/``; ``native`` loads it and exposes its entry points under the same
names (argument marshalling only). Importing this package loads nothing; the
library is opened on first use and a missing library is an error.
"""

__all__ = ["native", "synth", "workload"]
