"""MI355X (gfx950) implementation of the stabilized parallel mLSTM forward pass.

The compute lives in a C-ABI shared library (``libmlstm.so``, HIP kernels for
gfx950, declared in ``include/mlstm.h``); ``linear_recurrent_sequence_amd.mlstm``
is a thin ctypes binding over it.  Importing this package does not load the
library; the first call into the binding does, and fails loudly if it is
missing.  ``workloads`` draws the seeded synthetic inputs.
"""

import importlib

__all__ = ["mlstm", "workloads"]


def __getattr__(name):
    if name in __all__:
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
