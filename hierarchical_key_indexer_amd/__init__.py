"""LSA indexer for AMD MI355X: HIP kernels behind a C ABI (include/lsa.h).

``_abi`` is the ctypes binding of liblsa.so, ``indexer.LatentIndex`` owns the
device buffers of one index, ``build_lib.build()`` compiles the library.
"""
from . import _abi  # noqa: F401
from ._abi import IndexDesc, LsaError, SelectParams, load  # noqa: F401
