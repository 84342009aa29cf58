"""MI355X-native multi-head differential attention.

The compute lives in libdiffattn.so (hand-written HIP kernels for gfx950 behind
a C ABI, declared in include/diffattn.h); `binding` marshals torch tensors into
that ABI.  `workloads` holds the seeded synthetic inputs.  Importing the
package loads nothing; `binding` loads the library on first use and raises if
it is missing.
"""
__all__ = ["binding", "workloads"]
