"""fp64 CPU oracle for the Mamba-2 SSD forward and the decode state update.

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py`` may import anything from here.  The
HIP library and its Python binding never import, load or call this package,
and this package never imports them: the two sides share nothing but the
seeded input generator.

Contents
--------
``serial``   the plain serial recurrence in C (``ssd_oracle.c``), built with
             gcc + OpenMP and called through ctypes; the definition every GPU
             result is compared against.  Also its gradients (``backward``),
             by reverse-mode differentiation of the same loop.
``forms``    independent NumPy formulations used to pin the serial oracle:
             a NumPy serial loop, the quadratic (masked semiseparable-matrix)
             form and the four-step chunked form.
``metrics``  the two error measures that the parity tolerances are stated in.
``dt``       the layer's time-step preprocessing (bias, softplus, clamp) in
             fp64, for the library's fused preprocessing.
``conv``     the layer's causal depthwise convolution (+ SiLU) and its decode
             update, in fp64.
``norm``     the layer's gated RMS normalisation after the scan, in fp64.
``varlen``   packed variable-length sequences: the serial oracle run on every
             sequence of a row separately.
``gate``     the output gate y * silu(z) and a per-(head, column) D on top of
             the serial oracle, in fp64.
"""
from .serial import backward, build, forward, forward_slices, state_update, max_threads  # noqa: F401
from . import conv, dt, forms, gate, metrics, norm, varlen  # noqa: F401
