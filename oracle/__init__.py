"""Plain CPU oracle for causal softmax attention in a Gated MLA layer.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU
baseline use it; the GPU library never imports, links or calls it, and the two
share no code.  The arithmetic lives in ``gmla_oracle.c`` (double precision,
written as the definitions read); this module only builds that file with gcc,
marshals NumPy arrays to it, and composes its functions into a layer in the order
that the "Gated MLA" page's "Implementation order" section lists.
"""
from .oracle import (  # noqa: F401
    attend,
    attend_head,
    build,
    default_threads,
    gate,
    gated_mla_layer,
    library_path,
    linear,
    load,
    sigmoid,
)
