"""CPU oracle for the Sparse Delta Memory write/read (test infrastructure only).

Only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may import this package.
The product path (the HIP library and its Python binding) never imports it.
"""
from .sdm_oracle import (  # noqa: F401
    build,
    factor_scores,
    lib_path,
    round_bf16,
    softmax,
    topk,
    topk_one,
    write_read,
    write_read_backward,
    write_read_backward_bounds,
    e4m3_round,
    snap_rows,
    snap_scale_exp,
    U_F32,
)
