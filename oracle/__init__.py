"""CPU oracle for the HiNM sparse-weight x dense-activation product (test infrastructure).

This package is test infrastructure.  Only ``tests/``, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py`` (``cpu_baseline`` and its side-row
functions) may import or call it; the product
path (the HIP library and its Python binding) never does, and shares no code,
header, table or constant with it.

It is a plain, slow, obviously-correct numpy implementation of what the path
computes: the three-region allocation of FlexHiNM-GP, the 2:4 top-2 masks,
the per-tile input permutation, the packed serialisation, and a dense float64
product with the masked weight.  See ``oracle/hinm.py`` for each step and the
passage of the pages it follows.
"""
from .hinm import (  # noqa: F401
    DENSE, TWO_FOUR, PRUNED, KB_DENSE, KB_24, PAD_NIBBLE, LEGAL_NIBBLES,
    Plan, OracleError, plan, vector_scores, regions, index_lists, select24, mask_from,
    serialize, pack, unpack, masked_weight, spmm, retained_importance, boundary_search,
    boundary_grid, bf16_bits_to_f64,
)
