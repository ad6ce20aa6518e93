"""IVF-PQ approximate nearest-neighbour search on MI355X (gfx950).

The search runs in hand-written HIP kernels behind the C ABI of
``include/ivfpq.h`` (``libivfpq.so``); this package holds the ctypes binding
(``binding``), the in-tree build (``build_lib``) and host-side input tooling
(``datagen``: seeded generators, CPU index builder, index file).
"""
from .binding import (IVFPQError, FlatIndex, Index, ivfpq_assign_encode_ex,  # noqa: F401
                      ivfpq_build_index_ex, ivfpq_index_export,
                      ivfpq_compute_luts_ex,
                      ivfpq_coarse_ex, ivfpq_flat_free, ivfpq_flat_load_bf16,
                      ivfpq_flat_profile_begin, ivfpq_flat_profile_end, ivfpq_flat_search_bf16,
                      ivfpq_flat_search_bf16_ex, ivfpq_free_index, ivfpq_index_info, ivfpq_kmeans_ex,
                      ivfpq_last_error, ivfpq_load_index,
                      ivfpq_load_index_host, ivfpq_profile_begin, ivfpq_profile_end,
                      ivfpq_search, ivfpq_search_ex, ivfpq_select_topk_ex, ivfpq_status_string,
                      ivfpq_stream_read,
                      ivfpq_validate_host_index, ivfpq_validate_index_file)
