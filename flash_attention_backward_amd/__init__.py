"""Flash-attention backward (FLASH_ATTN_BACK) on AMD Instinct MI355X: a C-ABI HIP library
(libfa_back.so, include/fa_back.h) and its ctypes binding."""
from .fa_back import (  # noqa: F401
    DeviceProblem, FaBackError, Layout, Desc, Tensor, describe, fa_back_create, fa_back_destroy,
    fa_back_layout_query, fa_back_run, fa_back_run_noalloc, fa_back_run_timed, load_library, make_tensor, status_string, unpack,
)
