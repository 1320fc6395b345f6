"""MI355X-native batched paged MLA decode (absorbed form).

The compute path is the HIP library libmla_decode.so (C ABI in
include/mla_decode.h); paged_mla_decode_03_amd.binding is its ctypes binding.
Importing the package loads nothing; the first call loads the library and
raises if it is missing.
"""

from .binding import (  # noqa: F401
    decode,
    load_library,
    make_dims,
    mla_decode_paged,
    mla_decode_paged_workspace_size,
    mla_status_string,
    workspace_bytes_for,
)
