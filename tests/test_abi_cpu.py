"""C ABI checks that need no GPU: the library loads, exports every function
include/mla_decode.h declares, and rejects bad arguments with the documented
status codes before touching a device."""

import ctypes
import os
import re

import pytest

from paged_mla_decode_03_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla_decode.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert {"mla_decode_paged", "mla_decode_paged_workspace_size", "mla_status_string"} <= set(names)
    lib = binding.load_library()
    for n in names:
        assert hasattr(lib, n), f"{n} declared in mla_decode.h but not exported"


def test_struct_layout_matches_header():
    # int32 x5, (pad), int64, int32 x4 -> 48 bytes with natural alignment
    assert ctypes.sizeof(binding.MlaDims) == 48
    assert binding.MlaDims.num_pages.offset == 24


def test_status_strings():
    for code in range(14):
        s = binding.mla_status_string(code)
        assert isinstance(s, str) and s
    assert binding.mla_status_string(999) == "unknown status"


FAKE = 1 << 20  # aligned non-null host integer; never dereferenced (validation fails first)


def _call(dims, **over):
    args = dict(q=FAKE, kv=FAKE, bt=FAKE, sl=FAKE, qo=None, max_seq_len=128, max_q_len=1, out=FAKE, lse=None,
                ws=FAKE, ws_bytes=1 << 30)
    args.update(over)
    return binding.mla_decode_paged(args["q"], args["kv"], args["bt"], args["sl"], args["qo"], args["max_seq_len"],
                                    args["max_q_len"], 1.0, 1.0, True, args["out"], args["lse"], args["ws"],
                                    args["ws_bytes"], dims, stream=0)


def _dims(**over):
    d = dict(batch=2, num_heads=16, q_len_fixed=1, total_q=2, page_size=32, num_pages=8, block_table_stride=4,
             kv_dtype=0)
    d.update(over)
    return binding.make_dims(**d)


@pytest.mark.parametrize("over,code", [
    (dict(q=None), 1), (dict(kv=None), 1), (dict(bt=None), 1), (dict(sl=None), 1), (dict(out=None), 1),
    (dict(ws=None), 1),
])
def test_null_pointers(over, code):
    assert _call(_dims(), **over) == code


@pytest.mark.parametrize("dims_over,call_over,code", [
    (dict(num_heads=0), {}, 2), (dict(num_heads=24), {}, 2),
    (dict(page_size=8), {}, 3), (dict(page_size=48), {}, 3),
    (dict(kv_lora_rank=256), {}, 4), (dict(qk_rope_head_dim=32), {}, 4),
    (dict(kv_dtype=7), {}, 5),
    (dict(), dict(q=FAKE + 8), 6), (dict(), dict(out=FAKE + 2), 6),
    (dict(), dict(max_q_len=0), 8), (dict(q_len_fixed=2), {}, 8), (dict(total_q=3), {}, 8),
    (dict(block_table_stride=3), {}, 9),
    (dict(batch=0), {}, 10), (dict(batch=100000), {}, 10), (dict(), dict(max_seq_len=0), 10),
    (dict(batch=1000, q_len_fixed=2 ** 19, total_q=1000 * 2 ** 19, num_heads=16), dict(max_q_len=2 ** 19), 10),
])
def test_bad_arguments(dims_over, call_over, code):
    assert _call(_dims(**dims_over), **call_over) == code


def test_workspace_size_zero_for_rejected_shape():
    assert binding.mla_decode_paged_workspace_size(_dims(num_heads=24), 128, 1) == 0


MISALIGNED = 6


def test_options_struct_and_misaligned_option_pointers():
    # four pointers then three int32, in header order (padded to 48)
    assert ctypes.sizeof(binding.MlaOptions) == 48
    assert binding.MlaOptions.sinks.offset == 16
    assert binding.MlaOptions.sparse_top_k.offset == 40
    assert binding.MlaOptions.q_fp8.offset == 44
    for field in ("bmm1_scale", "bmm2_scale", "sinks"):
        opts = binding.MlaOptions(None, None, None)
        setattr(opts, field, FAKE + 2)
        rc = binding.mla_decode_paged_ex(FAKE, FAKE, FAKE, FAKE, None, 128, 1, 1.0, 1.0, True, FAKE, None, FAKE,
                                         1 << 30, _dims(), opts, stream=0)
        assert rc == MISALIGNED, (field, rc)
    # NULL options behave exactly like mla_decode_paged (here: the same shape error)
    bad = _dims(num_heads=20)
    rc_ex = binding.mla_decode_paged_ex(FAKE, FAKE, FAKE, FAKE, None, 128, 1, 1.0, 1.0, True, FAKE, None, FAKE,
                                        1 << 30, bad, None, stream=0)
    assert rc_ex == _call(bad)


def test_dcp_options_and_merge_partials_reject_bad_arguments():
    def ex(opts, lse=FAKE):
        return binding.mla_decode_paged_ex(FAKE, FAKE, FAKE, FAKE, None, 128, 1, 1.0, 1.0, True, FAKE, lse, FAKE,
                                           1 << 30, _dims(), opts, stream=0)
    BAD_SHAPE, NULL = 10, 1
    assert ex(binding.MlaOptions(None, None, None, FAKE, 0, 0)) == BAD_SHAPE      # cp_world < 1
    assert ex(binding.MlaOptions(None, None, None, FAKE, 4, 4)) == BAD_SHAPE      # cp_rank >= cp_world
    assert ex(binding.MlaOptions(None, None, None, FAKE, 4, -1)) == BAD_SHAPE     # cp_rank < 0
    assert ex(binding.MlaOptions(None, None, None, FAKE, 2, 1), lse=None) == NULL  # partial mode needs lse
    assert ex(binding.MlaOptions(None, None, None, FAKE + 2, 2, 1)) == MISALIGNED
    lib = binding.load_library()
    assert lib.mla_merge_partials(None, FAKE, 2, 16, FAKE, None, None) == NULL
    assert lib.mla_merge_partials(FAKE, FAKE, 0, 16, FAKE, None, None) == BAD_SHAPE
    assert lib.mla_merge_partials(FAKE, FAKE, 2, 0, FAKE, None, None) == BAD_SHAPE
    assert lib.mla_merge_partials(FAKE + 8, FAKE, 2, 16, FAKE, None, None) == MISALIGNED
    assert lib.mla_merge_partials(FAKE, FAKE + 2, 2, 16, FAKE, None, None) == MISALIGNED


NO_DEVICE = 12


def test_sparse_options_reject_bad_arguments():
    """The sparse top-k layout: shape checks come before any device query; a
    call that passes them (seq_lens may be NULL) reaches the device lookup."""
    BAD_SHAPE, BAD_BLOCK_TABLE, NULL = 10, 9, 1

    def ex(dims, k, sl=None, opts_over=None, lse=FAKE):
        opts = binding.MlaOptions(None, None, None, None, 1, 0, k)
        for f, v in (opts_over or {}).items():
            setattr(opts, f, v)
        return binding.mla_decode_paged_ex(FAKE, FAKE, FAKE, sl, None, 1, 1, 1.0, 1.0, False, FAKE, lse, FAKE,
                                           1 << 30, dims, opts, stream=0)
    sd = lambda **o: _dims(**{**dict(batch=3, q_len_fixed=1, total_q=3, block_table_stride=64), **o})
    assert ex(sd(), -1, sl=FAKE) == BAD_SHAPE                                   # negative top-k
    assert ex(sd(), 65) == BAD_BLOCK_TABLE                                      # list wider than its row
    assert ex(sd(total_q=1025, batch=1025), 64) == BAD_SHAPE                    # too many query rows
    assert ex(sd(block_table_stride=(1 << 20) + 1), (1 << 20) + 1) == BAD_SHAPE  # top-k above the limit
    assert ex(sd(num_heads=24), 64) == 2                                        # shared shape checks still apply
    assert ex(sd(), 64, opts_over=dict(seq_lens_global=FAKE, cp_world=2)) == BAD_SHAPE  # not with DCP
    assert ex(sd(), 64) == NO_DEVICE                                            # NULL seq_lens is fine here
    assert ex(sd(), 0) == NULL                                                  # ... but not in the paged layout
    opts = binding.MlaOptions(None, None, None, None, 1, 0, 65)
    assert binding.mla_decode_paged_ex_workspace_size(sd(), 1, 1, False, opts) == 0


def test_fp8_query_option_rejects_bad_combinations():
    BAD_DTYPE, BAD_SHAPE = 5, 10

    def ex(dims, opts):
        return binding.mla_decode_paged_ex(FAKE, FAKE, FAKE, FAKE, None, 128, 1, 1.0, 1.0, True, FAKE, None, FAKE,
                                           1 << 30, dims, opts, stream=0)
    q8 = binding.MlaOptions(None, None, None, None, 1, 0, 0, 1)
    assert ex(_dims(kv_dtype=0), q8) == BAD_DTYPE           # fp8 query with a bf16 cache
    assert ex(_dims(kv_dtype=1), q8) == NO_DEVICE           # fp8 query and fp8 cache: accepted
    sq8 = binding.MlaOptions(None, None, None, None, 1, 0, 4, 1)
    assert ex(_dims(kv_dtype=1), sq8) == BAD_SHAPE          # not in the sparse layout


def test_contract_check_rejects_bad_arguments():
    """mla_decode_check_contract: every host-side rejection comes before any
    device call."""
    lib = binding.load_library()

    def chk(bt=FAKE, sl=FAKE, qo=None, max_seq_len=128, max_q_len=1, dims=None, result=FAKE):
        d = dims if dims is not None else _dims()
        return lib.mla_decode_check_contract(bt, sl, qo, max_seq_len, max_q_len, 1, ctypes.byref(d), result, None)

    NULL, SHAPE, PAGE, QLEN, MIS = 1, 10, 3, 8, 6
    assert chk(bt=None) == NULL
    assert chk(sl=None) == NULL
    assert chk(result=None) == NULL
    assert lib.mla_decode_check_contract(FAKE, FAKE, None, 128, 1, 1, None, FAKE, None) == NULL
    assert chk(result=FAKE + 2) == MIS
    assert chk(dims=_dims(batch=0)) == SHAPE
    assert chk(dims=_dims(batch=1025)) == SHAPE
    assert chk(dims=_dims(num_pages=0)) == SHAPE
    assert chk(dims=_dims(block_table_stride=0)) == SHAPE
    assert chk(max_seq_len=0) == SHAPE
    assert chk(dims=_dims(page_size=48)) == PAGE
    assert chk(max_q_len=0) == QLEN
    assert chk(dims=_dims(total_q=0)) == QLEN
    assert chk(dims=_dims(q_len_fixed=0)) == QLEN
