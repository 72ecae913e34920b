"""CPU-only checks of the C ABI: the library loads, exports every declared entry
point, its structs match the binding's layout, and host validation rejects bad
arguments before any GPU work (no compute call is made here)."""

import ctypes
import os
import re
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn_mi355x.h")
DEBUG_HEADER = os.path.join(ROOT, "include", "attn_mi355x_debug.h")

binding = pytest.importorskip("exact_tiled_attention_fa2_amd.binding")


def _lib():
    try:
        return binding.lib()
    except RuntimeError as e:  # not built
        pytest.fail(str(e))


def _declared_functions(header=HEADER):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*(attn_[a-z0-9_]+)\s*\(", text,
                       flags=re.M)
    return sorted(set(names))


def _exported(path):
    out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True, text=True,
                         check=True).stdout
    return set(re.findall(r" T (attn_[a-z0-9_]+)", out))


def test_library_exports_every_declared_function():
    h = _lib()
    names = _declared_functions()
    assert {"attn_fwd", "attn_fwd_varlen", "attn_fwd_kvcache", "attn_bwd", "attn_bwd_varlen"} <= set(names)
    for n in names:
        assert hasattr(h, n), f"{n} declared in the header but not exported"
    assert set(names) <= _exported(binding.LIB_PATH)


def test_debug_library_exports_both_headers():
    """The debug build exports every entry point of both headers; the release build exports none
    of the debug header's and reads no environment variable."""
    from exact_tiled_attention_fa2_amd import debug
    debug_names = set(_declared_functions(DEBUG_HEADER))
    assert {"attn_debug_set_variants", "attn_debug_last_block_k", "attn_fwd_stats"} <= debug_names
    h = debug.debug_lib()
    for n in set(_declared_functions()) | debug_names:
        assert hasattr(h, n), f"{n} not exported by the debug library"
    assert debug_names <= _exported(debug.DEBUG_LIB_PATH)
    assert not (debug_names & _exported(binding.LIB_PATH))
    imports = subprocess.run(["nm", "-D", "--undefined-only", binding.LIB_PATH], capture_output=True,
                             text=True, check=True).stdout
    assert "getenv" not in imports


def test_version_and_status_strings():
    h = _lib()
    assert h.attn_version() == 140
    for code in range(-9, 1):
        assert binding.status_string(code)
    assert binding.status_string(-1234) == "unknown status"


_LAYOUT_C = r"""
#include <stddef.h>
#include <stdio.h>
#include "attn_mi355x.h"
#define F(T, f) printf(#T " " #f " %zu\n", offsetof(T, f));
int main(void) {
  printf("attn_softmax_opts size %zu\n", sizeof(attn_softmax_opts));
  printf("attn_fwd_args size %zu\n", sizeof(attn_fwd_args));
  printf("attn_varlen_args size %zu\n", sizeof(attn_varlen_args));
  printf("attn_kvcache_args size %zu\n", sizeof(attn_kvcache_args));
  printf("attn_bwd_args size %zu\n", sizeof(attn_bwd_args));
  printf("attn_bwd_varlen_args size %zu\n", sizeof(attn_bwd_varlen_args));
  %FIELDS%
  return 0;
}
"""


def test_struct_layouts_match_binding():
    structs = {"attn_softmax_opts": binding.SoftmaxOpts, "attn_fwd_args": binding.FwdArgs,
               "attn_varlen_args": binding.VarlenArgs, "attn_kvcache_args": binding.KvcacheArgs,
               "attn_bwd_args": binding.BwdArgs, "attn_bwd_varlen_args": binding.BwdVarlenArgs}
    fields = "\n".join(f"F({c}, {f})" for c, py in structs.items() for f, _ in py._fields_)
    with tempfile.TemporaryDirectory() as d:
        src = os.path.join(d, "layout.c")
        exe = os.path.join(d, "layout")
        open(src, "w").write(_LAYOUT_C.replace("%FIELDS%", fields))
        subprocess.run(["gcc", "-std=c99", "-I", os.path.dirname(HEADER), src, "-o", exe], check=True)
        lines = subprocess.run([exe], capture_output=True, text=True, check=True).stdout.splitlines()
    for line in lines:
        name, field, value = line.split()
        py = structs[name]
        if field == "size":
            assert ctypes.sizeof(py) == int(value), name
        else:
            assert getattr(py, field).offset == int(value), (name, field)


def _fwd_args(**over):
    base = dict(dtype=1, batch=2, seqlen_q=64, seqlen_k=64, heads_q=4, heads_kv=2, head_dim=128,
                q=16, k=16, v=16, o=16, lse=None,
                q_batch_stride=64 * 4 * 128, q_row_stride=4 * 128, q_head_stride=128,
                k_batch_stride=64 * 2 * 128, k_row_stride=2 * 128, k_head_stride=128,
                v_batch_stride=64 * 2 * 128, v_row_stride=2 * 128, v_head_stride=128,
                o_batch_stride=64 * 4 * 128, o_row_stride=4 * 128, o_head_stride=128)
    opts = dict(softmax_scale=0.0, causal=0, window_left=-1, window_right=-1, softcap=0.0,
                rescale_threshold=-1.0)
    for k, v in over.items():
        if k in opts:
            opts[k] = v
        else:
            base[k] = v
    a = binding.FwdArgs()
    for k, v in base.items():
        setattr(a, k, v)
    a.opts = binding.SoftmaxOpts(**opts)
    return a


# Each case is rejected by host validation before anything touches the GPU.
_BAD_FWD = [
    (dict(dtype=7), binding.ATTN_E_UNSUPPORTED),
    (dict(head_dim=96), binding.ATTN_E_UNSUPPORTED),
    (dict(heads_q=3), binding.ATTN_E_HEADS),
    (dict(heads_kv=0), binding.ATTN_E_HEADS),
    (dict(window_left=-2), binding.ATTN_E_WINDOW),
    (dict(window_right=-5), binding.ATTN_E_WINDOW),
    (dict(batch=-1), binding.ATTN_E_SHAPE),
    (dict(seqlen_k=-3), binding.ATTN_E_SHAPE),
    (dict(q=None), binding.ATTN_E_NULL),
    (dict(o=None), binding.ATTN_E_NULL),
    (dict(k=None), binding.ATTN_E_NULL),
    (dict(q=24), binding.ATTN_E_ALIGN),
    (dict(k_row_stride=2 * 128 + 4), binding.ATTN_E_ALIGN),
    (dict(q_row_stride=1 << 24), binding.ATTN_E_ALIGN),
    (dict(lse=18), binding.ATTN_E_ALIGN),
    (dict(softcap=-1.0), binding.ATTN_E_ARG),
    (dict(softmax_scale=float("nan")), binding.ATTN_E_ARG),
    (dict(causal=2), binding.ATTN_E_ARG),
    (dict(rescale_threshold=15.5), binding.ATTN_E_ARG),
    (dict(rescale_threshold=float("inf")), binding.ATTN_E_ARG),
]


@pytest.mark.parametrize("over,code", _BAD_FWD, ids=[str(o) for o, _ in _BAD_FWD])
def test_attn_fwd_rejects_bad_arguments(over, code):
    h = _lib()
    assert h.attn_fwd(ctypes.byref(_fwd_args(**over)), None) == code


def test_null_args_and_empty_problems_launch_nothing():
    h = _lib()
    assert h.attn_fwd(None, None) == binding.ATTN_E_NULL
    assert h.attn_fwd_varlen(None, None, 0, None) == binding.ATTN_E_NULL
    assert h.attn_fwd_kvcache(None, None, 0, None) == binding.ATTN_E_NULL
    # No query rows: OK without touching any pointer (they are NULL here).
    assert h.attn_fwd(ctypes.byref(_fwd_args(batch=0, q=None, k=None, v=None, o=None)), None) == 0
    assert h.attn_fwd(ctypes.byref(_fwd_args(seqlen_q=0, q=None, k=None, v=None, o=None)), None) == 0
    va = binding.VarlenArgs(1, 3, 0, 0, 0, 0, 4, 4, 64)
    va.opts = binding.SoftmaxOpts(0.0, 0, -1, -1, 0.0, -1.0)
    assert h.attn_fwd_varlen(ctypes.byref(va), None, 0, None) == 0
    ka = binding.KvcacheArgs(1, 0, 1, 128, 8, 2, 128, 0)
    ka.opts = binding.SoftmaxOpts(0.0, 0, -1, -1, 0.0, -1.0)
    assert h.attn_fwd_kvcache(ctypes.byref(ka), None, 0, None) == 0


def test_varlen_validation():
    h = _lib()
    va = binding.VarlenArgs(1, 2, 100, 100, 64, 64, 4, 2, 128, 16, 16, 16, 16, None, None, 16,
                            512, 128, 256, 128, 256, 128, 512, 128)
    va.opts = binding.SoftmaxOpts(0.0, 1, -1, -1, 0.0, -1.0)
    assert h.attn_fwd_varlen(ctypes.byref(va), None, 0, None) == binding.ATTN_E_NULL  # cu_seqlens_q
    va.cu_seqlens_q = 16
    va.heads_q = 5
    assert h.attn_fwd_varlen(ctypes.byref(va), None, 0, None) == binding.ATTN_E_HEADS
    va.heads_q = 4
    va.total_q = -1
    assert h.attn_fwd_varlen(ctypes.byref(va), None, 0, None) == binding.ATTN_E_SHAPE


def test_kvcache_workspace_and_splits():
    h = _lib()
    # cfg: B=32, Sq=1, Hq=32, Hkv=8, Sk=32768, D=128, 16 splits
    need = binding.attn_kvcache_workspace_bytes(32, 1, 32, 128, 16)
    assert need == 16 * 32 * 32 * 1 * (128 + 1) * 4
    assert binding.attn_kvcache_workspace_bytes(32, 1, 32, 128, 1) == 0
    s = binding.attn_kvcache_num_splits(32, 1, 32, 8, 32768, 128)
    assert 1 < s <= 128            # never forced to 1 when the grid would be small
    assert binding.attn_kvcache_num_splits(1, 1, 8, 8, 64, 128) == 1
    assert binding.attn_kvcache_num_splits(0, 1, 8, 8, 64, 128) == 1
    ka = binding.KvcacheArgs(1, 32, 1, 32768, 32, 8, 128, 16, 16, 16, 16, None, 16, None,
                             32 * 128, 32 * 128, 128, 32768 * 8 * 128, 8 * 128, 128,
                             32768 * 8 * 128, 8 * 128, 128, 32 * 128, 32 * 128, 128)
    ka.opts = binding.SoftmaxOpts(0.0, 0, -1, -1, 0.0, -1.0)
    assert h.attn_fwd_kvcache(ctypes.byref(ka), None, 0, None) == binding.ATTN_E_WORKSPACE
    assert h.attn_fwd_kvcache(ctypes.byref(ka), 16, need - 1, None) == binding.ATTN_E_WORKSPACE
    ka.num_splits = 999
    assert h.attn_fwd_kvcache(ctypes.byref(ka), 16, need, None) == binding.ATTN_E_ARG


def test_kvcache_noalloc_validation():
    """The allocation-free kv-cache entry validates like attn_fwd_kvcache and rejects a call whose
    split partials exceed its static scratch -- all on the host, before any HIP call (fake device
    pointers here).  The scratch size matches the header's ATTN_NOALLOC_SCRATCH_BYTES."""
    h = _lib()
    ka = binding.KvcacheArgs(1, 32, 1, 32768, 32, 8, 128, 16, 16, 16, 16, None, 16, None,
                             32 * 128, 32 * 128, 128, 32768 * 8 * 128, 8 * 128, 128,
                             32768 * 8 * 128, 8 * 128, 128, 32 * 128, 32 * 128, 128)
    ka.opts = binding.SoftmaxOpts(0.0, 0, -1, -1, 0.0, -1.0)
    assert h.attn_fwd_kvcache_noalloc(None, None) == binding.ATTN_E_NULL
    # 128 splits of 32 x 32 rows need 128 * 1024 * 129 * 4 B = 64.5 MiB > 64 MiB
    ka.num_splits = 128
    assert binding.attn_kvcache_workspace_bytes(32, 1, 32, 128, 128) > binding.ATTN_NOALLOC_SCRATCH_BYTES
    assert h.attn_fwd_kvcache_noalloc(ctypes.byref(ka), None) == binding.ATTN_E_WORKSPACE
    ka.num_splits = 999
    assert h.attn_fwd_kvcache_noalloc(ctypes.byref(ka), None) == binding.ATTN_E_ARG
    ka.num_splits, ka.q = 16, 24
    assert h.attn_fwd_kvcache_noalloc(ctypes.byref(ka), None) == binding.ATTN_E_ALIGN
    ka.q, ka.heads_q = 16, 30
    assert h.attn_fwd_kvcache_noalloc(ctypes.byref(ka), None) == binding.ATTN_E_HEADS
    ka.heads_q, ka.batch = 32, 0
    assert h.attn_fwd_kvcache_noalloc(ctypes.byref(ka), None) == 0       # empty: nothing launched
    with tempfile.TemporaryDirectory() as d:
        src, exe = os.path.join(d, "c.c"), os.path.join(d, "c")
        open(src, "w").write('#include <stdio.h>\n#include "attn_mi355x.h"\n'
                             'int main(void) { printf("%zu\\n", ATTN_NOALLOC_SCRATCH_BYTES); return 0; }\n')
        subprocess.run(["gcc", "-std=c99", "-I", os.path.dirname(HEADER), src, "-o", exe], check=True)
        out = subprocess.run([exe], capture_output=True, text=True, check=True).stdout
    assert int(out) == binding.ATTN_NOALLOC_SCRATCH_BYTES


def test_kvcache_paged_validation():
    """Page tables are checked on the host before any launch (fake device pointers here)."""
    h = _lib()
    ka = binding.KvcacheArgs(1, 2, 1, 512, 8, 2, 128, 1, 16, 16, 16, None, 16, None,
                             8 * 128, 8 * 128, 128, 64 * 2 * 128, 2 * 128, 128,
                             64 * 2 * 128, 2 * 128, 128, 8 * 128, 8 * 128, 128)
    ka.opts = binding.SoftmaxOpts(0.0, 0, -1, -1, 0.0, -1.0)
    ka.block_table, ka.block_table_stride, ka.page_block_size, ka.num_pages = 16, 8, 64, 20
    def call():
        return h.attn_fwd_kvcache(ctypes.byref(ka), None, 0, None)
    ka.page_block_size = 96                      # not a multiple of 64
    assert call() == binding.ATTN_E_ARG
    ka.page_block_size = 0
    assert call() == binding.ATTN_E_ARG
    ka.page_block_size = 64
    ka.reserved0 = 1
    assert call() == binding.ATTN_E_ARG
    ka.reserved0 = 0
    ka.block_table_stride = 7                    # 7 * 64 < seqlen_k = 512
    assert call() == binding.ATTN_E_SHAPE
    ka.block_table_stride = 8
    ka.num_pages = 0
    assert call() == binding.ATTN_E_SHAPE
    ka.num_pages = 20
    ka.block_table = 18                          # not 4-byte aligned
    assert call() == binding.ATTN_E_ALIGN


def test_alibi_validation():
    """ALiBi slopes are checked on the host (fake device pointers, no launch)."""
    h = _lib()
    a = _fwd_args()
    a.opts.alibi_slopes = 18                     # not 4-byte aligned
    assert h.attn_fwd(ctypes.byref(a), None) == binding.ATTN_E_ALIGN
    a.opts.alibi_slopes = 16
    a.opts.alibi_batch_stride = -1
    assert h.attn_fwd(ctypes.byref(a), None) == binding.ATTN_E_ARG



def _bwd_args(**over):
    """A valid dense backward argument block with fake (aligned) device pointers."""
    b, sq, sk, hq, hkv, d = 2, 64, 64, 4, 2, 128
    a = binding.BwdArgs()
    vals = dict(dtype=1, batch=b, seqlen_q=sq, seqlen_k=sk, heads_q=hq, heads_kv=hkv, head_dim=d,
                q=16, k=16, v=16, o=16, dout=16, lse=16, dq=16, dk=16, dv=16)
    for t, h in (("q", hq), ("o", hq), ("do", hq), ("dq", hq), ("k", hkv), ("v", hkv), ("dk", hkv), ("dv", hkv)):
        s = sq if h == hq else sk
        vals[f"{t}_batch_stride"] = s * h * d
        vals[f"{t}_row_stride"] = h * d
        vals[f"{t}_head_stride"] = d
    opts = dict(softmax_scale=0.0, causal=1, window_left=-1, window_right=-1, softcap=0.0,
                rescale_threshold=-1.0)
    for k, v in over.items():
        if k in opts:
            opts[k] = v
        else:
            vals[k] = v
    for k, v in vals.items():
        setattr(a, k, v)
    a.opts = binding.SoftmaxOpts(**opts)
    return a


_BAD_BWD = [
    (dict(head_dim=96), binding.ATTN_E_UNSUPPORTED),
    (dict(dtype=3), binding.ATTN_E_UNSUPPORTED),
    (dict(heads_q=3), binding.ATTN_E_HEADS),
    (dict(seqlen_q=-1), binding.ATTN_E_SHAPE),
    (dict(dout=None), binding.ATTN_E_NULL),
    (dict(lse=None), binding.ATTN_E_NULL),
    (dict(dk=None), binding.ATTN_E_NULL),
    (dict(dq=24), binding.ATTN_E_ALIGN),
    (dict(dv_row_stride=2 * 128 + 2), binding.ATTN_E_ALIGN),
    (dict(lse=18), binding.ATTN_E_ALIGN),
    (dict(window_left=-3), binding.ATTN_E_WINDOW),
    (dict(softcap=-2.0), binding.ATTN_E_ARG),
]


@pytest.mark.parametrize("over,code", _BAD_BWD, ids=[str(o) for o, _ in _BAD_BWD])
def test_attn_bwd_rejects_bad_arguments(over, code):
    h = _lib()
    need = binding.attn_bwd_workspace_bytes(2, 64, 4)
    assert h.attn_bwd(ctypes.byref(_bwd_args(**over)), 16, need, None) == code


def test_bwd_workspace_and_empty_problems():
    h = _lib()
    need = binding.attn_bwd_workspace_bytes(2, 64, 4)
    assert need == 2 * 64 * 4 * 4
    assert binding.attn_bwd_workspace_bytes(0, 64, 4) == 0
    assert binding.attn_bwd_varlen_workspace_bytes(1000, 8) == 1000 * 8 * 4
    a = _bwd_args()
    assert h.attn_bwd(ctypes.byref(a), None, 0, None) == binding.ATTN_E_WORKSPACE
    assert h.attn_bwd(ctypes.byref(a), 16, need - 4, None) == binding.ATTN_E_WORKSPACE
    assert h.attn_bwd(ctypes.byref(a), 24, need, None) == binding.ATTN_E_WORKSPACE   # misaligned
    assert h.attn_bwd(None, None, 0, None) == binding.ATTN_E_NULL
    assert h.attn_bwd_varlen(None, None, 0, None) == binding.ATTN_E_NULL
    empty = _bwd_args(batch=0, q=None, k=None, v=None, o=None, dout=None, lse=None, dq=None, dk=None, dv=None)
    assert h.attn_bwd(ctypes.byref(empty), None, 0, None) == 0
    va = binding.BwdVarlenArgs(1, 3, 0, 0, 0, 0, 4, 4, 64)
    va.opts = binding.SoftmaxOpts(0.0, 0, -1, -1, 0.0, -1.0)
    assert h.attn_bwd_varlen(ctypes.byref(va), None, 0, None) == 0
    va.total_q, va.total_k, va.max_seqlen_q, va.max_seqlen_k = 10, 10, 5, 5
    assert h.attn_bwd_varlen(ctypes.byref(va), None, 0, None) == binding.ATTN_E_NULL  # cu_seqlens
