"""Host-side checks of the C ABI: the library loads, exports every entry point
that include/locks.h declares, reports the documented slot sizes, and rejects
invalid arguments before enqueueing anything (no GPU needed: every call here
returns from host validation)."""
import ctypes
import os
import re

import pytest

from kv_cache_page_amd import locks as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "locks.h")).read()
    return sorted(set(re.findall(r"\b(locks_[a-z_]+)\s*\(", src)))


def test_exports_every_declared_symbol():
    names = _declared()
    assert set(names) == set(L.ENTRY_POINTS)
    lib = ctypes.CDLL(L._LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def test_slot_sizes():
    assert L.slot_bytes(L.Dims(8, 4, 8)) == 818 and L.slot_stride(L.Dims(8, 4, 8)) == 896
    assert L.slot_bytes(L.Dims(8, 4, 4)) == 490 and L.slot_bytes(L.Dims(8, 4, 16)) == 1474
    for r in range(1, 17):
        assert L.slot_bytes(L.Dims(8, 4, r)) == 64 * r + 16 * r + 128 + 2 * (r + 17)
        assert L.slot_stride(L.Dims(8, 4, r)) % 128 == 0


def test_invalid_dims_rejected():
    assert L.slot_bytes(L.Dims(8, 3, 8)) == 0            # group size 3 unsupported
    assert L.slot_bytes(L.Dims(8, 4, 17)) == 0           # rank > page size
    assert L.slot_bytes(L.Dims(8, 4, 8, head_dim=64)) == 0
    assert L.slot_bytes(L.Dims(0, 4, 8)) == 0
    assert L.workspace_bytes(L.Dims(8, 4, 8), 1, 8192, 1) == 0   # budget < 2
    assert L.workspace_bytes(L.Dims(8, 4, 8), 1, 1 << 17, 128) == 0  # too many pages
    assert L.workspace_bytes(L.Dims(8, 4, 8), 1, 8192, 128) > 0


def test_status_codes_before_launch():
    d = L.Dims(8, 4, 8)
    bd = ctypes.byref(d)
    bad = L.Dims(8, 3, 8)
    fake = ctypes.c_void_p(256)  # never dereferenced: every call below fails validation
    # build: negative count, null pool, bad dims, zero-sized pool
    assert L._build(bd, fake, 16, fake, -1, fake, None) == L.ERR_INVALID_ARG
    assert L._build(bd, None, 16, fake, 4, fake, None) == L.ERR_INVALID_ARG
    assert L._build(ctypes.byref(bad), fake, 16, fake, 4, fake, None) == L.ERR_UNSUPPORTED
    assert L._build(bd, fake, 0, fake, 4, fake, None) == L.ERR_INVALID_ARG
    assert L._build(bd, fake, 16, fake, 0, fake, None) == L.OK          # nothing to do
    assert L._build(bd, ctypes.c_void_p(258), 16, fake, 4, fake, None) == L.ERR_INVALID_ARG
    # score/select: budget < 2, null outputs, undersized workspace
    args = [fake, fake, 16, fake, fake, fake, 1, 8, 4, fake, fake, None, fake, 1 << 20, None]
    a = list(args); a[8] = 1
    assert L._score_select(bd, *a) == L.ERR_INVALID_ARG
    a = list(args); a[9] = None
    assert L._score_select(bd, *a) == L.ERR_INVALID_ARG
    a = list(args); a[13] = 16
    assert L._score_select(bd, *a) == L.ERR_WORKSPACE
    a = list(args); a[12] = None
    assert L._score_select(bd, *a) == L.ERR_WORKSPACE
    a = list(args); a[6] = -1
    assert L._score_select(bd, *a) == L.ERR_INVALID_ARG
    a = list(args); a[6] = 0
    assert L._score_select(bd, *a) == L.OK                                # empty batch
    # attention: null out, undersized workspace
    aargs = [fake, fake, fake, 16, fake, fake, fake, fake, 1, 8, 4, fake, None, fake, 1 << 20, None]
    a = list(aargs); a[11] = None
    assert L._sparse_attn(bd, *a) == L.ERR_INVALID_ARG
    a = list(aargs); a[14] = 8
    assert L._sparse_attn(bd, *a) == L.ERR_WORKSPACE
    # append / build_filled
    assert L._append(bd, None, fake, fake, fake, 16, fake, fake, 1, 8, None) == L.ERR_INVALID_ARG
    assert L._build_filled(bd, fake, 16, fake, fake, -2, 8, fake, None) == L.ERR_INVALID_ARG


def test_status_strings():
    for s in (L.OK, L.ERR_INVALID_ARG, L.ERR_UNSUPPORTED, L.ERR_WORKSPACE, L.ERR_HIP):
        assert L.status_string(s) and L.status_string(s) != "unknown status"
    with pytest.raises(L.LocksError):
        L._check(L.ERR_WORKSPACE, "x")


def test_kernel_fingerprint_does_not_depend_on_the_checkout_path(tmp_path):
    """bench.py reports counter traffic only while a kernel's fingerprint equals
    the one recorded beside its counters; the fingerprint must therefore be the
    same for the same sources wherever the repository sits."""
    import shutil
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    dst = os.path.join(str(tmp_path), "elsewhere")
    shutil.copytree(root, dst, ignore=shutil.ignore_patterns(
        ".git", "_work", "gpurun_out", "_build", "*.so", "__pycache__", "profiles"))
    code = "import bench; print(bench.kernel_fingerprint('step'), bench.kernel_fingerprint('score'))"
    here = subprocess.run([sys.executable, "-c", code], cwd=root, capture_output=True, text=True,
                          check=True).stdout
    there = subprocess.run([sys.executable, "-c", code], cwd=dst, capture_output=True, text=True,
                           check=True).stdout
    assert here == there and len(here.split()) == 2


def test_decode_step_rejects_before_launch():
    """locks_decode_step validates everything on the host first (fake device
    pointers: none of these calls may reach a launch). The 17000-page table
    takes the separate launches, whose selection fits in the workspace, so a
    workspace one byte short is rejected, and NULL selection outputs are
    accepted by validation (they are optional on every path)."""
    d = L.Dims(2, 4, 8)
    fake = ctypes.c_void_p(256)
    host_lens = (ctypes.c_int32 * 2)(17000 * 16 - 3, 300)
    need = L.workspace_bytes(d, 2, 17000, 64)
    assert need > 0

    def call(**kw):
        a = dict(q=fake, k_new=fake, v_new=fake, k_pool=fake, v_pool=fake, summ=fake, nb=40000,
                 table=fake, lens=fake, lens_host=ctypes.cast(host_lens, ctypes.c_void_p),
                 budgets=fake, S=2, MP=17000, KB=64, out=fake, lse=None, sel=None, cnt=None,
                 flags=0, ws=fake, ws_bytes=need - 1)
        a.update(kw)
        return L._decode_step(ctypes.byref(d), a["q"], a["k_new"], a["v_new"], a["k_pool"],
                              a["v_pool"], a["summ"], a["nb"], a["table"], a["lens"],
                              a["lens_host"], a["budgets"], a["S"], a["MP"], a["KB"], a["out"],
                              a["lse"], a["sel"], a["cnt"], a["flags"], a["ws"], a["ws_bytes"], None)

    assert call() == L.ERR_WORKSPACE                       # one byte short, NULL selection outputs
    assert call(ws=None, ws_bytes=need) == L.ERR_WORKSPACE
    assert call(sel=fake) == L.ERR_INVALID_ARG              # only one of sel_pages / sel_count
    assert call(out=None) == L.ERR_INVALID_ARG
    assert call(k_new=ctypes.c_void_p(264)) == L.ERR_INVALID_ARG   # not 16-byte aligned
    assert call(MP=70000) == L.ERR_UNSUPPORTED
    assert call(KB=1) == L.ERR_INVALID_ARG
    assert call(flags=2, ws_bytes=need) == L.ERR_INVALID_ARG  # unknown flag bit
    assert call(S=0) == L.OK                                # empty batch: nothing to do


def test_host_pool_argument_checks():
    """locks_host_pool_alloc / _free validation (no allocation is attempted)."""
    hp, dp = ctypes.c_void_p(123), ctypes.c_void_p(456)
    assert L._host_alloc(0, ctypes.byref(hp), ctypes.byref(dp)) == L.ERR_INVALID_ARG
    assert L._host_alloc(4096, None, ctypes.byref(dp)) == L.ERR_INVALID_ARG
    assert L._host_alloc(4096, ctypes.byref(hp), None) == L.ERR_INVALID_ARG
    assert L._host_free(None) == L.OK


def test_basis_width_and_merge_rule_dims():
    """The precision ablation's slot sizes, and invalid widths and rules."""
    assert L.slot_bytes(L.Dims(8, 4, 8, basis_bits=8)) == 1330
    assert L.slot_stride(L.Dims(8, 4, 8, basis_bits=8)) == 1408
    assert L.slot_bytes(L.Dims(8, 4, 8, basis_bits=2)) == 562
    assert L.slot_stride(L.Dims(8, 4, 8, basis_bits=2)) == 640
    assert L.slot_bytes(L.Dims(8, 4, 16, basis_bits=8)) == 16 * 128 + 256 + 128 + 2 * 33
    assert L.slot_bytes(L.Dims(8, 4, 8, basis_bits=4)) == L.slot_bytes(L.Dims(8, 4, 8)) == 818
    assert L.slot_bytes(L.Dims(8, 4, 8, basis_bits=3)) == 0
    assert L.slot_bytes(L.Dims(8, 4, 6, basis_bits=8)) == 0        # ablation ranks 4, 8, 16
    assert L.slot_bytes(L.Dims(8, 4, 6, basis_bits=4)) > 0
    for rule in ("share", "max", "mass", "per_head"):
        assert L.slot_bytes(L.Dims(8, 4, 8, merge_rule=rule)) == 818
    assert L.slot_bytes(L.Dims(8, 4, 8, merge_rule=4)) == 0
    assert L.slot_bytes(L.Dims(8, 4, 8, merge_rule=-1)) == 0


def test_per_head_rule_sizes_its_arrays_by_query_head():
    """LOCKS_MERGE_PER_HEAD: the workspace is that of num_kv_heads x
    group_size heads of one query head each (the selection rows and the
    mailboxes grow by G, the page scores stay the same size)."""
    H, G, MP, KB = 8, 4, 2048, 64
    shared = L.Dims(H, G, 8)
    per = L.Dims(H, G, 8, merge_rule="per_head")
    view = L.Dims(H * G, 1, 8)
    assert L.workspace_bytes(per, 2, MP, KB) == L.workspace_bytes(view, 2, MP, KB)
    assert L.workspace_bytes(per, 2, MP, KB) > L.workspace_bytes(shared, 2, MP, KB)
    assert L.selection_heads(per) == H * G and L.selection_heads(shared) == H
    # more KV heads than a view of int32 heads can hold
    assert L.workspace_bytes(L.Dims(2 ** 30, 4, 8, merge_rule="per_head"), 1, MP, KB) == 0
