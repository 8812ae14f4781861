"""The C ABI without a GPU: the library loads, exports every function the
header declares, and rejects invalid arguments before touching the device."""
import ctypes
import os
import subprocess

import pytest

import beam_search_step_amd as bs


def test_library_exports_every_declared_function():
    names = bs.declared_functions()
    assert len(names) == 25
    lib = bs.library()
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, f"not exported: {missing}"


def test_exports_match_header_exactly():
    out = subprocess.run(["nm", "-D", "--defined-only", bs.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = sorted({ln.split()[-1] for ln in out.splitlines() if " T bs_" in ln})
    assert exported == bs.declared_functions()
    # no other function leaves the library (helpers have internal linkage)
    others = [ln.split()[-1] for ln in out.splitlines()
              if ln.split()[-2] in ("T", "W") and not ln.split()[-1].startswith("bs_")]
    assert not others, f"exported helpers: {others}"


def test_library_is_built_for_gfx950():
    with open(bs.LIB_PATH, "rb") as f:
        blob = f.read()
    assert b"amdgcn-amd-amdhsa--gfx950" in blob


def test_strerror():
    assert bs.bs_strerror(bs.BS_OK) == "ok"
    assert bs.bs_strerror(bs.BS_EINVAL) == "invalid argument"
    assert bs.bs_strerror(bs.BS_ESTATE).startswith("call not valid")
    assert bs.bs_strerror(12345) == "unknown status"


def _cfg(**kw):
    base = dict(batch=2, beam=4, vocab=100, max_steps=8, eos_id=3, pad_id=-1, logits_dtype=0,
                lp=1, alpha=0.6, stop=1, num_return=1, tile_elems=0)
    base.update(kw)
    return bs.bs_config(**base)


@pytest.mark.parametrize("kw", [
    dict(batch=0), dict(beam=0), dict(beam=17), dict(vocab=0), dict(max_steps=0),
    dict(logits_dtype=2), dict(lp=3), dict(stop=3), dict(num_return=0), dict(num_return=5),
    dict(tile_elems=8), dict(alpha=float("nan")), dict(alpha=float("inf")), dict(beam=16, vocab=2 ** 27), dict(select=2),
    dict(batch=16384, beam=4), dict(batch=65536, beam=1),
])
def test_create_rejects_invalid_config(kw):
    h = ctypes.c_void_p(123)
    rc = bs.library().bs_create(ctypes.byref(_cfg(**kw)), None, ctypes.byref(h))
    assert rc == bs.BS_EINVAL
    assert h.value is None


def test_null_arguments_are_rejected():
    L = bs.library()
    assert L.bs_create(None, None, None) == bs.BS_EINVAL
    assert L.bs_step(None, None, 0, None, None, None, None) == bs.BS_EINVAL
    assert L.bs_reorder_kv(None, None, 0) == bs.BS_EINVAL
    assert L.bs_finalize(None, None, None, None) == bs.BS_EINVAL
    assert L.bs_reset(None) == bs.BS_EINVAL
    assert L.bs_verify(None, None, 0, None, None, None) == bs.BS_EINVAL
    assert L.bs_verify_noalloc(None, None, 0, 1, 1, 10, 10, None, None, None) == bs.BS_EINVAL
    assert L.bs_state_size(None, None) == bs.BS_EINVAL
    assert L.bs_state_save(None, None, 0) == bs.BS_EINVAL
    assert L.bs_state_load(None, None, 0) == bs.BS_EINVAL
    h = ctypes.c_void_p()
    assert L.bs_verify_create(0, 8, 100, 0, None, ctypes.byref(h)) == bs.BS_EINVAL
    assert L.bs_verify_create(2, 65, 100, 0, None, ctypes.byref(h)) == bs.BS_EINVAL
    assert L.bs_verify_create(1025, 64, 100, 0, None, ctypes.byref(h)) == bs.BS_EINVAL
    assert L.bs_kv_paged_create(None, 16, 64, ctypes.byref(h)) == bs.BS_EINVAL
    assert L.bs_kv_paged_reset(None) == bs.BS_EINVAL
    assert L.bs_kv_paged_table(None, None, None) == bs.BS_EINVAL
    assert L.bs_kv_paged_reorder(None, None, 1) == bs.BS_EINVAL
    assert L.bs_kv_paged_status(None, None, None) == bs.BS_EINVAL
    L.bs_destroy(None)
    L.bs_verify_destroy(None)
    L.bs_kv_paged_destroy(None)


def test_config_struct_layout_matches_header():
    # offsets of the C struct on x86-64: eight int32, a double, five int32
    # (padded to a multiple of 8)
    assert ctypes.sizeof(bs.bs_config) == 64
    assert bs.bs_config.alpha.offset == 32
    assert bs.bs_config.tile_elems.offset == 48
    assert bs.bs_config.prune.offset == 52
    assert bs.bs_config.select.offset == 56
    assert ctypes.sizeof(bs.bs_kv_desc) == 48
    # int32 then a pointer (8-aligned), then three int64
    assert ctypes.sizeof(bs.bs_kv_pool) == 40
    assert bs.bs_kv_pool.block_stride.offset == 16


def test_binding_checks_tensor_layouts():
    """The wrappers check a tensor before its pointer reaches a kernel: the
    library cannot see sizes, so too few rows or columns, non-contiguous rows,
    unevenly spaced rows or a wrong dtype would otherwise be read or written
    out of bounds."""
    import torch
    import beam_search_step_amd as bs
    f32 = {"float32"}
    ok = torch.zeros(12, 100)
    assert bs._rows(ok, "x", 12, 100, f32, need_gpu=False) == 100
    assert bs._rows(ok.view(3, 4, 100), "x", 12, 100, f32, need_gpu=False) == 100
    assert bs._rows(torch.zeros(12, 128)[:, :100], "x", 12, 100, f32, need_gpu=False) == 128
    assert bs._rows(torch.zeros(1, 100), "x", 1, 100, f32, need_gpu=False) == 100
    bad = [torch.zeros(11, 100),                       # too few rows
           torch.zeros(12, 99),                        # rows too short
           torch.zeros(100, 12).t(),                   # columns not contiguous
           torch.zeros(3, 5, 100)[:, :4],              # [a, b, n] rows unevenly spaced
           torch.zeros(12, 100, dtype=torch.float64),  # wrong dtype
           torch.zeros(1200)]                          # not rows
    for t in bad:
        with pytest.raises(ValueError):
            bs._rows(t, "x", 12, 100, f32, need_gpu=False)
    with pytest.raises(ValueError):                    # a CPU tensor
        bs._rows(ok, "x", 12, 100, f32)
