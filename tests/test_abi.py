"""The C ABI on the CPU: the library loads, exports what the header declares,
and host-side validation returns the documented status before any launch.

No call here reaches a kernel: every call either fails validation or is
rejected on call order, both of which return before touching the device."""
import ctypes

import pytest

from recurrent_state_storage_amd import rss


def _cfg(**kw):
    base = dict(batch=4, nheads=8, headdim=64, dstate=128, ngroups=8, window=16, capacity=20,
                max_draft=4, in_dtype=rss.RSS_DTYPE_BF16, read_copy=rss.RSS_COPY_NONE,
                kind=rss.RSS_KIND_MAMBA2)
    base.update(kw)
    return rss.rss_config(**base)


def _fake_bufs(cfg, misalign=None, null=None):
    """Aligned fake device addresses: never dereferenced by bind."""
    names = [n for n, _ in rss.rss_buffers._fields_]
    vals = {n: 0x100000 * (i + 1) for i, n in enumerate(names)}
    if cfg.read_copy == rss.RSS_COPY_NONE:
        vals["ckpt_lo"] = None
    if misalign:
        vals[misalign] += 4
    if null:
        vals[null] = None
    return rss.rss_buffers(**vals)


def _bind(cfg, bufs):
    h = ctypes.c_void_p()
    st = rss.library().rss_layer_bind(ctypes.byref(cfg), ctypes.byref(bufs), ctypes.byref(h))
    return st, h.value


def test_library_exports_every_declared_symbol():
    lib = rss.library()
    syms = rss.declared_symbols()
    assert len(syms) >= 16
    for s in syms:
        assert hasattr(lib, s), s
    assert set(syms) == set(rss._SIGS), "binding and header disagree"


def test_version_and_status_strings():
    assert rss.rss_version() == 10600
    for s in range(7):
        assert rss.status_string(s)
    assert rss.status_string(99) == "unknown status"


def test_largest_shapes_within_the_lds_budget_are_accepted():
    ok = [dict(headdim=256, dstate=256, window=57, capacity=64, max_draft=7),
          dict(headdim=256, dstate=256, window=51, capacity=58, max_draft=7, in_dtype=rss.RSS_DTYPE_F32),
          dict(headdim=256, dstate=256, window=64, capacity=64, max_draft=0, in_dtype=rss.RSS_DTYPE_F32),
          dict(headdim=256, dstate=256, window=57, capacity=64, max_draft=7,
               read_copy=rss.RSS_COPY_BF16),
          dict(kind=rss.RSS_KIND_GDN, headdim=256, dstate=256, window=64, capacity=64, max_draft=0,
               in_dtype=rss.RSS_DTYPE_F32),
          dict(kind=rss.RSS_KIND_KDA, headdim=256, dstate=256, window=48, capacity=48, max_draft=0,
               in_dtype=rss.RSS_DTYPE_F32)]
    for kw in ok:
        out = rss.rss_sizes()
        assert rss.library().rss_buffer_sizes(ctypes.byref(_cfg(**kw)), ctypes.byref(out)) == rss.RSS_OK, kw


def test_largest_ring_per_sequence_is_accepted():
    # R H max(P, N) = 2^31 - 64 * 256 * 1 ... just below the 32-bit offset bound
    cfg = _cfg(batch=1, nheads=131071, ngroups=1, headdim=256, capacity=64, window=60)
    out = rss.rss_sizes()
    assert rss.library().rss_buffer_sizes(ctypes.byref(cfg), ctypes.byref(out)) == rss.RSS_OK
    assert out.ring_x == 64 * 131071 * 256 * 2


def test_buffer_sizes():
    cfg = _cfg()
    s = rss.rss_buffer_sizes(cfg)
    assert s.ckpt == 4 * 8 * 64 * 128 * 4
    assert s.ckpt_lo == 0
    assert s.ring_x == 4 * 8 * 20 * 64 * 2
    assert s.ring_B == 4 * 8 * 20 * 128 * 2
    assert s.ring_dl == 4 * 8 * 20 * 2 * 4
    assert s.ptr == 4 * 8 * 16 and s.A == 32 and s.dev_err == 4
    s2 = rss.rss_buffer_sizes(_cfg(read_copy=rss.RSS_COPY_BF16, in_dtype=rss.RSS_DTYPE_F32))
    assert s2.ckpt_lo == 4 * 8 * 64 * 128 * 2 and s2.ring_x == 4 * 8 * 20 * 64 * 4
    s3 = rss.rss_buffer_sizes(_cfg(read_copy=rss.RSS_STATE_BF16))     # bf16-only checkpoint
    assert s3.ckpt == 4 * 8 * 64 * 128 * 2 and s3.ckpt_lo == 0


@pytest.mark.parametrize("kw,status", [
    (dict(dstate=96), rss.RSS_E_SHAPE),
    (dict(dstate=8), rss.RSS_E_SHAPE),
    (dict(headdim=0), rss.RSS_E_SHAPE),
    (dict(headdim=257), rss.RSS_E_SHAPE),
    (dict(nheads=6, ngroups=4), rss.RSS_E_SHAPE),
    (dict(ngroups=0), rss.RSS_E_SHAPE),
    (dict(batch=-1), rss.RSS_E_SHAPE),
    (dict(window=0), rss.RSS_E_SHAPE),
    (dict(capacity=65, window=16), rss.RSS_E_SHAPE),
    (dict(capacity=19), rss.RSS_E_CAPACITY),
    (dict(max_draft=8, capacity=30), rss.RSS_E_CAPACITY),
    (dict(max_draft=-1), rss.RSS_E_CAPACITY),
    (dict(in_dtype=7), rss.RSS_E_DTYPE),
    (dict(read_copy=3), rss.RSS_E_DTYPE),
    (dict(kind=3), rss.RSS_E_INVALID),
    (dict(kind=rss.RSS_KIND_GDN, ngroups=4, max_draft=0, in_dtype=rss.RSS_DTYPE_F32), rss.RSS_E_SHAPE),
    (dict(kind=rss.RSS_KIND_GDN, max_draft=0), rss.RSS_E_DTYPE),
    (dict(kind=rss.RSS_KIND_GDN, max_draft=0, in_dtype=rss.RSS_DTYPE_F32,
          read_copy=rss.RSS_COPY_BF16), rss.RSS_E_DTYPE),
    (dict(kind=rss.RSS_KIND_GDN, in_dtype=rss.RSS_DTYPE_F32), rss.RSS_E_CAPACITY),
    (dict(kind=rss.RSS_KIND_GDN, max_draft=0, in_dtype=rss.RSS_DTYPE_F32,
          read_copy=rss.RSS_STATE_BF16), rss.RSS_E_DTYPE),
    # LDS budget (160 KiB per workgroup) at the largest shapes
    (dict(headdim=256, dstate=256, window=57, capacity=64, max_draft=7, in_dtype=rss.RSS_DTYPE_F32),
     rss.RSS_E_SHAPE),
    (dict(kind=rss.RSS_KIND_KDA, headdim=256, dstate=256, window=49, capacity=49, max_draft=0,
          in_dtype=rss.RSS_DTYPE_F32), rss.RSS_E_SHAPE),
    # one sequence's slot-major ring past 2^31 elements (R H max(P, N)): refused
    (dict(batch=1, nheads=131072, ngroups=1, headdim=256, capacity=64, window=60), rss.RSS_E_SHAPE),
])
def test_config_validation(kw, status):
    cfg = _cfg(**kw)
    out = rss.rss_sizes()
    assert rss.library().rss_buffer_sizes(ctypes.byref(cfg), ctypes.byref(out)) == status
    st, h = _bind(cfg, _fake_bufs(_cfg()))
    assert st == status and h is None


def test_bind_pointer_checks():
    cfg = _cfg()
    for name in ("ckpt", "ring_x", "ring_B", "ring_dl", "ptr", "A", "dev_err"):
        assert _bind(cfg, _fake_bufs(cfg, null=name))[0] == rss.RSS_E_INVALID
        assert _bind(cfg, _fake_bufs(cfg, misalign=name))[0] == rss.RSS_E_INVALID
    dual = _cfg(read_copy=rss.RSS_COPY_BF16)
    assert _bind(dual, _fake_bufs(cfg))[0] == rss.RSS_E_INVALID   # dual needs ckpt_lo
    st, h = _bind(dual, _fake_bufs(dual))
    assert st == rss.RSS_OK and h
    assert rss.library().rss_layer_free(h) == rss.RSS_OK
    assert rss.library().rss_layer_free(None) == rss.RSS_OK
    assert rss.library().rss_layer_bind(ctypes.byref(cfg), None, None) == rss.RSS_E_INVALID


def test_gdn_layer_calls_are_kind_checked():
    gcfg = _cfg(kind=rss.RSS_KIND_GDN, max_draft=0, in_dtype=rss.RSS_DTYPE_F32)
    s = rss.rss_buffer_sizes(gcfg)
    assert s.A == 0 and s.ring_x == 4 * 8 * 20 * 64 * 4 and s.ring_B == 4 * 8 * 20 * 128 * 4
    st, h = _bind(gcfg, _fake_bufs(gcfg, null="A"))        # A is not needed for GDN
    assert st == rss.RSS_OK
    lib = rss.library()
    A = 0x7000000
    try:
        assert lib.rss_decode_step(h, A, A, A, A, A, None) == rss.RSS_E_INVALID
        assert lib.rss_verify_k_tokens(h, 0, A, A, A, A, A, None) == rss.RSS_E_INVALID
        assert lib.rss_gdn_decode_step(h, None, A, A, A, A, A, None) == rss.RSS_E_INVALID
    finally:
        lib.rss_layer_free(h)
    st, h = _bind(_cfg(), _fake_bufs(_cfg()))
    try:
        assert lib.rss_gdn_decode_step(h, A, A, A, A, A, A, None) == rss.RSS_E_INVALID
    finally:
        lib.rss_layer_free(h)
    assert lib.rss_gdn_eager_step(ctypes.byref(gcfg), None, A, A, A, A, A, A, None) == rss.RSS_E_INVALID


def test_kda_layer_sizes_and_kind_checks():
    kcfg = _cfg(kind=rss.RSS_KIND_KDA, max_draft=0, in_dtype=rss.RSS_DTYPE_F32)
    s = rss.rss_buffer_sizes(kcfg)
    assert s.A == 0 and s.ring_dl == 4 * 8 * 20 * 128 * 4       # one log-gate row per entry
    st, h = _bind(kcfg, _fake_bufs(kcfg, null="A"))
    assert st == rss.RSS_OK
    lib = rss.library()
    A = 0x7000000
    try:
        assert lib.rss_gdn_decode_step(h, A, A, A, A, A, A, None) == rss.RSS_E_INVALID
        assert lib.rss_decode_step(h, A, A, A, A, A, None) == rss.RSS_E_INVALID
        assert lib.rss_kda_decode_step(h, A, None, A, A, A, A, None) == rss.RSS_E_INVALID
    finally:
        lib.rss_layer_free(h)
    st, h = _bind(_cfg(), _fake_bufs(_cfg()))
    try:
        assert lib.rss_kda_decode_step(h, A, A, A, A, A, A, None) == rss.RSS_E_INVALID
    finally:
        lib.rss_layer_free(h)
    assert lib.rss_kda_eager_step(ctypes.byref(kcfg), None, A, A, A, A, A, A, None) == rss.RSS_E_INVALID
    bad = _cfg(kind=rss.RSS_KIND_KDA, max_draft=0, in_dtype=rss.RSS_DTYPE_F32, ngroups=4)
    assert _bind(bad, _fake_bufs(kcfg))[0] == rss.RSS_E_SHAPE


def test_verify_fold_capacity_rules_return_before_launch():
    """R + K + 1 > 64, and grouped B rows without room for a window plus two
    rounds, are refused on the host (the fake pointers are never launched on)."""
    A = 0x7000000
    lib = rss.library()
    big = _cfg(window=50, capacity=60, max_draft=4)                   # 60 + 4 + 1 > 64
    st, h = _bind(big, _fake_bufs(big))
    try:
        assert lib.rss_verify_k_tokens_fold(h, 50, 4, A, A, A, A, A, None) == rss.RSS_E_CAPACITY
    finally:
        lib.rss_layer_free(h)
    grp = _cfg(ngroups=4, window=8, capacity=12, max_draft=4)          # needs 8 + 9 = 17
    st, h = _bind(grp, _fake_bufs(grp))
    try:
        assert lib.rss_verify_k_tokens_fold(h, 8, 4, A, A, A, A, A, None) == rss.RSS_E_CAPACITY
    finally:
        lib.rss_layer_free(h)


def test_call_order_and_argument_errors_return_before_launch():
    cfg = _cfg()
    st, h = _bind(cfg, _fake_bufs(cfg))
    assert st == rss.RSS_OK
    lib = rss.library()
    try:
        A = 0x7000000
        # rollback with no verify round pending
        assert lib.rss_rollback(h, A, None) == rss.RSS_E_ORDER
        # null / misaligned inputs
        assert lib.rss_decode_step(h, None, A, A, A, A, None) == rss.RSS_E_INVALID
        assert lib.rss_decode_step(h, A + 2, A, A, A, A, None) == rss.RSS_E_INVALID
        assert lib.rss_verify_k_tokens(h, 5, A, A, A, A, A, None) == rss.RSS_E_CAPACITY
        assert lib.rss_verify_k_tokens(h, -1, A, A, A, A, A, None) == rss.RSS_E_INVALID
        assert lib.rss_verify_k_tokens_fold(h, 0, 2, A, A, A, A, A, None) == rss.RSS_E_INVALID
        assert lib.rss_verify_k_tokens_fold(h, 16, 5, A, A, A, A, A, None) == rss.RSS_E_CAPACITY
        assert lib.rss_flush_checkpoint(h, 0, None) == rss.RSS_E_INVALID
        assert lib.rss_decode_flush_step(h, 0, A, A, A, A, A, None) == rss.RSS_E_INVALID
        assert lib.rss_decode_flush_step(h, 16, A, A, A + 8, A, A, None) == rss.RSS_E_INVALID
        assert lib.rss_decode_flush_step_each(h, None, A, A, A, A, A, None) == rss.RSS_E_INVALID
        assert lib.rss_decode_flush_step_each(h, A + 4, A, A, A, A, A, None) == rss.RSS_E_INVALID
        assert lib.rss_flush_checkpoint_each(h, None, None) == rss.RSS_E_INVALID
        assert lib.rss_rollback(h, None, None) == rss.RSS_E_INVALID
        assert lib.rss_init_state(h, A + 4, None) == rss.RSS_E_INVALID
        v = ctypes.c_int32()
        assert lib.rss_get_device_error(None, ctypes.byref(v), None) == rss.RSS_E_INVALID
        assert lib.rss_get_device_error(h, None, None) == rss.RSS_E_INVALID
        assert lib.rss_decode_step(None, A, A, A, A, A, None) == rss.RSS_E_INVALID
        # eager entry points
        assert lib.rss_eager_step(ctypes.byref(cfg), None, A, A, A, A, A, A, 1, None) == rss.RSS_E_INVALID
        assert lib.rss_eager_step(ctypes.byref(cfg), A, A, A, A, A, A, A, 0, None) == rss.RSS_E_INVALID
        assert lib.rss_eager_step(ctypes.byref(cfg), A, A, A, A, A, A, A, 9, None) == rss.RSS_E_INVALID
        bad = _cfg(dstate=48)
        assert lib.rss_eager_step(ctypes.byref(bad), A, A, A, A, A, A, A, 1, None) == rss.RSS_E_SHAPE
        assert lib.rss_eager_verify(ctypes.byref(cfg), A, None, 4, A, A, A, A, A, A, None) == rss.RSS_E_INVALID
        assert lib.rss_eager_verify(ctypes.byref(cfg), A, A, 8, A, A, A, A, A, A, None) == rss.RSS_E_INVALID
        b16 = _cfg(read_copy=rss.RSS_STATE_BF16)          # snapshot pools are fp32 only
        assert lib.rss_eager_verify(ctypes.byref(b16), A, A, 4, A, A, A, A, A, A, None) == rss.RSS_E_DTYPE
        bad_mode = _cfg(read_copy=5)
        assert lib.rss_eager_step(ctypes.byref(bad_mode), A, A, A, A, A, A, A, 1, None) == rss.RSS_E_DTYPE
    finally:
        lib.rss_layer_free(h)


def test_binding_rejects_host_tensors():
    import torch
    cfg = _cfg(batch=1, nheads=2, ngroups=2, headdim=16, dstate=16)
    with pytest.raises(ValueError):
        rss.rss_eager_step(cfg, torch.zeros(1, 2, 16, 16), torch.zeros(1, 1, 2, 16),
                           torch.zeros(1, 1, 2, 16), torch.zeros(1, 1, 2, 16), torch.zeros(1, 1, 2),
                           torch.zeros(2), torch.zeros(1, 1, 2, 16))


def test_calibration_calls_validate_before_launch():
    lib = rss.library()
    ok = ctypes.c_void_p(0x100000)
    odd = ctypes.c_void_p(0x100004)
    for st in (lib.rss_calib_read(None, 16, ok, 0, None), lib.rss_calib_read(odd, 16, ok, 0, None),
               lib.rss_calib_read(ok, 24, ok, 0, None), lib.rss_calib_read(ok, 16, None, 0, None),
               lib.rss_calib_read(ok, 16, ok, -1, None),
               lib.rss_calib_copy(ok, None, 16, 0, None), lib.rss_calib_copy(ok, odd, 16, 0, None),
               lib.rss_calib_copy(ok, ok, 8, 0, None),
               lib.rss_calib_write(None, 16, 0, None), lib.rss_calib_write(odd, 16, 0, None),
               lib.rss_calib_write(ok, 20, 0, None), lib.rss_calib_write(ok, 16, -2, None),
               lib.rss_calib_tiles(None, 32768, 4, ok, 16, 0, None), lib.rss_calib_tiles(odd, 32768, 4, ok, 16, 0, None),
               lib.rss_calib_tiles(ok, 12288, 4, ok, 16, 0, None), lib.rss_calib_tiles(ok, 32768, -1, ok, 16, 0, None),
               lib.rss_calib_tiles(ok, 32768, 4, None, 16, 0, None), lib.rss_calib_tiles(ok, 32768, 4, odd, 16, 0, None),
               lib.rss_calib_tiles(ok, 32768, 4, ok, 24, 0, None), lib.rss_calib_tiles(ok, 32768, 4, ok, 4112, 0, None),
               lib.rss_calib_tiles(ok, 32768, 4, ok, -16, 0, None), lib.rss_calib_tiles(ok, 32768, 4, ok, 16, 2, None),
               lib.rss_calib_tiles(ok, 32768, 4, ok, 16, -1, None)):
        assert st == rss.RSS_E_INVALID
    # zero bytes launch nothing
    assert lib.rss_calib_read(ok, 0, ok, 0, None) == rss.RSS_OK
    assert lib.rss_calib_copy(ok, ok, 0, 0, None) == rss.RSS_OK
    assert lib.rss_calib_write(ok, 0, 0, None) == rss.RSS_OK
    assert lib.rss_calib_tiles(ok, 32768, 0, ok, 16, 0, None) == rss.RSS_OK
    assert lib.rss_calib_tiles(ok, 32768, 0, ok, 32768, 0, None) == rss.RSS_OK   # tile copy
    assert lib.rss_calib_tiles(ok, 32768, 0, ok, 16, 1, None) == rss.RSS_OK     # the other order
    assert lib.rss_calib_tiles(ok, 32768, 4, None, 32768, 0, None) == rss.RSS_E_INVALID
