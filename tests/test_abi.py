"""The C ABI library loads on a machine without a GPU, exports every function
include/moe_i4.h declares, and rejects bad arguments on the host before it
touches a device.  CPU only (no compute calls)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_i4.h")


def _declared():
    text = open(HEADER, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(moe_[a-z_0-9]+)\s*\(", text, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    import int4_expert_gemv_moe_amd as moe
    return moe.lib()


def test_header_declares_the_five_block_calls():
    names = _declared()
    for n in ("moe_router_topk", "moe_quant_act_i8", "moe_expert_swiglu_i4", "moe_layer_forward",
              "moe_layer_forward_batch"):
        assert n in names
    assert len(names) >= 10


def test_every_declared_symbol_is_exported(lib):
    for n in _declared():
        assert hasattr(lib, n), n


def test_status_strings(lib):
    assert lib.moe_status_str(0) == b"ok"
    assert lib.moe_status_str(-4) == b"workspace too small"
    assert lib.moe_status_str(-99) == b"unknown status"


def test_workspace_bytes_host_logic():
    import int4_expert_gemv_moe_amd as moe
    L = moe.lib()
    cfg = moe.config(6144, 2048, 256, 8)
    sizes = [L.moe_workspace_bytes(ctypes.byref(cfg), s, 1) for s in (1, 2, 64, 2048)]
    assert all(a < b for a, b in zip(sizes, sizes[1:]))
    # the union path stages (K+1) f32 rows of D per token
    assert sizes[-1] >= 2048 * 9 * 6144 * 4
    assert L.moe_workspace_bytes(ctypes.byref(cfg), 0, 0) == 0
    assert L.moe_workspace_bytes(ctypes.byref(cfg), 1, 7) == 0
    for bad in (moe.config(6000, 2048, 256, 8), moe.config(6144, 2048, 4, 8),
                moe.config(6144, 2048, 256, 65), moe.config(6144, 2048, 2000, 8),
                moe.config(6144, 2048, 256, 8, n_shared=2), moe.config(6144, 30, 256, 8),
                moe.config(6144, 2048, 256, 8, expert_topp=-0.1),
                moe.config(6144, 2048, 256, 8, expert_topp=1.5),
                moe.config(6144, 2048, 256, 8, expert_topp=float("nan"))):
        assert L.moe_workspace_bytes(ctypes.byref(bad), 1, 0) == 0


def test_host_validation_before_device():
    import int4_expert_gemv_moe_amd as moe
    L = moe.lib()
    cfg = moe.config(256, 128, 8, 2)
    layer = moe.LayerC()
    # null layer / x / out -> invalid argument, decided on the host
    assert L.moe_layer_forward(ctypes.byref(cfg), None, None, 1, None, 0, None, None, 0, None) == -1
    assert L.moe_layer_forward_batch(ctypes.byref(cfg), ctypes.byref(layer), None, 1, None, 0, None,
                                     None, 0, None) == -1
    bad = moe.config(250, 128, 8, 2)
    assert L.moe_layer_forward(ctypes.byref(bad), ctypes.byref(layer), None, 1, None, 0, None,
                               None, 0, None) == -2
    assert L.moe_pack_int4(None, 4, 8, None, None, None) == -1
    buf = ctypes.create_string_buffer(64)
    assert L.moe_pack_int4(buf, 4, 7, buf, buf, None) == -2  # odd C
    assert L.moe_quant_act_i8(buf, 5, 1, 8, buf, buf, None) == -1  # unknown dtype
    assert L.moe_quant_act_i8(buf, 0, 1, 12, buf, buf, None) == -2  # D % 8
    assert L.moe_rmsnorm(None, None, 1, 8, 1e-5, None, None) == -1


def test_given_routing_and_tier_host_checks():
    import int4_expert_gemv_moe_amd as moe
    L = moe.lib()
    cfg = moe.config(256, 128, 8, 2)
    layer = moe.LayerC()
    buf = ctypes.create_string_buffer(256)
    a16 = ctypes.addressof(buf) + (-ctypes.addressof(buf)) % 16
    for fn in (L.moe_layer_forward_routed, L.moe_layer_forward_batch_routed):
        # routing pointers: missing -> invalid argument, misaligned -> alignment
        assert fn(ctypes.byref(cfg), ctypes.byref(layer), None, 1, None, None, None, 0, None, 0,
                  None) == -1
        assert fn(ctypes.byref(cfg), ctypes.byref(layer), None, 1, a16, None, None, 0, None, 0,
                  None) == -1
        assert fn(ctypes.byref(cfg), ctypes.byref(layer), None, 1, a16 + 2, a16, None, 0, None, 0,
                  None) == -3
        assert fn(ctypes.byref(cfg), ctypes.byref(layer), None, 1, a16, a16 + 1, None, 0, None, 0,
                  None) == -3
    # the tier's copies: slab size must be a non-zero multiple of 16
    ids = (ctypes.c_int32 * 1)(0)
    assert L.moe_tier_fetch(a16, a16, 0, ids, ids, ids, 1, None) == -3
    assert L.moe_tier_fetch(a16, a16, 24, ids, ids, ids, 1, None) == -3
    assert L.moe_tier_fetch(None, a16, 32, ids, ids, ids, 1, None) == -1
    # a layout needs D and I multiples of 32
    lay = moe.SlabLayout()
    assert L.moe_slab_layout_of(ctypes.byref(moe.config(256, 48, 8, 2)), ctypes.byref(lay)) == -2
    # a tiered call: missing objects, or flags other than accumulate, are refused
    t = L.moe_tier_create(1, 8, 4)
    z = ctypes.c_size_t(0)
    assert L.moe_tier_forward(None, 0, ctypes.byref(cfg), ctypes.byref(layer), a16, a16, 32, a16, 1,
                              a16, 0, 0, a16, None, a16, 0, a16, 0, None) == -1
    assert L.moe_tier_forward(t, 0, ctypes.byref(cfg), ctypes.byref(layer), a16, a16, 32, a16, 1,
                              a16, 2, 0, a16, None, a16, 0, a16, 0, None) == -1
    # before any slot is mapped: the slab size must be a multiple of 16 that
    # holds the shape's layout, and every slot must be an index of the slot
    # stack (at most E slots)
    big = 1 << 40
    lay = moe.SlabLayout()
    assert L.moe_slab_layout_of(ctypes.byref(cfg), ctypes.byref(lay)) == 0
    hb = ctypes.create_string_buffer(1024)
    a256 = ctypes.addressof(hb) + (-ctypes.addressof(hb)) % 256
    rl = moe.LayerC(a256, a256, moe.Experts(), moe.Experts(), None, 0.0)

    def tier_call(tt, slab):
        return L.moe_tier_forward(tt, 0, ctypes.byref(cfg), ctypes.byref(rl), a256, a256, slab, a256,
                                  1, a256, 0, 0, a256, None, a256, big, a256, big, None)
    assert tier_call(t, lay.bytes + 8) == -3
    assert tier_call(t, lay.bytes - 16) == -2
    t_wide = L.moe_tier_create(1, cfg.E, cfg.E + 1)
    assert tier_call(t_wide, lay.bytes) == -2
    t_pin = L.moe_tier_create_pinned(1, cfg.E, cfg.E - 1, 2)
    assert tier_call(t_pin, lay.bytes) == -2
    t_few = L.moe_tier_create(1, cfg.E - 1, 2)   # fewer experts than the layer
    assert tier_call(t_few, lay.bytes) == -2
    for tt in (t_wide, t_pin, t_few):
        L.moe_tier_destroy(tt)
    L.moe_tier_destroy(t)
    # tier objects: invalid sizes give no object
    assert not L.moe_tier_create(0, 8, 4) and not L.moe_tier_create(1, 8, 0)
    assert not L.moe_tier_create_pinned(1, 8, 4, 8)   # pinned slots < experts


def test_prenorm_flag_host_checks():
    """MOE_F_PRENORM: gamma and eps are checked on the host, unknown flag bits
    are refused, and out == x is accepted only with the flag (the calls stop
    at the workspace check here, before any device work)."""
    import numpy as np
    import int4_expert_gemv_moe_amd as moe
    L = moe.lib()
    cfg = moe.config(256, 128, 8, 2)
    host = np.zeros(1 << 16, np.uint8)
    base = host.ctypes.data + (-host.ctypes.data) % 256  # 256-byte aligned host address
    q = moe.QMat(base, base, 0, 0)
    ex = moe.Experts(q, q, q)
    layer = moe.LayerC(base, base, ex, ex, base, 1e-5)
    x = ctypes.c_void_p(base)
    ws = ctypes.c_void_p(base)
    for fn in (L.moe_layer_forward, L.moe_layer_forward_batch):
        def call(flags, out=x, lay=layer):
            return fn(ctypes.byref(cfg), ctypes.byref(lay), x, 1, out, flags, None, ws, 256, None)
        assert call(8) == -1                                   # unknown flag bit
        assert call(moe.F_ACCUMULATE) == -1                    # out overlaps x without the flag
        assert call(moe.F_ACCUMULATE | moe.F_PRENORM) == -4    # in place: only the workspace is short
        no_gamma = moe.LayerC(base, base, ex, ex, None, 1e-5)
        assert call(moe.F_PRENORM, lay=no_gamma) == -1
        for eps in (0.0, -1.0, float("inf"), float("nan")):
            assert call(moe.F_PRENORM, lay=moe.LayerC(base, base, ex, ex, base, eps)) == -1
        assert call(moe.F_PRENORM, lay=moe.LayerC(base, base, ex, ex, base + 4, 1e-5)) == -3
        # out inside x but not equal to it stays refused
        assert call(moe.F_ACCUMULATE | moe.F_PRENORM, out=ctypes.c_void_p(base + 16)) == -1


def test_bf16_token_flag_host_checks():
    """MOE_F_X_BF16: accepted by the union calls only and not with
    MOE_F_PRENORM; x then spans S * D * 2 bytes (the calls stop at the
    workspace check here, before any device work)."""
    import numpy as np
    import int4_expert_gemv_moe_amd as moe
    L = moe.lib()
    cfg = moe.config(256, 128, 8, 2)
    host = np.zeros(1 << 16, np.uint8)
    base = host.ctypes.data + (-host.ctypes.data) % 256
    q = moe.QMat(base, base, 0, 0)
    ex = moe.Experts(q, q, q)
    layer = moe.LayerC(base, base, ex, ex, base, 1e-5)
    x = ctypes.c_void_p(base)
    ws = ctypes.c_void_p(base)
    out = ctypes.c_void_p(base + 2 * 256)  # just past one bf16 row of 256
    bf = moe.F_X_BF16

    def fwd(fn, flags, o=out):
        return fn(ctypes.byref(cfg), ctypes.byref(layer), x, 1, o, flags, None, ws, 256, None)

    def routed(fn, flags, o=out):
        return fn(ctypes.byref(cfg), ctypes.byref(layer), x, 1, x, x, o, flags, ws, 256, None)

    assert fwd(L.moe_layer_forward, bf) == -1                     # per-token path: refused
    assert routed(L.moe_layer_forward_routed, bf) == -1
    assert fwd(L.moe_layer_forward_batch, bf) == -4               # union: only the workspace is short
    assert routed(L.moe_layer_forward_batch_routed, bf) == -4
    assert fwd(L.moe_layer_forward_batch, bf | moe.F_PRENORM) == -1
    # out one float32 row further would overlap a float32 x, not a bf16 one
    assert fwd(L.moe_layer_forward_batch, 0) == -1
    assert fwd(L.moe_layer_forward_batch, bf, ctypes.c_void_p(base + 256)) == -1


def test_int8_format_host_checks():
    """The int8 weight format's calls validate on the host: null pointers,
    shapes, expert index, alignment of the codes and the workspace size."""
    import int4_expert_gemv_moe_amd as moe
    L = moe.lib()
    buf = ctypes.create_string_buffer(512)
    a16 = ctypes.addressof(buf) + (-ctypes.addressof(buf)) % 256
    assert L.moe_quantize_rows_i8(None, 4, 8, a16, a16, None) == -1
    assert L.moe_quantize_rows_i8(a16, 0, 8, a16, a16, None) == -2
    assert L.moe_quantize_rows_i8(a16 + 2, 4, 8, a16, a16, None) == -3
    cfg = moe.config(256, 128, 8, 2)
    # workspace: h [S][I] f32 on a 256-byte boundary
    up = lambda n: (n + 255) // 256 * 256
    assert L.moe_workspace_bytes(ctypes.byref(cfg), 3, moe.WS_SWIGLU8) == up(3 * 128 * 4)
    m = moe.Q8Mat(a16, a16, 0, 0)
    ex = moe.ExpertsI8(m, m, m)
    ws_need = L.moe_workspace_bytes(ctypes.byref(cfg), 1, moe.WS_SWIGLU8)
    call = lambda xq, e, expert, ws_bytes: L.moe_expert_swiglu_i8(
        ctypes.byref(cfg), xq, a16, 1, e, expert, a16, None, None, None, None, a16, ws_bytes, None)
    assert call(a16, None, 0, ws_need) == -1                     # no experts
    assert call(a16, ctypes.byref(ex), 8, ws_need) == -1         # expert index out of range
    assert call(a16 + 8, ctypes.byref(ex), 0, ws_need) == -3     # codes not 16-byte aligned
    bad = moe.ExpertsI8(moe.Q8Mat(a16 + 4, a16, 0, 0), m, m)
    assert call(a16, ctypes.byref(bad), 0, ws_need) == -3        # weight codes misaligned
    odd = moe.ExpertsI8(m, moe.Q8Mat(a16, a16, 24, 0), m)
    assert call(a16, ctypes.byref(odd), 0, ws_need) == -3        # stride not a multiple of 16
    assert call(a16, ctypes.byref(ex), 0, ws_need - 16) == -4    # workspace too small


def test_int2_format_host_checks():
    import int4_expert_gemv_moe_amd as moe
    L = moe.lib()
    buf = ctypes.create_string_buffer(512)
    a16 = ctypes.addressof(buf) + (-ctypes.addressof(buf)) % 256
    assert L.moe_pack_int2(None, 4, 8, a16, a16, None) == -1
    assert L.moe_pack_int2(a16, 4, 0, a16, a16, None) == -2
    assert L.moe_pack_int2(a16 + 1, 4, 8, a16, a16, None) == -3
    m = moe.QMat(a16, a16, 0, 0)
    ex = moe.Experts(m, m, m)
    cfg = moe.config(256, 128, 8, 2)
    need = L.moe_workspace_bytes(ctypes.byref(cfg), 1, moe.WS_SWIGLU8)
    call = lambda c, xq, expert, ws_bytes: L.moe_expert_swiglu_i2(
        ctypes.byref(c), xq, a16, 1, ctypes.byref(ex), expert, a16, None, None, None, None, a16,
        ws_bytes, None)
    assert call(moe.config(256, 96, 8, 2), a16, 0, need) == -2   # I % 64
    assert call(cfg, a16, -1, need) == -1                        # expert index
    assert call(cfg, a16 + 4, 0, need) == -3                     # activation codes misaligned
    assert call(cfg, a16, 0, need - 16) == -4                    # workspace too small


def test_block32_host_checks():
    import int4_expert_gemv_moe_amd as moe
    L = moe.lib()
    buf = ctypes.create_string_buffer(512)
    a16 = ctypes.addressof(buf) + (-ctypes.addressof(buf)) % 256
    assert L.moe_quant_act_b32(None, 1, 64, a16, a16, None) == -1
    assert L.moe_quant_act_b32(a16, 1, 48, a16, a16, None) == -2      # D % 32
    assert L.moe_quant_act_b32(a16 + 4, 1, 64, a16, a16, None) == -3  # x misaligned
    m = moe.QMat(a16, a16, 0, 0)
    ex = moe.Experts(m, m, m)
    cfg = moe.config(256, 128, 8, 2)
    need = L.moe_workspace_bytes(ctypes.byref(cfg), 1, moe.WS_SWIGLU8)
    call = lambda xq, expert, ws_bytes, hq=None: L.moe_expert_swiglu_i4_b32(
        ctypes.byref(cfg), xq, a16, 1, ctypes.byref(ex), expert, a16, hq, None, a16, ws_bytes, None)
    assert call(a16, 8, need) == -1                  # expert index
    assert call(a16 + 8, 0, need) == -3              # codes misaligned
    assert call(a16, 0, need, hq=a16 + 8) == -3      # hidden-code probe misaligned
    assert call(a16, 0, need - 16) == -4             # workspace too small


def test_mla_host_checks():
    import int4_expert_gemv_moe_amd as moe
    L = moe.lib()
    buf = ctypes.create_string_buffer(512)
    a = ctypes.addressof(buf) + (-ctypes.addressof(buf)) % 256
    good = moe.MlaConfig(64, 512, 192, 64, 256, 0.0625)
    assert L.moe_mla_workspace_bytes(ctypes.byref(good), 1, 4096) > 64 * 32 * 512 * 4
    for bad, S, T in ((moe.MlaConfig(64, 500, 192, 64, 256, 0.0625), 1, 8),   # kvl % 64
                      (moe.MlaConfig(64, 2048, 192, 64, 256, 0.0625), 1, 8),  # kvl > 1024
                      (moe.MlaConfig(64, 512, 192, 65, 256, 0.0625), 1, 8),   # rope > 64
                      (good, 4, 3), (good, 1, 16385)):                         # T < S, T too long
        assert L.moe_mla_workspace_bytes(ctypes.byref(bad), S, T) == 0
        assert L.moe_mla_decode(ctypes.byref(bad), a, S, a, a, a, T, a, a, 1 << 20, None) == -2
    need = L.moe_mla_workspace_bytes(ctypes.byref(good), 1, 64)
    assert L.moe_mla_decode(ctypes.byref(good), None, 1, a, a, a, 64, a, a, need, None) == -1
    assert L.moe_mla_decode(ctypes.byref(good), a + 2, 1, a, a, a, 64, a, a, need, None) == -3
    assert L.moe_mla_decode(ctypes.byref(good), a, 1, a, a, a, 64, a, a, need - 16, None) == -4


def test_shared_i8_layer_host_checks():
    import int4_expert_gemv_moe_amd as moe
    L = moe.lib()
    buf = ctypes.create_string_buffer(8192)
    a = ctypes.addressof(buf) + (-ctypes.addressof(buf)) % 256
    out = a + 4096  # apart from x (2 x 256 floats)
    cfg = moe.config(256, 128, 8, 2)
    m = moe.Q8Mat(a, a, 0, 0)
    e8 = moe.ExpertsI8(m, m, m)
    q = moe.QMat(a, a, 0, 0)
    layer = moe.LayerC(a, a, moe.Experts(q, q, q), moe.Experts(), None, 0.0)  # shared not read
    need = L.moe_workspace_bytes(ctypes.byref(cfg), 2, moe.WS_SHARED8)
    assert need > L.moe_workspace_bytes(ctypes.byref(moe.config(256, 128, 8, 2, n_shared=0)), 2, 0)
    assert L.moe_workspace_bytes(ctypes.byref(moe.config(256, 128, 8, 2, n_shared=0)), 2,
                                 moe.WS_SHARED8) == 0
    call = lambda c, e, x, flags, ws_bytes: L.moe_layer_forward_shared_i8(
        ctypes.byref(c), ctypes.byref(layer), e, x, 2, out, flags, a, ws_bytes, None)
    assert call(moe.config(256, 128, 8, 2, n_shared=0), ctypes.byref(e8), a, 0, need) == -2
    assert call(cfg, None, a, 0, need) == -1                  # no int8 shared expert
    assert call(cfg, ctypes.byref(e8), a, 2, need) == -1      # PRENORM is not supported
    assert call(cfg, ctypes.byref(e8), a + 4, 0, need) == -3  # x misaligned
    assert call(cfg, ctypes.byref(e8), a, 0, need - 16) == -4
    # the union variant: the same checks against the union workspace
    need_b = L.moe_workspace_bytes(ctypes.byref(cfg), 2, moe.WS_BATCH)
    callb = lambda c, e, x, flags, ws_bytes: L.moe_layer_forward_batch_shared_i8(
        ctypes.byref(c), ctypes.byref(layer), e, x, 2, out, flags, a, ws_bytes, None)
    assert callb(moe.config(256, 128, 8, 2, n_shared=0), ctypes.byref(e8), a, 0, need_b) == -2
    assert callb(cfg, None, a, 0, need_b) == -1                      # no int8 shared expert
    assert callb(cfg, ctypes.byref(e8), a, moe.F_PRENORM, need_b) == -1  # only MOE_F_ACCUMULATE
    assert callb(cfg, ctypes.byref(e8), a, moe.F_X_BF16, need_b) == -1
    assert callb(cfg, ctypes.byref(e8), a + 4, 0, need_b) == -3      # x misaligned
    assert callb(cfg, ctypes.byref(e8), a, 0, need_b - 16) == -4


def test_noalloc_entry_point_refuses_oversize_calls_on_the_host():
    """moe_layer_forward_noalloc compares the call's workspace need with its
    fixed scratch before touching the device."""
    import int4_expert_gemv_moe_amd as moe
    L = moe.lib()
    cfg = moe.config(6144, 2048, 256, 8)
    assert L.moe_layer_forward_noalloc(ctypes.byref(cfg), None, None, 129, None, 0, None) == -4
    assert L.moe_layer_forward_noalloc(ctypes.byref(cfg), None, None, 0, None, 0, None) == -1
    assert L.moe_workspace_bytes(ctypes.byref(cfg), 128, 0) <= moe.NOALLOC_WS_BYTES
