"""C-ABI contract of libgdn.so, checked on a host without a GPU.

The library must load, export every symbol ``include/gdn.h`` declares, carry the
header's ABI version and struct layout, and reject bad arguments with a status
code before anything reaches the GPU (the GLM-5.3 ledger's host ABI contract
test freezes buffer order, fp32 state and the separate q scale the same way).
No call here launches a kernel.
"""
import ctypes
import os
import re
import subprocess

import pytest

import gated_deltanet_causal_amd as gdn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(gdn.LIBRARY):
        from gated_deltanet_causal_amd import build
        build.build()
    return gdn.load_library()


def header_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:gdn_status_t|int|const char\*)\s+(gdn_\w+)\s*\(", text, re.M)))


def test_header_declares_the_binding_exports():
    assert header_functions() == sorted(gdn.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", gdn.LIBRARY], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\bT\s+(gdn_\w+)", out))
    missing = set(header_functions()) - exported
    assert not missing, f"not exported: {missing}"
    for name in header_functions():
        assert hasattr(lib, name)


def test_abi_version_matches_header(lib):
    m = re.search(r"#define\s+GDN_ABI_VERSION\s+(\d+)", open(HEADER).read())
    assert lib.gdn_abi_version() == int(m.group(1))


def test_config_struct_layout_and_defaults(lib):
    assert ctypes.sizeof(gdn.GDNConfig) == 12 * 4
    assert [f for f, _ in gdn.GDNConfig._fields_] == [
        "num_k_heads", "num_v_heads", "head_k_dim", "head_v_dim", "conv_width", "chunk_size", "conv_act",
        "decay_per_key_channel", "qk_l2norm", "l2_eps", "rms_eps", "q_scale"]
    cfg = gdn.config()
    assert (cfg.num_k_heads, cfg.num_v_heads, cfg.head_k_dim, cfg.head_v_dim) == (16, 48, 128, 128)
    assert (cfg.conv_width, cfg.chunk_size, cfg.conv_act, cfg.decay_per_key_channel) == (4, 64, 1, 0)
    assert cfg.qk_l2norm == 1
    assert cfg.l2_eps == pytest.approx(1e-6) and cfg.rms_eps == pytest.approx(1e-6)
    assert cfg.q_scale == pytest.approx(1 / 128 ** 0.5)
    assert cfg.conv_channels == 10240


def test_status_strings(lib):
    for s in range(6):
        assert lib.gdn_status_string(s)
    assert lib.gdn_status_string(99) == b"unknown status"


def _cfg(**kw):
    return gdn.config(**kw)


def test_config_validation(lib):
    size = ctypes.c_size_t()
    ok = lib.gdn_chunk_prefill_workspace_size(ctypes.byref(_cfg()), 1, 4096, ctypes.byref(size))
    assert ok == gdn.GDN_OK and size.value > 0
    for kw, want in [(dict(head_k_dim=64), gdn.GDN_ERR_UNSUPPORTED), (dict(conv_width=3), gdn.GDN_ERR_UNSUPPORTED),
                     (dict(chunk_size=32), gdn.GDN_ERR_UNSUPPORTED), (dict(num_v_heads=47), gdn.GDN_ERR_INVALID_ARG),
                     (dict(num_k_heads=0), gdn.GDN_ERR_INVALID_ARG), (dict(conv_act=2), gdn.GDN_ERR_INVALID_ARG),
                     (dict(l2_eps=-1.0), gdn.GDN_ERR_INVALID_ARG), (dict(qk_l2norm=2), gdn.GDN_ERR_INVALID_ARG)]:
        got = lib.gdn_chunk_prefill_workspace_size(ctypes.byref(_cfg(**kw)), 1, 64, ctypes.byref(size))
        assert got == want, kw
    assert lib.gdn_chunk_prefill_workspace_size(None, 1, 64, ctypes.byref(size)) == gdn.GDN_ERR_INVALID_ARG


def test_workspace_size_grows_with_tokens_and_sequences(lib):
    def ws(n, t):
        s = ctypes.c_size_t()
        assert lib.gdn_chunk_prefill_workspace_size(ctypes.byref(_cfg()), n, t, ctypes.byref(s)) == 0
        return s.value
    assert ws(1, 4096) < ws(1, 8192) and ws(1, 4096) < ws(8, 4096)


FAKE = ctypes.c_void_p(0x10000)        # never dereferenced: validation fails first


def test_seqlens_validation_before_launch(lib):
    cfg = _cfg()
    for cu, want in [([1, 5], gdn.GDN_ERR_SEQLENS), ([0, 4], gdn.GDN_ERR_SEQLENS), ([0, 6, 5], gdn.GDN_ERR_SEQLENS)]:
        hc = (ctypes.c_int32 * len(cu))(*cu)
        got = lib.gdn_conv1d_prefill(ctypes.byref(cfg), gdn.GDN_BF16, FAKE, 10240, FAKE, None, None,
                                     ctypes.c_void_p(0x20000), 10240, FAKE, hc, len(cu) - 1, 5, None)
        assert got == want, cu


def test_conv_prefill_argument_checks(lib):
    cfg = _cfg()
    hc = (ctypes.c_int32 * 2)(0, 5)
    call = lambda **kw: lib.gdn_conv1d_prefill(
        ctypes.byref(cfg), kw.get("dtype", gdn.GDN_BF16), kw.get("x", FAKE), kw.get("xs", 10240), FAKE,
        None, None, kw.get("y", ctypes.c_void_p(0x200000)), kw.get("ys", 10240), FAKE, hc, 1, 5, None)
    assert call(x=None) == gdn.GDN_ERR_INVALID_ARG
    assert call(xs=10000) == gdn.GDN_ERR_INVALID_ARG                 # stride < channels
    assert call(xs=10244) == gdn.GDN_ERR_INVALID_ARG                 # stride not a multiple of 8
    assert call(y=ctypes.c_void_p(0x10000 + 64)) == gdn.GDN_ERR_INVALID_ARG   # y overlaps x
    assert call(dtype=7) == gdn.GDN_ERR_UNSUPPORTED


def test_chunk_prefill_argument_checks(lib):
    cfg = _cfg()
    hc = (ctypes.c_int32 * 2)(0, 64)

    def call(**kw):
        return lib.gdn_chunk_prefill(
            ctypes.byref(kw.get("cfg", cfg)), gdn.GDN_BF16, gdn.GDN_F32, FAKE, FAKE, kw.get("qks", 10240),
            FAKE, 10240, FAKE, FAKE, None, FAKE, hc, 1, 64, ctypes.c_void_p(0x4000000), None,
            kw.get("ws", ctypes.c_void_p(0x8000000)), kw.get("wsb", 0), None)
    assert call() == gdn.GDN_ERR_WORKSPACE                                  # zero-size workspace
    assert call(ws=None, wsb=1 << 30) == gdn.GDN_ERR_WORKSPACE
    assert call(qks=100) == gdn.GDN_ERR_INVALID_ARG
    assert call(cfg=_cfg(decay_per_key_channel=1)) == gdn.GDN_ERR_WORKSPACE     # supported; workspace checked


def test_decode_and_norm_argument_checks(lib):
    cfg = _cfg()
    got = lib.gdn_decode_step(ctypes.byref(cfg), gdn.GDN_BF16, gdn.GDN_BF16, FAKE, FAKE, FAKE, FAKE, FAKE,
                              FAKE, FAKE, None, FAKE, 4, None)
    assert got == gdn.GDN_ERR_INVALID_ARG                                  # state missing
    got = lib.gdn_decode_step(ctypes.byref(cfg), gdn.GDN_BF16, gdn.GDN_BF16, FAKE, FAKE, FAKE, FAKE, FAKE,
                              FAKE, FAKE, FAKE, FAKE, -1, None)
    assert got == gdn.GDN_ERR_INVALID_ARG
    got = lib.gdn_gated_rmsnorm(ctypes.byref(cfg), gdn.GDN_F32, gdn.GDN_BF16, gdn.GDN_BF16, FAKE, FAKE, FAKE,
                                FAKE, 4, None)
    assert got == gdn.GDN_ERR_INVALID_ARG                                  # in place across dtypes
    got = lib.gdn_gated_rmsnorm(ctypes.byref(cfg), gdn.GDN_F32, gdn.GDN_BF16, gdn.GDN_F32, FAKE, FAKE, FAKE,
                                ctypes.c_void_p(0x10000 + 256), 4, None)
    assert got == gdn.GDN_ERR_INVALID_ARG                                  # partial overlap
    far = ctypes.c_void_p(0x40000000)
    got = lib.gdn_gated_rmsnorm(ctypes.byref(cfg), gdn.GDN_F32, gdn.GDN_BF16, gdn.GDN_BF16,
                                ctypes.c_void_p(0x10000 + 8), FAKE, FAKE, far, 4, None)
    assert got == gdn.GDN_ERR_INVALID_ARG                                  # o not 16-byte aligned


def test_empty_calls_launch_nothing(lib):
    """Zero-sized work returns OK without touching the device."""
    cfg = _cfg()
    assert lib.gdn_conv1d_step(ctypes.byref(cfg), gdn.GDN_BF16, None, 10240, None, None, None, 10240, 0, None) == 0
    assert lib.gdn_decode_step(ctypes.byref(cfg), gdn.GDN_BF16, gdn.GDN_BF16, None, None, None, None, None,
                               None, None, None, None, 0, None) == 0
    assert lib.gdn_gated_rmsnorm(ctypes.byref(cfg), gdn.GDN_F32, gdn.GDN_F32, gdn.GDN_F32, None, None, None,
                                 None, 0, None) == 0
    # no rows, output dtype other than o's: empty buffers may both sit at address 0
    assert lib.gdn_gated_rmsnorm(ctypes.byref(cfg), gdn.GDN_F32, gdn.GDN_BF16, gdn.GDN_BF16, None, None, None,
                                 None, 0, None) == 0


def test_decode_rejects_batches_past_the_shift_grid(lib):
    """The q / k conv-state shift after the step takes the sequences on grid.y (at most
    65535): a larger batch is refused before anything is launched, for every decode call."""
    cfg = _cfg()
    for fn in (lib.gdn_decode_step, lib.gdn_decode_step_h16):
        got = fn(ctypes.byref(cfg), gdn.GDN_BF16, gdn.GDN_BF16, FAKE, FAKE, FAKE, FAKE, FAKE,
                 FAKE, FAKE, FAKE, FAKE, 65536, None)
        assert got == gdn.GDN_ERR_INVALID_ARG
    got = lib.gdn_decode_step_ab(ctypes.byref(cfg), gdn.GDN_BF16, gdn.GDN_BF16, FAKE, FAKE, FAKE, FAKE, FAKE,
                                 FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 65536, None)
    assert got == gdn.GDN_ERR_INVALID_ARG


def test_decode_rejects_grids_past_int32(lib):
    """One workgroup per (sequence, value head): B * Hv must fit a 32-bit grid."""
    cfg = _cfg(num_k_heads=1, num_v_heads=1 << 20)
    got = lib.gdn_decode_step(ctypes.byref(cfg), gdn.GDN_BF16, gdn.GDN_BF16, FAKE, FAKE, FAKE, FAKE, FAKE,
                              FAKE, FAKE, FAKE, FAKE, 4096, None)
    assert got == gdn.GDN_ERR_INVALID_ARG


def _prefill_ws(lib, n, t, dtype=gdn.GDN_BF16, cfg=None):
    s = ctypes.c_size_t()
    assert lib.gdn_prefill_workspace_size(ctypes.byref(cfg or _cfg()), dtype, n, t, ctypes.byref(s)) == 0
    return s.value


def test_prefill_workspace_holds_the_prenorm_output_only_when_unfused(lib):
    """Six or more sequences of 48 value heads (bf16, scalar decay) apply the norm inside the
    chunk kernels: no fp32 pre-norm buffer.  Fewer, fp32 or per-key-channel decay keep it."""
    T = 4096
    o_bytes = T * 48 * 128 * 4
    fused, unfused = _prefill_ws(lib, 6, T), _prefill_ws(lib, 5, T)

    def chunk_ws(n):
        s = ctypes.c_size_t()
        assert lib.gdn_chunk_prefill_workspace_size(ctypes.byref(_cfg()), n, T, ctypes.byref(s)) == 0
        return s.value
    assert abs((unfused - fused) - (o_bytes - (chunk_ws(6) - chunk_ws(5)))) <= 512
    assert _prefill_ws(lib, 6, T, gdn.GDN_F32) - fused >= o_bytes + T * 10240 * 2 - 4096
    assert _prefill_ws(lib, 6, T, cfg=_cfg(decay_per_key_channel=1)) > fused + o_bytes - 4096
    assert _prefill_ws(lib, 1, T) > _prefill_ws(lib, 1, T // 2)


def test_prefill_argument_checks(lib):
    cfg = _cfg()
    hc = (ctypes.c_int32 * 2)(0, 64)
    need = _prefill_ws(lib, 1, 64)

    def call(**kw):
        return lib.gdn_prefill(
            ctypes.byref(cfg), gdn.GDN_BF16, gdn.GDN_BF16, kw.get("x", FAKE), kw.get("xs", 10240), FAKE,
            None, None, FAKE, FAKE, kw.get("z", ctypes.c_void_p(0x2000000)), FAKE, None, FAKE, hc, 1, 64,
            ctypes.c_void_p(0x4000000), None, kw.get("ws", ctypes.c_void_p(0x8000000)), kw.get("wsb", need),
            None)
    assert call(wsb=0) == gdn.GDN_ERR_WORKSPACE
    assert call(ws=None) == gdn.GDN_ERR_WORKSPACE
    assert call(wsb=need - 1) == gdn.GDN_ERR_WORKSPACE
    assert call(z=None) == gdn.GDN_ERR_INVALID_ARG
    assert call(z=ctypes.c_void_p(0x2000000 + 8)) == gdn.GDN_ERR_INVALID_ARG     # z not 16-byte aligned
    assert call(xs=10244) == gdn.GDN_ERR_INVALID_ARG
    assert call(ws=ctypes.c_void_p(0x10000 + 4096)) == gdn.GDN_ERR_INVALID_ARG  # workspace overlaps x
    assert call(ws=ctypes.c_void_p(0x4000000)) == gdn.GDN_ERR_INVALID_ARG       # workspace overlaps out
    assert lib.gdn_prefill(ctypes.byref(cfg), gdn.GDN_BF16, gdn.GDN_BF16, None, 10240, FAKE, None, None,
                           None, None, None, None, None, FAKE, (ctypes.c_int32 * 1)(0), 0, 0, None, None,
                           None, 0, None) == 0                                   # nothing to do


def test_derived_gate_calls_argument_checks(lib):
    """The *_ab calls take a, b, A_log, dt_bias in place of g, beta: all four are required,
    and per-key-channel decay (whose gates the pages do not derive) is unsupported."""
    cfg, pc = _cfg(), _cfg(decay_per_key_channel=1)

    def decode(c, A_log=FAKE, a=FAKE):
        return lib.gdn_decode_step_ab(ctypes.byref(c), gdn.GDN_BF16, gdn.GDN_BF16, FAKE, FAKE, FAKE, a, FAKE,
                                      A_log, FAKE, FAKE, FAKE, FAKE, FAKE, 4, None)
    assert decode(pc) == gdn.GDN_ERR_UNSUPPORTED
    assert decode(cfg, A_log=None) == gdn.GDN_ERR_INVALID_ARG
    assert decode(cfg, a=None) == gdn.GDN_ERR_INVALID_ARG
    hc = (ctypes.c_int32 * 2)(0, 64)

    def chunk(c, dt_bias=FAKE):
        return lib.gdn_chunk_prefill_ab(ctypes.byref(c), gdn.GDN_BF16, gdn.GDN_F32, FAKE, FAKE, 10240, FAKE,
                                        10240, FAKE, FAKE, FAKE, dt_bias, None, FAKE, hc, 1, 64,
                                        ctypes.c_void_p(0x4000000), None, ctypes.c_void_p(0x8000000), 0, None)
    assert chunk(pc) == gdn.GDN_ERR_UNSUPPORTED
    assert chunk(cfg, dt_bias=None) == gdn.GDN_ERR_INVALID_ARG
    assert chunk(cfg) == gdn.GDN_ERR_WORKSPACE          # gates accepted; the workspace is checked next


def test_verify_argument_checks(lib):
    cfg = _cfg()
    size = ctypes.c_size_t()
    assert lib.gdn_verify_workspace_size(ctypes.byref(cfg), 64, 4, ctypes.byref(size)) == 0
    assert size.value == 64 * 4 * (48 * 128 + 16 * 128) * 4
    assert lib.gdn_verify_workspace_size(ctypes.byref(cfg), 64, 0, ctypes.byref(size)) == gdn.GDN_ERR_INVALID_ARG
    assert lib.gdn_verify_workspace_size(ctypes.byref(cfg), 64, 65, ctypes.byref(size)) == gdn.GDN_ERR_INVALID_ARG

    def verify(K=4, ws=ctypes.c_void_p(0x8000000), wsb=size.value, state=ctypes.c_void_p(0x4000000)):
        return lib.gdn_verify(ctypes.byref(cfg), gdn.GDN_BF16, gdn.GDN_BF16, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                              FAKE, state, ctypes.c_void_p(0x2000000), 64, K, ws, wsb, None)
    assert verify(K=0) == gdn.GDN_ERR_INVALID_ARG
    assert verify(wsb=size.value - 1) == gdn.GDN_ERR_WORKSPACE
    assert verify(state=None) == gdn.GDN_ERR_INVALID_ARG
    assert verify(state=ctypes.c_void_p(0x8000000)) == gdn.GDN_ERR_INVALID_ARG   # state overlaps the workspace
    got = lib.gdn_verify_commit(ctypes.byref(cfg), gdn.GDN_BF16, None, FAKE, FAKE, FAKE, FAKE, 64, 4,
                                ctypes.c_void_p(0x8000000), size.value, None)
    assert got == gdn.GDN_ERR_INVALID_ARG                                         # accepted missing
    assert lib.gdn_verify(ctypes.byref(cfg), gdn.GDN_BF16, gdn.GDN_BF16, None, None, None, None, None, None, None,
                          None, None, 0, 4, None, 0, None) == 0                   # nothing to do


def test_state_convert_and_h16_decode_argument_checks(lib):
    conv = lambda sd, dd, src=FAKE, n=64: lib.gdn_state_convert(src, sd, ctypes.c_void_p(0x2000000), dd, n, None)
    assert conv(gdn.GDN_F32, gdn.GDN_BF16) == gdn.GDN_ERR_UNSUPPORTED
    assert conv(gdn.GDN_F16, gdn.GDN_F16) == gdn.GDN_ERR_UNSUPPORTED
    assert conv(gdn.GDN_F32, gdn.GDN_F16, src=ctypes.c_void_p(0x10008)) == gdn.GDN_ERR_INVALID_ARG
    assert conv(gdn.GDN_F32, gdn.GDN_F16, src=ctypes.c_void_p(0x2000000 - 64)) == gdn.GDN_ERR_INVALID_ARG  # overlap
    assert conv(gdn.GDN_F32, gdn.GDN_F16, n=0) == 0
    cfg = _cfg()
    got = lib.gdn_decode_step_h16(ctypes.byref(cfg), gdn.GDN_BF16, gdn.GDN_BF16, FAKE, FAKE, FAKE, FAKE, FAKE,
                                  FAKE, FAKE, None, FAKE, 4, None)
    assert got == gdn.GDN_ERR_INVALID_ARG                                  # state missing
    got = lib.gdn_decode_step(ctypes.byref(cfg), gdn.GDN_F16, gdn.GDN_BF16, FAKE, FAKE, FAKE, FAKE, FAKE,
                              FAKE, FAKE, FAKE, FAKE, 4, None)
    assert got == gdn.GDN_ERR_UNSUPPORTED                                  # fp16 is not an activation dtype


def test_noalloc_chunk_prefill_rejects_sizes_past_its_scratch(lib):
    """gdn_chunk_prefill_noalloc refuses any size whose workspace exceeds the fixed array
    (before any HIP call, so this runs without a GPU); an empty batch is a no-op."""
    cfg = _cfg()
    limit = 128 << 20
    s = ctypes.c_size_t()
    assert lib.gdn_chunk_prefill_workspace_size(ctypes.byref(cfg), 1, 8192, ctypes.byref(s)) == 0
    assert s.value > limit
    hc = (ctypes.c_int32 * 2)(0, 8192)
    got = lib.gdn_chunk_prefill_noalloc(ctypes.byref(cfg), gdn.GDN_BF16, gdn.GDN_F32, FAKE, FAKE, 10240, FAKE,
                                        10240, FAKE, FAKE, None, FAKE, hc, 1, 8192, FAKE, None, None)
    assert got == gdn.GDN_ERR_WORKSPACE
    h0 = (ctypes.c_int32 * 1)(0)
    assert lib.gdn_chunk_prefill_noalloc(ctypes.byref(cfg), gdn.GDN_BF16, gdn.GDN_F32, None, None, 10240, None,
                                         10240, None, None, None, FAKE, h0, 0, 0, None, None, None) == 0
