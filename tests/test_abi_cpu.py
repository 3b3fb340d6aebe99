"""The C ABI on the CPU: the library loads, exports every entry point that
include/moe.h declares, sizes workspaces, and rejects bad arguments on the
host before anything is enqueued (no GPU needed: no call here reaches a
kernel launch)."""
import ctypes

import pytest

import sparse_moe_decode_gemv_amd as M

FAKE = 0x7F0000000000          # a 16-byte aligned address that is never touched


def k3():
    return M.make_shape(7168, 896, 16, 2048, 1, 2048)


def test_library_exports_every_declared_function():
    names = M.header_functions()
    assert {"moe_router_topk", "moe_decode_layer", "moe_decode_stack",
            "moe_workspace_size", "moe_expert_gateup", "moe_group_by_expert",
            "moe_decode_layer_timed", "moe_stream_read",
            "moe_decode_layer_noalloc"} <= set(names)
    L = M.lib()
    for n in names:
        assert hasattr(L, n), n
    assert M.lib().moe_status_string(0) == b"ok"


def test_workspace_size_grows_with_tokens():
    a, b = M.workspace_size(k3(), 1), M.workspace_size(k3(), 64)
    assert 0 < a < b
    assert b < 64 << 20


@pytest.mark.parametrize("shape,status", [
    ((7168, 896, 16, 2048, 1, 2048), 0),
    ((512, 32, 4, 256, 0, 0), 0),
    ((7168, 896, 16, 128, 1, 128), 0),
    ((7168, 896, 17, 2048, 1, 2048), 0),
    ((7000, 896, 16, 2048, 1, 2048), M.MOE_ERR_UNSUPPORTED),   # H % 256
    ((16384, 896, 16, 2048, 1, 2048), M.MOE_ERR_UNSUPPORTED),  # H too large
    ((2304, 64, 4, 256, 0, 0), M.MOE_ERR_UNSUPPORTED),         # 9 blocks per lane
    ((7168, 896, 16, 2000, 1, 2000), M.MOE_ERR_UNSUPPORTED),   # F % 128
    ((7168, 896, 16, 8320, 1, 8320), M.MOE_ERR_UNSUPPORTED),   # F > 8192
    ((7168, 896, 16, 2048, 1, 1024), M.MOE_OK),                # Fs != F
    ((7168, 896, 16, 2048, 1, 1000), M.MOE_ERR_UNSUPPORTED),   # Fs % 128
    ((7168, 896, 16, 2048, 2, 2048), M.MOE_ERR_UNSUPPORTED),   # two shared
    ((7168, 2048, 16, 2048, 0, 0), M.MOE_ERR_UNSUPPORTED),     # E > 1024
    ((7168, 896, 33, 2048, 0, 0), M.MOE_ERR_UNSUPPORTED),      # k > 32
    ((512, 4, 5, 256, 0, 0), M.MOE_ERR_INVALID_ARG),           # k > E
    ((0, 4, 1, 256, 0, 0), M.MOE_ERR_INVALID_ARG),
    ((512, 4, 0, 256, 0, 0), M.MOE_ERR_INVALID_ARG),
])
def test_shape_validation(shape, status):
    n = ctypes.c_size_t(0)
    rc = M.lib().moe_workspace_size(ctypes.byref(M.make_shape(*shape)), 1, ctypes.byref(n))
    assert rc == status


def test_token_limits():
    n = ctypes.c_size_t(0)
    s = k3()
    assert M.lib().moe_workspace_size(ctypes.byref(s), 64, ctypes.byref(n)) == 0
    assert M.lib().moe_workspace_size(ctypes.byref(s), 65, ctypes.byref(n)) == M.MOE_ERR_UNSUPPORTED
    assert M.lib().moe_workspace_size(ctypes.byref(s), -1, ctypes.byref(n)) == M.MOE_ERR_INVALID_ARG


def _weights(**over):
    m = M.MoeMxMat(FAKE, FAKE)
    w = M.MoeLayerWeights(FAKE, m, m, m, m, m, m)
    for k, v in over.items():
        setattr(w, k, v)
    return w


def _layer(shape=None, w=None, x=FAKE, res=FAKE, out=FAKE + (1 << 20), T=1, ws=FAKE + (2 << 20),
           wsb=1 << 26):
    s = shape or k3()
    w = w or _weights()
    return M.lib().moe_decode_layer(ctypes.byref(s), ctypes.byref(w), x, res, out, T, None, None,
                                    ws, wsb, None)


def test_layer_argument_errors():
    assert _layer(T=0) == M.MOE_OK                                  # empty batch: no-op
    assert _layer(T=65) == M.MOE_ERR_UNSUPPORTED
    assert _layer(T=-1) == M.MOE_ERR_INVALID_ARG
    assert _layer(x=None) == M.MOE_ERR_INVALID_ARG
    assert _layer(x=FAKE + 8) == M.MOE_ERR_INVALID_ARG              # misaligned x
    assert _layer(out=None) == M.MOE_ERR_INVALID_ARG
    assert _layer(out=FAKE, res=FAKE + (4 << 20)) == M.MOE_ERR_INVALID_ARG   # out aliases x
    assert _layer(ws=None) == M.MOE_ERR_WORKSPACE
    assert _layer(wsb=1024) == M.MOE_ERR_WORKSPACE
    assert _layer(ws=FAKE) == M.MOE_ERR_INVALID_ARG                  # ws overlaps x
    bad = M.MoeMxMat(FAKE + 4, FAKE)
    assert _layer(w=_weights(gate=bad)) == M.MOE_ERR_INVALID_ARG    # misaligned codes
    assert _layer(w=_weights(router_w=None)) == M.MOE_ERR_INVALID_ARG
    assert _layer(w=_weights(s_down=M.MoeMxMat(None, None))) == M.MOE_ERR_INVALID_ARG
    s0 = M.make_shape(7168, 896, 16, 2048, 0, 0)                   # no shared: ignored
    assert _layer(shape=s0, w=_weights(s_down=M.MoeMxMat(None, None)), T=0) == M.MOE_OK


def test_router_and_stack_argument_errors():
    L, s = M.lib(), k3()
    assert L.moe_router_topk(ctypes.byref(s), FAKE, None, 1, FAKE, FAKE, None, FAKE, 1 << 26,
                             None) == M.MOE_ERR_INVALID_ARG
    assert L.moe_router_topk(ctypes.byref(s), FAKE, FAKE, 1, FAKE, FAKE, None, FAKE, 16,
                             None) == M.MOE_ERR_WORKSPACE
    arr = (M.MoeLayerWeights * 2)(_weights(), _weights())
    g = (ctypes.c_void_p * 2)(FAKE, None)
    assert L.moe_decode_stack(ctypes.byref(s), arr, g, 1e-6, 2, FAKE + (1 << 20), 1, None, None,
                              FAKE + (2 << 20), 1 << 26, None) == M.MOE_ERR_INVALID_ARG
    assert L.moe_decode_stack(ctypes.byref(s), arr, g, -1.0, 2, FAKE, 1, None, None, FAKE,
                              1 << 26, None) == M.MOE_ERR_INVALID_ARG
    assert L.moe_decode_stack(ctypes.byref(s), arr, g, 1e-6, 0, FAKE, 1, None, None, FAKE,
                              1 << 26, None) == M.MOE_OK
    assert L.moe_workspace_init(None, 16, None) == M.MOE_ERR_WORKSPACE


def test_python_binding_raises_on_error():
    with pytest.raises(M.MoeError):
        M.workspace_size(M.make_shape(7000, 896, 16, 2048, 1, 2048), 1)


def test_measurement_entry_points_validate_on_the_host():
    """The timed layer and the streaming read reject bad arguments before
    anything is enqueued (no GPU needed)."""
    import ctypes
    L = M.lib()
    s = k3()
    w = M.MoeLayerWeights()
    ev = (ctypes.c_void_p * 16)(*([FAKE] * 16))
    nk = ctypes.c_int32(-1)
    args = (ctypes.byref(s), ctypes.byref(w), FAKE, FAKE, FAKE + (1 << 20), 1, None, None, FAKE,
            1 << 26, None)
    assert L.moe_decode_layer_timed(*args, None, 3, ctypes.byref(nk)) == M.MOE_ERR_INVALID_ARG
    assert L.moe_decode_layer_timed(*args, ev, M.MOE_MAX_LAYER_KERNELS + 1,
                                    ctypes.byref(nk)) == M.MOE_ERR_INVALID_ARG
    assert L.moe_decode_layer_timed(*args, ev, 3, None) == M.MOE_ERR_INVALID_ARG
    zero = (ctypes.c_void_p * 2)(FAKE, None)
    assert L.moe_decode_layer_timed(*args, zero, 1, ctypes.byref(nk)) == M.MOE_ERR_INVALID_ARG
    # weights missing: the layer's own validation still runs first
    assert L.moe_decode_layer_timed(*args, ev, 3, ctypes.byref(nk)) == M.MOE_ERR_INVALID_ARG
    assert nk.value in (-1, 0)
    assert L.moe_stream_read(None, 1024, FAKE, None) == M.MOE_ERR_INVALID_ARG
    assert L.moe_stream_read(FAKE, 1000, FAKE, None) == M.MOE_ERR_INVALID_ARG
    assert L.moe_stream_read(FAKE + 8, 1024, FAKE, None) == M.MOE_ERR_INVALID_ARG
    assert L.moe_stream_read(FAKE, 1024, None, None) == M.MOE_ERR_INVALID_ARG


def test_noalloc_entry_rejects_shapes_beyond_its_scratch_on_the_host():
    """A shape whose workspace exceeds the library's scratch array is refused
    before any device call; one that fits only fails later on weights."""
    import ctypes
    L = M.lib()
    s = k3()
    n = ctypes.c_size_t(0)
    assert L.moe_workspace_size(ctypes.byref(s), 64, ctypes.byref(n)) == 0
    assert n.value > M.MOE_NOALLOC_SCRATCH_BYTES
    w = M.MoeLayerWeights()
    assert L.moe_decode_layer_noalloc(ctypes.byref(s), ctypes.byref(w), FAKE, FAKE,
                                      FAKE + (1 << 20), 64, None, None, None) == M.MOE_ERR_UNSUPPORTED
    assert L.moe_decode_layer_noalloc(ctypes.byref(s), ctypes.byref(w), FAKE, FAKE,
                                      FAKE + (1 << 20), 65, None, None, None) == M.MOE_ERR_UNSUPPORTED
    assert L.moe_decode_layer_noalloc(None, ctypes.byref(w), FAKE, FAKE, FAKE, 1, None, None,
                                      None) == M.MOE_ERR_INVALID_ARG
    assert L.moe_decode_layer_noalloc(ctypes.byref(s), ctypes.byref(w), FAKE, FAKE, FAKE, 0, None,
                                      None, None) == M.MOE_OK
    # the limit the header states: the K3-sized layer fits up to 24 tokens
    assert M.workspace_size(s, 24) <= M.MOE_NOALLOC_SCRATCH_BYTES < M.workspace_size(s, 25)
    assert L.moe_decode_layer_noalloc(ctypes.byref(s), ctypes.byref(w), FAKE, FAKE,
                                      FAKE + (1 << 20), 25, None, None, None) == M.MOE_ERR_UNSUPPORTED


def test_shared_expert_of_another_width():
    """shared_ffn may differ from ffn (a multiple of 128) at any token count:
    single-token calls give it its own activation planes and down pass, and
    batched calls its own gate/up and down passes, so the workspace grows
    with it; widths outside the limits are refused before any device call."""
    import ctypes
    L = M.lib()
    s = M.make_shape(1024, 24, 4, 256, 1, 512)
    n = ctypes.c_size_t(0)
    assert L.moe_workspace_size(ctypes.byref(s), 1, ctypes.byref(n)) == M.MOE_OK
    assert n.value > M.workspace_size(M.make_shape(1024, 24, 4, 256, 1, 256), 1)
    for T in (2, 17, 64):
        assert L.moe_workspace_size(ctypes.byref(s), T, ctypes.byref(n)) == M.MOE_OK
        assert n.value > M.workspace_size(M.make_shape(1024, 24, 4, 256, 1, 256), T)
    for fs in (200, 8320):
        bad = M.make_shape(1024, 24, 4, 256, 1, fs)
        assert L.moe_workspace_size(ctypes.byref(bad), 1, ctypes.byref(n)) == M.MOE_ERR_UNSUPPORTED
    zero = M.make_shape(1024, 24, 4, 256, 1, 0)
    assert L.moe_workspace_size(ctypes.byref(zero), 1, ctypes.byref(n)) == M.MOE_ERR_INVALID_ARG
