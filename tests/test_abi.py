"""The C ABI without a GPU: the library loads, exports every function the header
declares, rejects bad arguments before touching the device, and its workspace grows
with one chunk of rows and with V*H, never with S*L*V."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "grpo.h")


def _declared():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(grpo_[a-z_]+)\s*\(", txt)))


@pytest.fixture(scope="module")
def lib():
    import grpo_loss_amd
    return grpo_loss_amd.load_library()


def test_exports_every_declared_symbol(lib):
    names = _declared()
    assert {"grpo_advantages", "grpo_loss_fwd", "grpo_loss_bwd",
            "grpo_workspace_bytes", "grpo_status_string"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for code in range(0, -11, -1):
        s = lib.grpo_status_string(code)
        assert s and s != b"unknown status"
    assert lib.grpo_status_string(-99) == b"unknown status"


def test_workspace_bytes(lib):
    f = lib.grpo_workspace_bytes
    assert f(8, 20480, 4096, 128256, 1, 0) > 0
    assert f(8, 20480, 4096, 128256, 1, 0) == f(8, 20480, 4096, 128256, 1, 0)
    assert f(0, 10, 64, 10, 1, 0) == 0          # S < 1
    assert f(2, 10, 100, 10, 1, 0) == 0         # H not a multiple of 8
    assert f(2, 10, 72, 10, 1, 0) > 0           # H a multiple of 8 (FMA kernels)
    assert f(2, 10, 64, 10, 7, 0) == 0          # bad dtype
    # O(chunk): doubling L adds only per-row bookkeeping (indices, partials: about 1 KB a
    # row), against 2 * 2 * V bytes a row for materialised policy and reference logits
    a = f(8, 20480, 4096, 128256, 1, 0)
    b = f(8, 40960, 4096, 128256, 1, 0)
    assert (b - a) / (8 * 20480) < 1024 < 2 * 2 * 128256
    materialised = 2 * 2 * 8 * 20480 * 128256
    assert a < materialised / 20


def test_workspace_follows_chunk_rows(lib):
    """Without dW the backward is split over the vocabulary: the chunk buffer holds one
    chunk of rows x one piece of about 32768 entries (chunk_rows and vocab_piece set
    them), plus the chunk's fp32 dX sums; the headline shape stays under 0.5 GiB.  With
    dW the single pass keeps one chunk of rows x the whole vocabulary."""
    import grpo_loss_amd as g
    f = lib.grpo_workspace_bytes_opts
    shape = (8, 20480, 4096, 128256, 1, 0)
    default = f(*shape, None)
    assert default == lib.grpo_workspace_bytes(*shape)
    assert default < 0.5 * 2 ** 30
    assert f(*shape, ctypes.byref(g.options(chunk_rows=4096))) == default
    assert f(*shape, ctypes.byref(g.options(vocab_piece=32768))) == default  # 4 x 126 tiles
    # 501 tiles in pieces of at most 64 tiles: 8 pieces of 63 tiles (16128 entries)
    half = f(*shape, ctypes.byref(g.options(vocab_piece=16384)))
    assert default - half >= 0.95 * 4096 * (32256 - 16128) * 2   # (more partial slots)
    big = f(*shape, ctypes.byref(g.options(chunk_rows=8192)))
    assert big - default >= 4096 * 32256 * 2 + 4096 * 4096 * 4     # terms + dX sums
    # with dW: one chunk of rows x the padded vocabulary
    train = lib.grpo_workspace_bytes(8, 4096, 4096, 128256, 1, 1)
    assert train >= 4096 * 128256 * 2
    assert f(*shape, ctypes.byref(g.options(chunk_rows=300))) == 0
    assert f(*shape, ctypes.byref(g.options(vocab_piece=100))) == 0


def test_workspace_for_few_token_blocks(lib):
    """MFMA shapes with 1 to 40 token blocks: the plan (vocabulary pieces, phase counts,
    partial buffers) is well defined wherever fewer than 8 token blocks let the forward's
    phases span several XCDs, and the workspace grows with the rows."""
    f = lib.grpo_workspace_bytes
    for V in (300, 5003, 151936):
        for need_dw in (0, 1):
            prev = 0
            for rows in (1, 200, 256, 700, 1000, 1800, 2047, 4096, 10000):
                b = f(1, rows, 256, V, 1, need_dw)
                assert b > 0, (V, need_dw, rows)
                assert b >= prev, (V, need_dw, rows)
                prev = b


def test_bad_arguments_rejected_before_launch(lib):
    p = ctypes.c_void_p(16)   # never dereferenced: validation fails first
    nul = None
    rc = lib.grpo_loss_fwd(nul, p, p, 1, p, p, p, 2, 3, 64, 5, ctypes.c_float(0.04), p, p,
                           nul, nul, nul, p, nul, p, ctypes.c_size_t(1 << 40), nul)
    assert rc == -1
    rc = lib.grpo_loss_fwd(p, p, p, 9, p, p, p, 2, 3, 64, 5, ctypes.c_float(0.04), p, p,
                           nul, nul, nul, p, nul, p, ctypes.c_size_t(1 << 40), nul)
    assert rc == -3
    rc = lib.grpo_loss_fwd(p, p, p, 1, p, p, p, 2, 3, 100, 5, ctypes.c_float(0.04), p, p,
                           nul, nul, nul, p, nul, p, ctypes.c_size_t(1 << 40), nul)
    assert rc == -2
    odd = ctypes.c_void_p(18)
    rc = lib.grpo_loss_fwd(odd, p, p, 1, p, p, p, 2, 3, 64, 5, ctypes.c_float(0.04), p, p,
                           nul, nul, nul, p, nul, p, ctypes.c_size_t(1 << 40), nul)
    assert rc == -4
    rc = lib.grpo_loss_fwd(p, p, p, 1, p, p, p, 2, 3, 64, 5, ctypes.c_float(0.04), p, p,
                           nul, nul, nul, p, nul, p, ctypes.c_size_t(8), nul)
    assert rc == -5
    rc = lib.grpo_loss_bwd(p, p, 1, p, p, p, 2, 3, 64, 5, nul, ctypes.c_float(0.0), p, nul, 0,
                           p, nul, p, ctypes.c_size_t(1 << 40), nul)
    assert rc == -2                              # loss_scale must be > 0
    rc = lib.grpo_advantages(p, 1, 1, 1, ctypes.c_float(1e-4), 1, p, nul)
    assert rc == -2                              # unbiased std needs G >= 2
    rc = lib.grpo_advantages(nul, 1, 8, 1, ctypes.c_float(1e-4), 1, p, nul)
    assert rc == -1


def test_options(lib):
    import grpo_loss_amd as g
    d = g.GRPOOptions()
    lib.grpo_default_options(ctypes.byref(d))
    assert (d.kl_estimator, d.detach_ratio, d.normalization, d.temperature) == (0, 1, 0, 1.0)
    lib.grpo_default_options(None)               # tolerated
    p = ctypes.c_void_p(16)
    nul = None
    assert (d.fp8_logits, d.chunk_rows) == (0, 0)
    bad = [g.options(temperature=0.0), g.options(temperature=float("nan")),
           g.options(temperature=1e4), g.GRPOOptions(3, 1, 0, 1.0), g.GRPOOptions(0, 2, 0, 1.0),
           g.GRPOOptions(0, 1, 2, 1.0), g.options(chunk_rows=100), g.options(chunk_rows=-256),
           g.options(chunk_rows=128), g.options(chunk_rows=65536 + 256)]
    for o in bad:
        rc = lib.grpo_loss_fwd(p, p, p, 1, p, p, p, 2, 3, 64, 5, ctypes.c_float(0.04), p, p,
                               nul, nul, nul, p, ctypes.byref(o), p, ctypes.c_size_t(1 << 40),
                               nul)
        assert rc == -8
        rc = lib.grpo_loss_bwd(p, p, 1, p, p, p, 2, 3, 64, 5, nul, ctypes.c_float(1.0), p, nul,
                               0, p, ctypes.byref(o), p, ctypes.c_size_t(1 << 40), nul)
        assert rc == -8


def test_fused_and_scale_bad_arguments(lib):
    p = ctypes.c_void_p(16)
    nul = None
    f = ctypes.c_float
    # grpo_loss_fwd_bwd: NULL dXq, bad dtype, loss_scale 0, bad option
    rc = lib.grpo_loss_fwd_bwd(p, p, p, 1, p, p, p, 2, 3, 64, 5, f(0.04), nul, f(1.0), p, p,
                               nul, nul, nul, p, nul, nul, 0, p, nul, p,
                               ctypes.c_size_t(1 << 40), nul)
    assert rc == -1
    rc = lib.grpo_loss_fwd_bwd(p, p, p, 9, p, p, p, 2, 3, 64, 5, f(0.04), nul, f(1.0), p, p,
                               nul, nul, nul, p, p, nul, 0, p, nul, p,
                               ctypes.c_size_t(1 << 40), nul)
    assert rc == -3
    rc = lib.grpo_loss_fwd_bwd(p, p, p, 1, p, p, p, 2, 3, 64, 5, f(0.04), nul, f(0.0), p, p,
                               nul, nul, nul, p, p, nul, 0, p, nul, p,
                               ctypes.c_size_t(1 << 40), nul)
    assert rc == -2
    import grpo_loss_amd as g
    o = g.options(temperature=-1.0)
    rc = lib.grpo_loss_fwd_bwd(p, p, p, 1, p, p, p, 2, 3, 64, 5, f(0.04), nul, f(1.0), p, p,
                               nul, nul, nul, p, p, nul, 0, p, ctypes.byref(o), p,
                               ctypes.c_size_t(1 << 40), nul)
    assert rc == -8
    rc = lib.grpo_loss_fwd_bwd(p, p, p, 1, p, p, p, 2, 3, 64, 5, f(0.04), nul, f(1.0), p, p,
                               nul, nul, nul, p, p, nul, 0, p, nul, p, ctypes.c_size_t(8), nul)
    assert rc == -5
    # grpo_scale_grad: NULL grad, H not a multiple of 8, bad scale
    assert lib.grpo_scale_grad(p, 1, 4, 64, nul, 0, nul, f(1.0), p, nul) == -1
    assert lib.grpo_scale_grad(p, 1, 4, 12, nul, 0, p, f(1.0), p, nul) == -2
    assert lib.grpo_scale_grad(p, 1, 4, 64, nul, 0, p, f(0.0), p, nul) == -2
    assert lib.grpo_scale_grad(p, 7, 4, 64, nul, 0, p, f(1.0), p, nul) == -3


def test_fp8_options_and_quantizer_arguments(lib):
    import grpo_loss_amd as g
    p = ctypes.c_void_p(16)
    nul = None
    f = ctypes.c_float
    o8 = g.options(fp8_logits=True)
    base = lib.grpo_workspace_bytes(8, 4096, 4096, 128256, 1, 0)
    with8 = lib.grpo_workspace_bytes_opts(8, 4096, 4096, 128256, 1, 0, ctypes.byref(o8))
    # the e4m3 copies: N H (two sides) + V H bytes and the scales
    assert with8 - base >= 2 * 8 * 4096 * 4096 + 128256 * 4096
    assert lib.grpo_workspace_bytes_opts(8, 4096, 4096, 128256, 1, 0, None) == base
    assert lib.grpo_workspace_bytes_opts(2, 64, 64, 1000, 0, 0, ctypes.byref(o8)) == 0  # fp32
    bad = g.GRPOOptions(0, 1, 0, 1.0, 2)
    assert lib.grpo_workspace_bytes_opts(8, 4096, 4096, 128256, 1, 0, ctypes.byref(bad)) == 0
    # fp8 logits with fp32 inputs, or H not a multiple of 256: rejected before any launch
    rc = lib.grpo_loss_fwd(p, p, p, 0, p, p, p, 2, 3, 64, 5, f(0.04), p, p, nul, nul, nul, p,
                           ctypes.byref(o8), p, ctypes.c_size_t(1 << 40), nul)
    assert rc == -8
    rc = lib.grpo_loss_fwd_bwd(p, p, p, 1, p, p, p, 2, 3, 64, 5, f(0.04), nul, f(1.0), p, p,
                               nul, nul, nul, p, p, nul, 0, p, ctypes.byref(o8), p,
                               ctypes.c_size_t(1 << 40), nul)
    assert rc == -8
    rc = lib.grpo_loss_bwd(p, p, 1, p, p, p, 2, 3, 64, 5, nul, f(1.0), p, nul, 0, p,
                           ctypes.byref(bad), p, ctypes.c_size_t(1 << 40), nul)
    assert rc == -8
    assert lib.grpo_quantize_e4m3(nul, 1, 4, 64, p, p, nul) == -1
    assert lib.grpo_quantize_e4m3(p, 1, 4, 62, p, p, nul) == -2
    assert lib.grpo_quantize_e4m3(p, 5, 4, 64, p, p, nul) == -3
    assert lib.grpo_quantize_e4m3(p, 1, 4, 64, ctypes.c_void_p(17), p, nul) == -4


def test_trace_options_validated(lib):
    """Kernel tracing: an unknown kernel, a negative capacity, or events missing for a
    positive capacity are option errors, raised before any launch."""
    import grpo_loss_amd as g
    p = ctypes.c_void_p(16)
    nul = None
    for kernel, cap, with_events in ((6, 0, False), (-1, 0, False), (1, -1, False),
                                     (1, 4, False)):
        o = g.options()
        o.trace_kernel, o.trace_capacity = kernel, cap
        if with_events:
            o.trace_events = (ctypes.c_void_p * 8)()
        rc = lib.grpo_loss_fwd(p, p, p, 1, p, p, p, 2, 3, 64, 5, ctypes.c_float(0.04), p, p,
                               nul, nul, nul, p, ctypes.byref(o), p, ctypes.c_size_t(1 << 40),
                               nul)
        assert rc == -8, (kernel, cap)
    d = g.GRPOOptions()
    lib.grpo_default_options(ctypes.byref(d))
    assert (d.trace_kernel, d.trace_capacity) == (0, 0) and not d.trace_events


def test_noalloc_rejects_before_launch(lib):
    """grpo_loss_fwd_noalloc validates like grpo_loss_fwd and rejects a forward larger than
    its fixed array with GRPO_ERR_SCRATCH, all before touching a device."""
    p = ctypes.c_void_p(256)
    nul = None
    f = ctypes.c_float(0.04)
    assert lib.grpo_loss_fwd_noalloc(nul, p, p, 1, p, p, p, 2, 3, 64, 5, f, p, p, nul, nul,
                                     nul, p, nul, nul) == -1
    assert lib.grpo_loss_fwd_noalloc(p, p, p, 1, p, p, p, 2, 3, 100, 5, f, p, p, nul, nul, nul,
                                     p, nul, nul) == -2
    # the long-context forward: 118 MB of partials, past the 64 MiB array
    assert lib.grpo_loss_fwd_noalloc(p, p, p, 1, p, p, p, 8, 20480, 4096, 128256, f, p, p,
                                     nul, nul, nul, p, nul, nul) == -9


def test_offload_options_validated(lib):
    """Gradient offload: host buffers need a copy stream other than the call's stream, the
    offload takes dXq NULL (and dW for dw_host), the workspace grows by two staging slots
    of a chunk's rows, and grpo_grad_restore checks its arguments, all before any launch."""
    import grpo_loss_amd as g
    p = ctypes.c_void_p(256)
    cs = ctypes.c_void_p(4096)
    nul = None
    f = ctypes.c_float
    S, L, H, V = 8, 20480, 4096, 128256
    base = lib.grpo_workspace_bytes_opts(S, L, H, V, 1, 0, None)
    o = g.options()
    o.dx_host = 512
    assert lib.grpo_workspace_bytes_opts(S, L, H, V, 1, 0, ctypes.byref(o)) == 0  # no stream
    o.copy_stream = cs.value
    grown = lib.grpo_workspace_bytes_opts(S, L, H, V, 1, 0, ctypes.byref(o))
    assert grown - base == 2 * 4096 * H * 2
    o.dx_host = 520                                    # not 16-byte aligned
    assert lib.grpo_workspace_bytes_opts(S, L, H, V, 1, 0, ctypes.byref(o)) == 0
    o.dx_host = 512

    def fb(dXq, dW, opts, stream, ws=1 << 40):
        return lib.grpo_loss_fwd_bwd(p, p, p, 1, p, p, p, 2, 3, 256, 5, f(0.04), nul, f(1.0), p,
                                     p, nul, nul, nul, p, dXq, dW, 0, p, opts, p,
                                     ctypes.c_size_t(ws), stream)
    assert fb(p, nul, ctypes.byref(o), nul) == -8      # dXq given with dx_host
    assert fb(nul, nul, ctypes.byref(o), cs) == -8     # copy stream == call stream
    o2 = g.options()
    o2.dw_host, o2.copy_stream = 512, cs.value
    assert fb(p, nul, ctypes.byref(o2), nul) == -8     # dw_host without a device dW
    assert fb(nul, nul, None, nul) == -1               # no dXq, no offload
    # valid arguments get as far as the device check (no GPU here)
    assert fb(nul, nul, ctypes.byref(o), nul) == -7
    # restore
    rb = lib.grpo_restore_workspace_bytes(1, 1000)
    assert rb >= 2 * 1000 * 4
    assert lib.grpo_restore_workspace_bytes(0, 1000) == 0

    def rs(dxh, dwh, dX, dW, ws=1 << 40, H=256, mask=p):
        return lib.grpo_grad_restore(dxh, dwh, 1, mask, 1, 1000, H, 50, nul, f(1.0), dX, dW, p,
                                     p, ctypes.c_size_t(ws), nul)
    assert rs(p, nul, nul, nul) == -1                  # dx_host without dXq
    assert rs(nul, nul, nul, nul) == -1                # nothing to restore
    assert rs(p, nul, p, nul, mask=nul) == -1          # dX needs the mask
    assert rs(p, nul, p, nul, H=100) == -2
    assert rs(p, nul, p, nul, ws=8) == -5
    assert rs(ctypes.c_void_p(264), nul, p, nul) == -4
    assert rs(p, p, p, p) == -7                        # valid: as far as the device check
