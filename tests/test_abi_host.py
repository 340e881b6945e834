"""Host-side checks of the C ABI (no GPU needed: every call here returns before
anything is enqueued)."""
import ctypes
import os
import re
import subprocess

import pytest

import frame_wise_delta_gram_amd as vda

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "vda.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(vda.LIB_PATH):
        pytest.skip("libvda.so not built")
    return vda.load_library()


def header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(vda_[a-z_]+)\s*\(", src)))


def test_header_declares_the_binding_surface():
    assert header_functions() == sorted(vda.EXPORTED)


def test_descriptor_layout_matches_header():
    src = open(HEADER).read()
    body = re.search(r"typedef struct vda_desc \{(.*?)\} vda_desc_t;", src, flags=re.S).group(1)
    body = re.sub(r"/\*.*?\*/", "", body, flags=re.S)
    fields = re.findall(r"(int32_t|float)\s+(\w+);", body)
    assert [n for _, n in fields] == [n for n, _ in vda.VdaDesc._fields_]
    assert ctypes.sizeof(vda.VdaDesc) == 4 * len(fields)


def test_prep_descriptor_layout_matches_header():
    src = open(HEADER).read()
    body = re.search(r"typedef struct vda_prep_desc \{(.*?)\} vda_prep_desc_t;", src,
                     flags=re.S).group(1)
    body = re.sub(r"/\*.*?\*/", "", body, flags=re.S)
    fields = re.findall(r"(int32_t|float)\s+(\w+);", body)
    assert [n for _, n in fields] == [n for n, _ in vda.VdaPrepDesc._fields_]
    assert ctypes.sizeof(vda.VdaPrepDesc) == 4 * len(fields)


def prep_desc(**kw):
    base = dict(batch=2, heads=3, frames=7, height=9, width=13, d_k=64, d_v=32, eps=1e-6,
                dtype=vda.VDA_DTYPE_BF16)
    base.update(kw)
    return vda.make_prep_desc(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(), vda.VDA_OK),
    (dict(batch=-1), vda.VDA_ERR_INVALID_ARG),
    (dict(width=-2), vda.VDA_ERR_INVALID_ARG),
    (dict(d_k=24), vda.VDA_ERR_INVALID_ARG),
    (dict(d_v=256), vda.VDA_ERR_INVALID_ARG),
    (dict(eps=0.0), vda.VDA_ERR_INVALID_ARG),
    (dict(eps=float("nan")), vda.VDA_ERR_INVALID_ARG),
    (dict(dtype=5), vda.VDA_ERR_BAD_DTYPE),
    (dict(batch=300, heads=300), vda.VDA_ERR_INVALID_ARG),
    (dict(height=2048, width=2048), vda.VDA_ERR_INVALID_ARG),
    (dict(frames=(1 << 20) + 1), vda.VDA_ERR_INVALID_ARG),
    # the convolution grid: a K and a V workgroup per (unit, 8 x 8 tile) must
    # stay under 2^22 workgroups with the Q pass's 1024 (2,096,000 sweeps pass,
    # 2,097,000 do not)
    (dict(batch=1000, heads=1, height=8, width=8 * 2096), vda.VDA_OK),
    (dict(batch=1000, heads=1, height=8, width=8 * 2097), vda.VDA_ERR_INVALID_ARG),
    (dict(batch=0), vda.VDA_OK),
    (dict(height=0), vda.VDA_OK),
])
def test_prep_descriptor_checks(lib, kw, status):
    assert vda.vda_prep_check_desc(prep_desc(**kw)) == status


def test_prep_argument_errors(lib):
    d = prep_desc()
    P = [4096 * (i + 1) for i in range(10)]
    assert lib.vda_prep(ctypes.byref(d), None, *P[1:], None) == vda.VDA_ERR_INVALID_ARG
    # q and q_out are left out together or not at all
    assert lib.vda_prep(ctypes.byref(d), *P[:7], None, *P[8:], None) == vda.VDA_ERR_INVALID_ARG
    assert lib.vda_prep(ctypes.byref(d), *P[:9], None, None) == vda.VDA_ERR_INVALID_ARG
    assert lib.vda_prep(ctypes.byref(d), P[0] + 8, *P[1:], None) == vda.VDA_ERR_MISALIGNED
    assert lib.vda_prep(ctypes.byref(d), *P[:3], P[3] + 2, *P[4:], None) == \
        vda.VDA_ERR_MISALIGNED
    assert lib.vda_prep(None, *P, None) == vda.VDA_ERR_INVALID_ARG
    e = prep_desc(frames=0)
    assert lib.vda_prep(ctypes.byref(e), *([None] * 10), None) == vda.VDA_OK


def test_package_exposes_every_entry_point():
    for name in vda.EXPORTED:
        assert callable(getattr(vda, name, None)), name


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", vda.LIB_PATH], stdout=subprocess.PIPE,
                         text=True, check=True).stdout
    exported = set(re.findall(r" T (vda_[a-z_]+)$", out, flags=re.M))
    for name in header_functions():
        assert name in exported, name
        assert hasattr(lib, name)


def desc(**kw):
    base = dict(units=2, frames=12, tokens=40, text_tokens=7, d_k=64, d_v=32, chunk=5, radius=1,
                rms_eps=1e-6, seed_mode=0, dtype=vda.VDA_DTYPE_BF16)
    base.update(kw)
    return vda.make_desc(**base)


def test_workspace_formula(lib):
    d = desc()
    n = 3
    def a(x):
        return (x + 255) // 256 * 256
    units, Fp1, dk, dv = 2, 13, 64, 32
    expect = (a(units * Fp1 * dk * dk * 4) + a(units * Fp1 * dv * dk * 4) + a(units * Fp1 * dk * dk * 4)
              + a(units * n * dk * dk * 4) + 2 * a(units * n * dv * dk * 4)
              + a(units * 2 * (n + 1) * dv * dk * 4) + a(units * n * dk * dk * 4)
              + a(units * n * dk * dk * 4))  # Mc^T and the reverse transitions (decay)
    assert vda.vda_workspace_bytes(d) == expect
    # bf16 with d_k = d_v = 128 adds the readout's split S~ images (69632 bytes per chunk)
    d128 = desc(d_k=128, d_v=128)
    kk = 128 * 128 * 4
    expect128 = (a(units * Fp1 * kk) * 3 + a(units * n * kk) * 3 + 2 * a(units * n * kk)
                 + a(units * 2 * (n + 1) * kk) + a(units * n * 2 * 128 * 136 * 2))
    assert vda.vda_workspace_bytes(d128) == expect128
    assert vda.vda_workspace_bytes(desc(d_k=128, d_v=128, dtype=vda.VDA_DTYPE_F32)) == \
        expect128 - a(units * n * 2 * 128 * 136 * 2)
    assert vda.vda_workspace_bytes(desc(units=0)) == 0
    assert vda.vda_workspace_bytes(desc(frames=0)) == 0
    assert vda.vda_workspace_bytes(desc(d_k=12)) == 0  # invalid -> 0
    assert lib.vda_workspace_bytes(None) == 0


@pytest.mark.parametrize("kw,status", [
    (dict(), vda.VDA_OK),
    (dict(d_k=8), vda.VDA_ERR_INVALID_ARG),
    (dict(d_k=144), vda.VDA_ERR_INVALID_ARG),
    (dict(d_v=24), vda.VDA_ERR_INVALID_ARG),
    (dict(chunk=0), vda.VDA_ERR_INVALID_ARG),
    (dict(radius=-1), vda.VDA_ERR_INVALID_ARG),
    (dict(units=-1), vda.VDA_ERR_INVALID_ARG),
    (dict(tokens=-5), vda.VDA_ERR_INVALID_ARG),
    (dict(rms_eps=-1.0), vda.VDA_ERR_INVALID_ARG),
    (dict(rms_eps=float("nan")), vda.VDA_ERR_INVALID_ARG),
    (dict(rms_eps=float("inf")), vda.VDA_ERR_INVALID_ARG),
    (dict(seed_mode=2), vda.VDA_ERR_INVALID_ARG),
    (dict(anchors=2), vda.VDA_ERR_INVALID_ARG),
    (dict(anchors=1), vda.VDA_OK),
    (dict(rule=1), vda.VDA_OK),
    (dict(rule=2), vda.VDA_OK),
    (dict(rule=3), vda.VDA_ERR_INVALID_ARG),
    (dict(fp32_products=2), vda.VDA_ERR_INVALID_ARG),
    (dict(fp32_products=-1), vda.VDA_ERR_INVALID_ARG),
    (dict(solver=2), vda.VDA_ERR_INVALID_ARG),
    (dict(solver=1, rule=1), vda.VDA_ERR_INVALID_ARG),
    (dict(rule=-1), vda.VDA_ERR_INVALID_ARG),
    (dict(units=70000), vda.VDA_ERR_INVALID_ARG),
    (dict(tokens=4194304), vda.VDA_ERR_INVALID_ARG),
    (dict(text_tokens=4194304), vda.VDA_ERR_INVALID_ARG),
    (dict(tokens=4194303, units=1, frames=1), vda.VDA_OK),
    (dict(units=65535, frames=20000), vda.VDA_ERR_INVALID_ARG),
    (dict(units=1, frames=1048577, chunk=100, tokens=1), vda.VDA_ERR_INVALID_ARG),
    (dict(units=1, frames=1048576, chunk=100, tokens=1), vda.VDA_OK),
    # readout grid: units x chunks x 512-row blocks below 2^22 (64 x 3400 x 20 > 2^22,
    # 64 x 3200 x 20 < 2^22)
    (dict(units=64, frames=17000, chunk=5, tokens=2048), vda.VDA_ERR_INVALID_ARG),
    (dict(units=64, frames=16000, chunk=5, tokens=2048), vda.VDA_OK),
    (dict(dtype=7), vda.VDA_ERR_BAD_DTYPE),
    (dict(units=0, frames=0, tokens=0), vda.VDA_OK),
    (dict(d_k=16, d_v=128), vda.VDA_OK),
    # the query map: q_heads divides units (0 and 1 mean the unit layout), q_l2_eps
    # is 0 or a finite normal float
    (dict(q_heads=2), vda.VDA_OK),
    (dict(q_heads=1, q_l2_eps=1e-6), vda.VDA_OK),
    (dict(q_heads=3), vda.VDA_ERR_INVALID_ARG),
    (dict(q_heads=-1), vda.VDA_ERR_INVALID_ARG),
    (dict(q_heads=70000), vda.VDA_ERR_INVALID_ARG),
    (dict(q_l2_eps=-1e-6), vda.VDA_ERR_INVALID_ARG),
    (dict(q_l2_eps=float("nan")), vda.VDA_ERR_INVALID_ARG),
    (dict(q_l2_eps=float("inf")), vda.VDA_ERR_INVALID_ARG),
    (dict(q_l2_eps=1e-40), vda.VDA_ERR_INVALID_ARG),
    (dict(q_l2_eps=1.1754944e-38), vda.VDA_OK),
])
def test_descriptor_checks(lib, kw, status):
    assert vda.vda_check_desc(desc(**kw)) == status


def test_out_dtype_must_match(lib):
    d = desc()
    d.out_dtype = vda.VDA_DTYPE_F32
    assert vda.vda_check_desc(d) == vda.VDA_ERR_BAD_DTYPE


def call_forward(lib, d, **ptrs):
    names = ["q", "k", "v", "beta", "gate", "text_k", "text_v", "text_beta", "rms_weight", "out",
             "workspace"]
    args = [ptrs.get(n, 4096 * (i + 1)) for i, n in enumerate(names)]
    ws_bytes = ptrs.get("ws_bytes", vda.vda_workspace_bytes(d))
    return lib.vda_forward(ctypes.byref(d), *args, ws_bytes, None)


def test_forward_argument_errors(lib):
    d = desc()
    assert call_forward(lib, d, k=None) == vda.VDA_ERR_INVALID_ARG
    assert call_forward(lib, d, q=None) == vda.VDA_ERR_INVALID_ARG
    assert call_forward(lib, d, text_v=None) == vda.VDA_ERR_INVALID_ARG
    assert call_forward(lib, d, workspace=None) == vda.VDA_ERR_INVALID_ARG
    assert call_forward(lib, d, ws_bytes=vda.vda_workspace_bytes(d) - 1) == \
        vda.VDA_ERR_WORKSPACE_TOO_SMALL
    assert call_forward(lib, d, q=4096 + 8) == vda.VDA_ERR_MISALIGNED
    assert call_forward(lib, d, workspace=4096 + 128) == vda.VDA_ERR_MISALIGNED
    assert call_forward(lib, d, rms_weight=4096 + 4) == vda.VDA_ERR_MISALIGNED
    assert lib.vda_forward(None, *([None] * 11), 0, None) == vda.VDA_ERR_INVALID_ARG
    # empty problems need no pointers at all and enqueue nothing
    e = desc(units=0)
    assert lib.vda_forward(ctypes.byref(e), *([None] * 11), 0, None) == vda.VDA_OK
    e = desc(frames=0)
    assert lib.vda_forward(ctypes.byref(e), *([None] * 11), 0, None) == vda.VDA_OK


def test_debug_tap_argument_errors(lib):
    d = desc()
    P = [4096 * (i + 1) for i in range(9)]
    ws = vda.vda_workspace_bytes(d)
    assert lib.vda_debug_stats(ctypes.byref(d), None, *P[1:8], P[8], ws, None) == \
        vda.VDA_ERR_INVALID_ARG
    assert lib.vda_debug_solve(ctypes.byref(d), *P[:6], None, P[7], P[8], ws, None) == \
        vda.VDA_ERR_INVALID_ARG
    assert lib.vda_debug_chunks(ctypes.byref(d), *P[:6], P[6], P[7], None, P[8], ws, None) == \
        vda.VDA_ERR_INVALID_ARG
    assert lib.vda_debug_states(ctypes.byref(d), *P[:8], P[8], ws - 256, None) == \
        vda.VDA_ERR_WORKSPACE_TOO_SMALL


def call_forward_decay(lib, d, **ptrs):
    names = ["q", "k", "v", "beta", "alpha", "gate", "text_k", "text_v", "text_beta",
             "rms_weight", "out", "workspace"]
    args = [ptrs.get(n, 4096 * (i + 1)) for i, n in enumerate(names)]
    ws_bytes = ptrs.get("ws_bytes", vda.vda_workspace_bytes(d))
    return lib.vda_forward_decay(ctypes.byref(d), *args, ws_bytes, None)


def test_forward_decay_argument_errors(lib):
    d = desc()
    assert call_forward_decay(lib, d, alpha=None) == vda.VDA_ERR_INVALID_ARG
    assert call_forward_decay(lib, d, alpha=4096 + 4) == vda.VDA_ERR_MISALIGNED
    assert call_forward_decay(lib, d, k=None) == vda.VDA_ERR_INVALID_ARG
    assert call_forward_decay(lib, d, ws_bytes=vda.vda_workspace_bytes(d) - 1) == \
        vda.VDA_ERR_WORKSPACE_TOO_SMALL
    bad = desc(d_k=12)
    assert call_forward_decay(lib, bad) == vda.VDA_ERR_INVALID_ARG
    # the batched comparison rules run without decay
    assert call_forward_decay(lib, desc(rule=1)) == vda.VDA_ERR_INVALID_ARG
    # empty problems need no gates
    e = desc(units=0)
    assert lib.vda_forward_decay(ctypes.byref(e), *([None] * 12), 0, None) == vda.VDA_OK
    # one segment per frame: a problem whose per-chunk readout grid fits but whose
    # per-frame grid (units x frames x 512-row blocks) does not is refused by the
    # decay entry points only: 64 x 8000 chunks x 6 blocks < 2^22 <= 64 x 40000 x 2
    big = desc(units=64, frames=40000, tokens=513, text_tokens=0)
    assert vda.vda_check_desc(big) == vda.VDA_OK
    assert call_forward_decay(lib, big) == vda.VDA_ERR_INVALID_ARG
    P = [4096 * (i + 1) for i in range(12)]
    ws = vda.vda_workspace_bytes(d)
    assert lib.vda_debug_chunks_decay(ctypes.byref(d), *P[:3], None, *P[4:11], P[11], ws,
                                      None) == vda.VDA_ERR_INVALID_ARG
    assert lib.vda_debug_chunks_decay(ctypes.byref(d), *P[:8], None, *P[9:11], P[11], ws,
                                      None) == vda.VDA_ERR_INVALID_ARG
    assert lib.vda_debug_states_decay(ctypes.byref(d), *P[:3], None, *P[4:9], P[11], ws,
                                      None) == vda.VDA_ERR_INVALID_ARG


def test_frame_maps_tap_host_checks(lib):
    """vda_debug_frame_maps refuses the batched rules, missing outputs and a
    misaligned flag before anything is enqueued (no GPU here: nothing is)."""
    import ctypes
    fake = ctypes.c_void_p(1 << 20)  # never dereferenced: every call fails its checks first
    d = desc()
    ws_bytes = vda.vda_workspace_bytes(d)
    P = [fake] * 6
    assert lib.vda_debug_frame_maps(ctypes.byref(desc(rule=1)), *P, fake, fake, None, fake,
                                    ws_bytes, None) == vda.VDA_ERR_INVALID_ARG
    assert lib.vda_debug_frame_maps(ctypes.byref(d), *P, None, fake, None, fake, ws_bytes,
                                    None) == vda.VDA_ERR_INVALID_ARG
    assert lib.vda_debug_frame_maps(ctypes.byref(d), *P, fake, None, None, fake, ws_bytes,
                                    None) == vda.VDA_ERR_INVALID_ARG
    assert lib.vda_debug_frame_maps(ctypes.byref(d), *P, fake, fake, ctypes.c_void_p((1 << 20) + 2),
                                    fake, ws_bytes, None) == vda.VDA_ERR_MISALIGNED
    assert lib.vda_debug_frame_maps(None, *P, fake, fake, None, fake, ws_bytes,
                                    None) == vda.VDA_ERR_INVALID_ARG


def test_status_strings(lib):
    for s in (0, -1, -2, -3, -4, -5, -6, -7):
        assert vda.vda_status_string(s) and vda.vda_status_string(s) != "unknown status"
    assert "positive definite" in vda.vda_status_string(vda.VDA_ERR_NOT_SPD)
    assert vda.vda_status_string(42) == "unknown status"


# ---- argument checks of the torch-level forward() (binding.py): every
# mismatch raises before the library is asked to enqueue anything.  This
# container has no GPU, so every non-empty tensor here is a CPU tensor, which
# forward() refuses by name; the empty-problem cases reach the library, which
# returns without touching a GPU.
def _tensors(units=2, F=3, U=4, dk=16, dv=16, T=2, dtype=None):
    import torch
    dt = dtype or torch.bfloat16
    return dict(q=torch.zeros(units, F, U, dk, dtype=dt), k=torch.zeros(units, F, U, dk, dtype=dt),
                v=torch.zeros(units, F, U, dv, dtype=dt), beta=torch.zeros(units, F, U),
                gate=torch.zeros(units, F, U, dv, dtype=dt),
                text_k=torch.zeros(units, T, dk, dtype=dt),
                text_v=torch.zeros(units, T, dv, dtype=dt), text_beta=torch.zeros(units, T),
                rms_weight=torch.ones(dv))


def _call(t, **kw):
    return vda.forward(t["q"], t["k"], t["v"], t["beta"], t["gate"], t["text_k"], t["text_v"],
                       t["text_beta"], t["rms_weight"], stream=0, **kw)


def test_torch_forward_rejects_host_and_misshapen_tensors(lib):
    import torch
    t = _tensors()
    with pytest.raises(ValueError, match="^k must be a contiguous GPU tensor"):
        _call(t)  # k is checked first: the descriptor comes from its shape
    bad = dict(t, k=torch.zeros(2, 3, 4, 16, dtype=torch.float16))
    with pytest.raises(TypeError):
        _call(bad)
    with pytest.raises(TypeError):
        _call(dict(t, k=[[0.0]]))
    # an empty problem (units = 0) passes the device checks, so the shape and
    # dtype checks of everything else are reached
    e = _tensors(units=0)
    with pytest.raises(ValueError, match="^q: expected shape"):
        _call(dict(e, q=torch.zeros(0, 3, 4, 32, dtype=torch.bfloat16)))
    with pytest.raises(ValueError, match="^out: expected shape"):
        _call(e, out=torch.zeros(0, 3, 4, 32, dtype=torch.bfloat16))
    with pytest.raises(TypeError, match="^out: expected"):
        _call(e, out=torch.zeros(0, 3, 4, 16, dtype=torch.float32))
    with pytest.raises(TypeError, match="^workspace"):
        _call(e, workspace=torch.zeros(16, dtype=torch.float32))
    with pytest.raises(TypeError, match="^alpha"):
        _call(e, alpha=torch.zeros(0, 3, 16, dtype=torch.float64))
    with pytest.raises(ValueError, match="^text_v: expected shape"):
        _call(dict(e, text_v=torch.zeros(0, 5, 16, dtype=torch.bfloat16)))
    with pytest.raises(ValueError, match="all None"):
        _call(dict(e, text_v=None))
    with pytest.raises(TypeError, match="^text_k"):
        _call(dict(e, text_k=torch.zeros(2, dtype=torch.bfloat16)))


def test_torch_forward_accepts_no_text(lib):
    e = _tensors(units=0)
    out = _call(dict(e, text_k=None, text_v=None, text_beta=None))
    assert tuple(out.shape) == (0, 3, 4, 16)


def call_noalloc(lib, d, **ptrs):
    names = ["q", "k", "v", "beta", "gate", "text_k", "text_v", "text_beta", "rms_weight", "out"]
    args = [ptrs.get(n, 4096 * (i + 1)) for i, n in enumerate(names)]
    return lib.vda_forward_noalloc(ctypes.byref(d), *args, None)


def test_noalloc_host_checks(lib):
    """vda_forward_noalloc refuses, on the host and before any GPU call, every
    problem whose workspace exceeds its fixed scratch, and checks its pointers
    like vda_forward (this container has no GPU: any call that got past the
    checks would report a HIP error)."""
    assert vda.VDA_NOALLOC_MAX_BYTES == 64 << 20
    small = desc()
    assert vda.vda_workspace_bytes(small) <= vda.VDA_NOALLOC_MAX_BYTES
    # the 768p head share needs 420 MB
    big = desc(units=16, frames=90, tokens=4032, text_tokens=512, d_k=128, d_v=128)
    assert vda.vda_workspace_bytes(big) > vda.VDA_NOALLOC_MAX_BYTES
    assert call_noalloc(lib, big) == vda.VDA_ERR_SCRATCH_TOO_SMALL
    # the largest problem of a family that fits, and the next one up
    fits = [f for f in range(1, 200)
            if vda.vda_workspace_bytes(desc(units=4, frames=f, d_k=128, d_v=128))
            <= vda.VDA_NOALLOC_MAX_BYTES]
    f = max(fits)
    assert f < 199
    assert call_noalloc(lib, desc(units=4, frames=f + 1, d_k=128, d_v=128)) == \
        vda.VDA_ERR_SCRATCH_TOO_SMALL
    assert call_noalloc(lib, small, k=None) == vda.VDA_ERR_INVALID_ARG
    assert call_noalloc(lib, small, out=None) == vda.VDA_ERR_INVALID_ARG
    assert call_noalloc(lib, small, q=4096 + 8) == vda.VDA_ERR_MISALIGNED
    assert call_noalloc(lib, desc(d_k=12)) == vda.VDA_ERR_INVALID_ARG
    assert lib.vda_forward_noalloc(None, *([None] * 10), None) == vda.VDA_ERR_INVALID_ARG
    e = desc(units=0)
    assert lib.vda_forward_noalloc(ctypes.byref(e), *([None] * 10), None) == vda.VDA_OK
    assert "scratch" in vda.vda_status_string(vda.VDA_ERR_SCRATCH_TOO_SMALL)
