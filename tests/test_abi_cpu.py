"""CPU-side checks of the C ABI: the library loads, exports every declared
symbol, sizes its workspace, and rejects bad arguments before touching the GPU.
No compute call is made here."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "adaflash.h")


@pytest.fixture(scope="module")
def lib():
    import diffusion_drafter_verification_amd as ada
    if not os.path.exists(ada.LIB_PATH):
        from diffusion_drafter_verification_amd import build
        build.build()
    return ada.load_library()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"ADAFLASH_API\s+[\w\s\*]*?\b(adaflash_\w+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("adaflash_verify", "adaflash_opd_loss_fwd_bwd", "adaflash_workspace_bytes",
              "adaflash_last_error", "adaflash_version"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for n in declared_functions():
        assert hasattr(lib, n), n


def test_only_the_abi_is_exported():
    import subprocess
    import diffusion_drafter_verification_amd as ada
    out = subprocess.run(["nm", "-D", "--defined-only", ada.LIB_PATH], capture_output=True, text=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    assert {n for n in exported if "adaflash" in n} == set(declared_functions())


def test_version(lib):
    assert lib.adaflash_version() >= 100


def test_workspace_bytes(lib):
    assert lib.adaflash_workspace_bytes(128, 16, 151936) > 0
    assert lib.adaflash_workspace_bytes(0, 16, 151936) > 0     # empty batch still valid
    assert lib.adaflash_workspace_bytes(4, 0, 64) == 0          # k < 1
    assert lib.adaflash_workspace_bytes(4, 65, 64) == 0         # k > 64
    assert lib.adaflash_workspace_bytes(4, 16, 0) == 0          # V < 1
    assert lib.adaflash_workspace_bytes(-1, 16, 64) == 0
    assert lib.adaflash_workspace_bytes(4, 16, (1 << 20) + 1) == 0
    # Grows with the batch and the vocabulary.
    assert lib.adaflash_workspace_bytes(256, 16, 151936) > lib.adaflash_workspace_bytes(128, 16, 151936)
    assert lib.adaflash_workspace_bytes(128, 16, 300000) > lib.adaflash_workspace_bytes(128, 16, 151936)


FAKE = 0x1000  # never dereferenced: every call below fails validation first


def _verify(lib, **kw):
    args = dict(dtype=1, target=FAKE, draft=FAKE, tokens=FAKE, vl=FAKE, uni=FAKE, B=2, k=4, V=64, T=1.0,
                acc=FAKE, out=FAKE, mg=None, c=10.0, lam=1.0, ro=FAKE, ce=None, rk=None, g=None, st=None,
                ws=FAKE, wsb=1 << 30, stream=None)
    args.update(kw)
    a = args
    return lib.adaflash_verify(a["dtype"], a["target"], a["draft"], a["tokens"], a["vl"], a["uni"], a["B"],
                               a["k"], a["V"], a["T"], a["acc"], a["out"], a["mg"], a["c"], a["lam"], a["ro"],
                               a["ce"], a["rk"], a["g"], a["st"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(T=-1.0), -1), (dict(T=float("nan")), -1), (dict(T=float("inf")), -1),
    (dict(k=0), -1), (dict(k=65), -1), (dict(V=0), -1), (dict(B=-3), -1),
    (dict(dtype=7), -1), (dict(ro=None), -1), (dict(target=None), -1),
    (dict(draft=None), -1),                      # T > 0 needs draft logits
    (dict(uni=None), -1), (dict(tokens=None), -1), (dict(acc=None), -1),
    (dict(ws=None), -2), (dict(wsb=16), -2),
    (dict(ce=FAKE, c=0.0), -1), (dict(ce=FAKE, c=-1.0), -1), (dict(g=FAKE, lam=-0.5), -1),
    (dict(g=FAKE, lam=float("inf")), -1),
])
def test_verify_rejects_bad_arguments(lib, kw, code):
    assert _verify(lib, **kw) == code
    assert len(lib.adaflash_last_error()) > 0


def test_greedy_without_supervision_needs_no_draft_logits(lib):
    # Validation passes a NULL draft at T == 0; the bad workspace size then fails it.
    assert _verify(lib, T=0.0, draft=None, uni=None, wsb=16) == -2


def test_opd_rejects_bad_arguments(lib):
    f = lib.adaflash_opd_loss_fwd_bwd
    ok = dict(dtype=1, t=FAKE, d=FAKE, vl=None, B=2, k=4, V=64, c=10.0, lam=1.0, ro=FAKE, ce=None, rk=None,
              g=None, st=None, ws=FAKE, wsb=1 << 30, stream=None)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return f(a["dtype"], a["t"], a["d"], a["vl"], a["B"], a["k"], a["V"], a["c"], a["lam"], a["ro"],
                 a["ce"], a["rk"], a["g"], a["st"], a["ws"], a["wsb"], a["stream"])

    assert call(c=0.0) == -1
    assert call(lam=-1.0) == -1
    assert call(d=None) == -1
    assert call(ro=None) == -1
    assert call(wsb=0) == -2
    assert call(k=100) == -1


# ------------------------------------------------------------- length head

def test_length_head_workspace_bytes(lib):
    f = lib.adaflash_length_head_workspace_bytes
    f.restype = ctypes.c_size_t
    assert f(128, 16, 4096, 256) > 0
    assert f(0, 16, 4096, 256) > 0
    assert f(4, 16, 4096 + 8, 256) == 0     # H not a multiple of 16
    assert f(4, 16, 8, 256) == 0            # H < 16
    assert f(4, 0, 64, 8) == 0
    assert f(4, 65, 64, 8) == 0
    assert f(4, 16, 64, 0) == 0
    assert f(4, 16, 64, 8193) == 0
    assert f(256, 16, 4096, 256) > f(128, 16, 4096, 256)


FAKE_ALIGNED = 0x10000


@pytest.mark.parametrize("kw,code", [
    (dict(H=24), -1), (dict(k=0), -1), (dict(Hp=0), -1), (dict(gamma=0.0), -1), (dict(gamma=float("inf")), -1),
    (dict(h=None), -1), (dict(h=FAKE_ALIGNED + 2), -1), (dict(W1=FAKE_ALIGNED + 8), -1),
    (dict(ws=None), -2), (dict(wsb=16), -2), (dict(b2=float("nan")), -1), (dict(a_hat=None, k_hat=None), -1),
])
def test_length_head_forward_rejects_bad_arguments(lib, kw, code):
    a = dict(h=FAKE_ALIGNED, W1=FAKE_ALIGNED, b1=FAKE_ALIGNED, w2=FAKE_ALIGNED, b2=0.0, B=4, k=16, H=64, Hp=8,
             gamma=1.0, a_hat=FAKE_ALIGNED, k_hat=FAKE_ALIGNED, ws=FAKE_ALIGNED, wsb=1 << 30)
    a.update(kw)
    f = lib.adaflash_length_head_forward
    vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    f.restype = i32
    f.argtypes = [vp, vp, vp, vp, f32, i32, i32, i32, i32, f32, vp, vp, vp, sz, vp]
    rc = f(a["h"], a["W1"], a["b1"], a["w2"], a["b2"], a["B"], a["k"], a["H"], a["Hp"], a["gamma"], a["a_hat"],
           a["k_hat"], a["ws"], a["wsb"], None)
    assert rc == code
    lib.adaflash_last_error.restype = ctypes.c_char_p
    assert lib.adaflash_last_error()


def test_length_head_backward_rejects_bad_arguments(lib):
    f = lib.adaflash_length_head_backward
    vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    f.restype = i32
    f.argtypes = [vp, vp, vp, vp, f32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    P = FAKE_ALIGNED
    # Missing gradient outputs, missing accept lengths, bad sizes: rejected before any launch.
    assert f(P, P, P, P, 0.0, 4, 16, 64, 8, P, P, P, None, P, P, P, P, 1 << 30, None) == -1
    assert f(P, P, P, P, 0.0, 4, 16, 64, 8, None, P, P, P, P, P, P, P, 1 << 30, None) == -1
    assert f(P, P, P, P, 0.0, 4, 16, 40, 8, P, P, P, P, P, P, P, P, 1 << 30, None) == -1
    assert f(P, P, P, P, 0.0, 4, 16, 64, 8, P, P, P, P, P, P, P, P, 16, None) == -2


# ----------------------------------------------------------- loss variants

@pytest.mark.parametrize("variant,p1,p2,code", [
    (0, 0.0, 0.0, -1), (6, 0.0, 0.0, -1), (2, 0.0, 0.0, -1), (2, float("inf"), 0.0, -1),
    (3, 1.5, 0.01, -1), (3, 0.8, 0.0, -1), (5, 0.0, 0.0, -1), (5, float("nan"), 0.0, -1),
])
def test_loss_variant_rejects_bad_arguments(lib, variant, p1, p2, code):
    f = lib.adaflash_loss_variant_fwd_bwd
    vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    f.restype = i32
    f.argtypes = [i32, vp, vp, vp, i32, i32, i32, i32, f32, f32, vp, vp, vp, vp, vp, sz, vp]
    P = 0x10000
    rc = f(1, P, P, None, 4, 16, 64, variant, p1, p2, P, P, P, None, P, 1 << 30, None)
    assert rc == code


# ------------------------------------------- packed forms, cached head, timing

def test_packed_and_cached_forms_reject_bad_arguments(lib):
    vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    P = FAKE_ALIGNED
    f = lib.adaflash_opd_loss_fwd_bwd_packed
    f.restype = i32
    f.argtypes = [i32, vp, vp, vp, i32, i32, i32, f32, f32, vp, vp, vp, vp, vp, vp, sz, vp]
    assert f(1, P, P, P, 4, 16, 1000, 0.0, 1.0, P, P, P, P, P, P, 1 << 30, None) == -1  # clip c <= 0
    assert f(1, P, P, P, 4, 16, 1000, 1.0, 1.0, None, P, P, P, P, P, 1 << 30, None) == -1  # no row_offsets
    g = lib.adaflash_length_head_forward_cached
    g.restype = i32
    g.argtypes = [vp, vp, vp, vp, f32, i32, i32, i32, i32, f32, vp, vp, vp, vp, sz, vp]
    assert g(P, P, P, P, 0.0, 4, 16, 64, 8, 1.0, P, P, None, P, 1 << 30, None) == -1  # no z1 cache
    h = lib.adaflash_length_head_backward_cached
    h.restype = i32
    h.argtypes = [vp, vp, vp, vp, f32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    assert h(P, P, P, P, 0.0, 4, 16, 64, 8, P, P, P, P, P, P, P, None, P, 1 << 30, None) == -1


def test_timing_hook_argument_checks(lib):
    lib.adaflash_timing_enable.restype = ctypes.c_int
    lib.adaflash_timing_enable.argtypes = [ctypes.c_int]
    lib.adaflash_timing_read.restype = ctypes.c_int
    lib.adaflash_timing_read.argtypes = [ctypes.c_void_p, ctypes.c_int]
    assert lib.adaflash_timing_enable(-1) == -1
    assert lib.adaflash_timing_enable(0) == 0  # disabling creates nothing
    assert lib.adaflash_timing_read(None, 4) == -1
    assert lib.adaflash_timing_read(None, 0) == 0  # nothing recorded
    lib.adaflash_timing_every.restype = ctypes.c_int
    lib.adaflash_timing_every.argtypes = [ctypes.c_int]
    assert lib.adaflash_timing_every(0) == -1
    assert lib.adaflash_timing_every(1) == 0


# ---------------------------------------------- binding argument checks

def _good_verify_args(B=3, k=4, V=64, dt=None):
    import torch
    dt = dt or torch.bfloat16
    return dict(target=torch.zeros(B, k + 1, V, dtype=dt), draft=torch.zeros(B, k, V, dtype=dt),
                tokens=torch.zeros(B, k, dtype=torch.int32), verify_len=torch.ones(B, dtype=torch.int32),
                uniforms=torch.zeros(B, k + 1), T=1.0, accept_len=torch.zeros(B, dtype=torch.int32),
                out_tokens=torch.zeros(B, k + 1, dtype=torch.int32), margins=torch.zeros(B, k + 1),
                clip_c=10.0, lam=1.0, row_offsets=torch.zeros(B + 1, dtype=torch.int32),
                loss_ce=torch.zeros(B * k), loss_rkl=torch.zeros(B * k),
                grad_draft=torch.zeros(B * k, V, dtype=dt), status=torch.zeros(1, dtype=torch.int32),
                ws=torch.zeros(16, dtype=torch.uint8))


@pytest.mark.parametrize("name,bad,exc,what", [
    ("tokens", lambda a: a["tokens"].long(), TypeError, "tokens"),
    ("verify_len", lambda a: a["verify_len"].long(), TypeError, "verify_len"),
    ("uniforms", lambda a: a["uniforms"][:, :-1].contiguous(), ValueError, "uniforms"),
    ("uniforms", lambda a: a["uniforms"].double(), TypeError, "uniforms"),
    ("draft", lambda a: a["draft"][:, :-1].contiguous(), ValueError, "draft"),
    ("draft", lambda a: a["draft"].float(), TypeError, "draft"),
    ("draft", lambda a: None, ValueError, "draft"),
    ("grad_draft", lambda a: a["grad_draft"][:-1].contiguous(), ValueError, "grad_draft"),
    ("grad_draft", lambda a: a["grad_draft"].float(), TypeError, "grad_draft"),
    ("loss_ce", lambda a: a["loss_ce"][:-1].contiguous(), ValueError, "loss_ce"),
    ("out_tokens", lambda a: a["out_tokens"][:, :-1].contiguous(), ValueError, "out_tokens"),
    ("accept_len", lambda a: a["accept_len"].float(), TypeError, "accept_len"),
    ("row_offsets", lambda a: a["row_offsets"][:-1].contiguous(), ValueError, "row_offsets"),
    ("margins", lambda a: a["margins"].half(), TypeError, "margins"),
    ("status", lambda a: a["status"].long(), TypeError, "status"),
    ("ws", lambda a: a["ws"].float(), TypeError, "workspace"),
])
def test_binding_rejects_mismatched_tensors(lib, name, bad, exc, what):
    """Every tensor's dtype and shape is checked on the host before the
    library sees a pointer (a short buffer would otherwise be overrun on the
    device).  The tensors are CPU tensors: the check must fire before the
    binding asks for device pointers."""
    import diffusion_drafter_verification_amd as ada
    a = _good_verify_args()
    a[name] = bad(a)
    with pytest.raises(exc, match=what):
        ada.adaflash_verify(**a)


@pytest.mark.parametrize("name,bad,exc,what", [
    ("tokens", lambda a: a["tokens"].long(), TypeError, "tokens"),
    ("grad_draft", lambda a: a["grad_draft"][:-1].contiguous(), ValueError, "grad_draft"),
    ("target", lambda a: a["target"], ValueError, "GPU tensors only"),
])
def test_prepared_call_is_checked_like_a_direct_one(lib, name, bad, exc, what):
    import diffusion_drafter_verification_amd as ada
    a = _good_verify_args()
    a[name] = bad(a)
    with pytest.raises(exc, match=what):
        ada.adaflash_verify(**a, prepare=True)


def test_length_head_bindings_check_tensors(lib):
    import torch
    import diffusion_drafter_verification_amd as ada
    B, k, H, Hp = 2, 4, 64, 32
    h = torch.zeros(B, k, H, dtype=torch.bfloat16)
    W1 = torch.zeros(Hp, H, dtype=torch.bfloat16)
    b1, w2 = torch.zeros(Hp), torch.zeros(Hp)
    a_hat, k_hat = torch.zeros(B), torch.zeros(B, dtype=torch.int32)
    with pytest.raises(TypeError, match="hidden"):
        ada.adaflash_length_head_forward(h.float(), W1, b1, w2, 0.0, 1.0, a_hat, k_hat, None)
    with pytest.raises(ValueError, match="W1"):
        ada.adaflash_length_head_forward(h, W1[:, :H - 1].contiguous(), b1, w2, 0.0, 1.0, a_hat, k_hat, None)
    with pytest.raises(ValueError, match="b1"):
        ada.adaflash_length_head_forward(h, W1, b1[:-1].contiguous(), w2, 0.0, 1.0, a_hat, k_hat, None)
    with pytest.raises(ValueError, match="a_hat"):
        ada.adaflash_length_head_forward(h, W1, b1, w2, 0.0, 1.0, a_hat[:1].contiguous(), k_hat, None)
    with pytest.raises(ValueError, match="z1_cache"):
        ada.adaflash_length_head_forward(h, W1, b1, w2, 0.0, 1.0, a_hat, k_hat, None,
                                         z1_cache=torch.zeros(B * k, Hp + 1))
    al = torch.zeros(B, dtype=torch.int32)
    with pytest.raises(ValueError, match="dW1"):
        ada.adaflash_length_head_backward(h, W1, b1, w2, 0.0, al, al, torch.zeros(B), torch.zeros(Hp, H + 1),
                                          b1, w2, torch.zeros(1), None)
    with pytest.raises(TypeError, match="verify_len"):
        ada.adaflash_length_head_backward(h, W1, b1, w2, 0.0, al, al.long(), torch.zeros(B), torch.zeros(Hp, H),
                                          b1, w2, torch.zeros(1), None)
    with pytest.raises(ValueError, match="GPU tensors only"):
        ada.adaflash_length_head_backward(h, W1, b1, w2, 0.0, al, al, torch.zeros(B), torch.zeros(Hp, H),
                                          b1.clone(), w2.clone(), torch.zeros(1), None, prepare=True)


def test_binding_accepts_well_formed_tensors_up_to_the_device_check(lib):
    """With every dtype and shape right, the only complaint about CPU tensors
    is that they are not on the GPU."""
    import diffusion_drafter_verification_amd as ada
    with pytest.raises(ValueError, match="GPU tensors only"):
        ada.adaflash_verify(**_good_verify_args())
    a = _good_verify_args()
    a.update(T=0.0, draft=None, uniforms=None, loss_ce=None, loss_rkl=None, grad_draft=None)
    with pytest.raises(ValueError, match="GPU tensors only"):
        ada.adaflash_verify(**a)


def test_opd_and_variant_bindings_check_tensors(lib):
    import torch
    import diffusion_drafter_verification_amd as ada
    B, k, V = 2, 3, 32
    t = torch.zeros(B, k + 1, V, dtype=torch.bfloat16)
    d = torch.zeros(B, k, V, dtype=torch.bfloat16)
    ro = torch.zeros(B + 1, dtype=torch.int32)
    ce = torch.zeros(B * k)
    g = torch.zeros(B * k, V, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="draft"):
        ada.adaflash_opd_loss_fwd_bwd(t, d[:, :2].contiguous(), None, 10.0, 1.0, ro, ce, ce, g, None, None)
    with pytest.raises(TypeError, match="verify_len"):
        ada.adaflash_opd_loss_fwd_bwd(t, d, torch.ones(B, dtype=torch.int64), 10.0, 1.0, ro, ce, ce, g, None, None)
    with pytest.raises(ValueError, match="grad_draft"):
        ada.adaflash_opd_loss_fwd_bwd(t, d, None, 10.0, 1.0, ro, ce, ce, g[:, :V - 1].contiguous(), None, None)
    with pytest.raises(ValueError, match="loss_ce"):
        ada.adaflash_loss_variant_fwd_bwd(t, d, None, "rkl", 0.0, 0.0, ro, ce[:2].contiguous(), g, None, None)
    # packed forms: the draft must hold target rows - B rows
    tp = torch.zeros(7, V, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="packed draft"):
        ada.adaflash_opd_loss_fwd_bwd_packed(tp, torch.zeros(4, V, dtype=torch.bfloat16),
                                             torch.ones(B, dtype=torch.int32), k, 10.0, 1.0, ro, ce, ce, g, None,
                                             None)
    a = _good_verify_args(B, k, V)
    a["target"] = torch.zeros(B * 2 + 1, V, dtype=torch.bfloat16)
    a["draft"] = torch.zeros(B + 2, V, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="packed draft"):
        ada.adaflash_verify_packed(**a)


def test_noalloc_entry_point_rejects_sizes_beyond_its_array(lib):
    """adaflash_verify_noalloc checks the batch against its fixed device array
    before anything else (no GPU needed for the rejection)."""
    import diffusion_drafter_verification_amd as ada
    f = lib.adaflash_verify_noalloc
    null = [None] * 5
    assert lib.adaflash_workspace_bytes(4096, 16, 151936) > ada.NOALLOC_WORKSPACE_BYTES
    rc = f(1, *null, 4096, 16, 151936, 1.0, None, None, None, 10.0, 1.0, None, None, None, None, None, None)
    assert rc == -4 and b"no-allocation" in lib.adaflash_last_error()
    rc = f(1, *null, 4, 0, 151936, 1.0, None, None, None, 10.0, 1.0, None, None, None, None, None, None)
    assert rc == -1


_REMARKS = """\
x.hip:10:1: remark: Function Name: _Z6good_kv [-Rpass-analysis=kernel-resource-usage]
   10 | __global__ void good_k() {
      | ^
x.hip:10:1: remark:     VGPRs: 61 [-Rpass-analysis=kernel-resource-usage]
x.hip:10:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]
x.hip:10:1: remark:     SGPRs Spill: 22 [-Rpass-analysis=kernel-resource-usage]
x.hip:10:1: remark:     VGPRs Spill: 0 [-Rpass-analysis=kernel-resource-usage]
x.hip:20:1: remark: Function Name: _Z7spill_kv [-Rpass-analysis=kernel-resource-usage]
x.hip:20:1: remark:     ScratchSize [bytes/lane]: 20 [-Rpass-analysis=kernel-resource-usage]
x.hip:20:1: remark:     VGPRs Spill: 5 [-Rpass-analysis=kernel-resource-usage]
x.hip:30:1: remark: Function Name: _Z7stack_kv [-Rpass-analysis=kernel-resource-usage]
x.hip:30:1: remark:     ScratchSize [bytes/lane]: 16 [-Rpass-analysis=kernel-resource-usage]
x.hip:30:1: remark:     VGPRs Spill: 0 [-Rpass-analysis=kernel-resource-usage]
"""


def test_build_rejects_kernels_with_scratch_or_spilled_vgprs():
    """The build's resource check flags a scratch segment and spilled VGPRs,
    and lets SGPR spills (into VGPR lanes) pass."""
    from diffusion_drafter_verification_amd.build import scratch_users
    assert scratch_users(_REMARKS) == [("_Z7spill_kv", "scratch bytes per lane", 20),
                                       ("_Z7spill_kv", "spilled VGPRs", 5),
                                       ("_Z7stack_kv", "scratch bytes per lane", 16)]
    assert scratch_users(_REMARKS.split("x.hip:20:1")[0]) == []
