"""The C ABI without a GPU: libssd.so loads, exports every function that
include/ssd.h declares, and refuses bad arguments on the host (before any HIP
call) with the documented status and a message naming the argument."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssd.h")


@pytest.fixture(scope="module")
def lib():
    import selective_state_space_14_amd as ssd
    if not os.path.exists(ssd.LIB_PATH):
        from selective_state_space_14_amd import build
        build.build(verbose=False)
    return ssd.load()


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(ssd_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_the_three_operations():
    names = declared_functions()
    for n in ("ssd_conv_fwd", "ssd_chunk_scan_fwd", "ssd_step", "ssd_chunk_scan_workspace_size", "ssd_mixer_fwd",
              "ssd_mixer_workspace_size", "ssd_resume_fwd", "ssd_s6_scan_fwd", "ssd_s6_workspace_size",
              "ssd_last_error", "ssd_status_string", "ssd_version"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), f"libssd.so does not export {name}"


def test_version_and_status_strings(lib):
    assert lib.ssd_version() == 2
    assert lib.ssd_status_string(0) == b"SSD_OK"
    assert lib.ssd_status_string(2) == b"SSD_ERR_BAD_SHAPE"
    assert lib.ssd_status_string(99) == b"SSD_ERR_UNKNOWN"


FAKE = 0x10000          # 16-byte aligned, never dereferenced: every call below fails validation
MIS = 0x10008           # 8-byte aligned only


def scan_args(**over):
    a = dict(B=2, L=128, H=32, P=64, N=64, G=8, chunk=64, dtype=1,
             x=FAKE, xs=3072, Bm=FAKE, bs=3072, Cm=FAKE, cs=3072, dt=FAKE, dts=32, dt_softplus=0, dt_bias=None,
             A=FAKE, D=None, z=None, zs=0, doc=None, len=None, h0=None, hf=None, y=FAKE, ys=2048, ws=None, wsb=0,
             stream=None)
    a.update(over)
    return a


def call_scan(lib, a):
    return lib.ssd_chunk_scan_fwd(a["B"], a["L"], a["H"], a["P"], a["N"], a["G"], a["chunk"], a["dtype"],
                                  a["x"], a["xs"], a["Bm"], a["bs"], a["Cm"], a["cs"], a["dt"], a["dts"],
                                  a["dt_softplus"], a["dt_bias"], a["A"], a["D"], a["z"], a["zs"], a["doc"],
                                  a["len"], a["h0"], a["hf"], a["y"], a["ys"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("over,status,needle", [
    (dict(H=30, G=8), 2, "H=30 is not divisible by G=8"),
    (dict(len=FAKE, h0=FAKE), 2, "lengths cannot be combined"),
    (dict(len=FAKE, hf=FAKE), 2, "lengths cannot be combined"),
    (dict(P=32), 3, "P=32"),
    (dict(N=48), 3, "N=48"),
    (dict(chunk=128), 3, "chunk=128"),
    (dict(dtype=2), 3, "dtype=2"),
    (dict(B=-1), 2, "B=-1"),
    (dict(L=-5), 2, "L=-5"),
    (dict(L=(1 << 30) + 1), 2, "L=1073741825 is above"),
    (dict(L=266240, H=128, G=8), 2, "reach 2^31 bytes per batch row"),
    (dict(x=None), 1, "x is NULL"),
    (dict(dt=None), 1, "dt is NULL"),
    (dict(A=None), 1, "A is NULL"),
    (dict(xs=1000), 2, "x row stride 1000"),
    (dict(dts=8), 2, "dt row stride 8"),
    (dict(x=MIS), 4, "x="),
    (dict(xs=3076), 4, "x row stride 3076"),
    (dict(h0=MIS), 4, "init_state"),
    (dict(dt_softplus=2), 3, "dt_softplus=2"),
    (dict(y=FAKE, hf=FAKE), 2, "y must not alias final_state"),
])
def test_scan_refusals(lib, over, status, needle):
    st = call_scan(lib, scan_args(**over))
    assert st == status, (st, lib.ssd_last_error())
    assert needle in lib.ssd_last_error().decode()


def call_conv(lib, **over):
    a = dict(B=2, L=100, H=32, P=64, N=64, G=8, K=4, dtype=1, raw=FAKE, rs=3072, w=FAKE, b=None, dtr=None, dtrs=0,
             dtb=None, doc=None, si=None, so=None, act=0, out=FAKE + 0x1000, os_=3072, dto=None, stream=None)
    a.update(over)
    return lib.ssd_conv_fwd(a["B"], a["L"], a["H"], a["P"], a["N"], a["G"], a["K"], a["dtype"], a["raw"], a["rs"],
                            a["w"], a["b"], a["dtr"], a["dtrs"], a["dtb"], a["doc"], a["si"], a["so"], a["act"],
                            a["out"], a["os_"], a["dto"], a["stream"])


@pytest.mark.parametrize("over,status,needle", [
    (dict(K=3), 3, "K=3"),
    (dict(L=(1 << 30) + 1), 2, "L=1073741825 is above"),
    (dict(act=7), 3, "act=7"),
    (dict(dtype=5), 3, "dtype=5"),
    (dict(w=None), 1, "conv_w is NULL"),
    (dict(raw=None), 1, "xbc_raw is NULL"),
    (dict(out=FAKE), 2, "must not alias"),
    (dict(rs=100), 2, "xbc_raw row stride 100"),
    (dict(dto=FAKE), 1, "dt_out is given but dt_raw is NULL"),
    (dict(dtr=FAKE, dtrs=4), 2, "dt_raw row stride 4"),
    (dict(si=MIS), 4, "conv_state_in"),
])
def test_conv_refusals(lib, over, status, needle):
    st = call_conv(lib, **over)
    assert st == status, (st, lib.ssd_last_error())
    assert needle in lib.ssd_last_error().decode()


def call_mixer(lib, **over):
    a = dict(B=2, L=100, H=32, P=64, N=64, G=8, K=4, chunk=64, dtype=1, raw=FAKE, rs=3072, w=FAKE, b=None,
             dtr=FAKE, dtrs=32, dtb=None, A=FAKE, D=None, z=None, zs=0, doc=None, len=None, si=None, so=None, h0=None,
             hf=None, act=0, y=FAKE + 0x100000, ys=2048, ws=None, wsb=0, stream=None)
    a.update(over)
    return lib.ssd_mixer_fwd(a["B"], a["L"], a["H"], a["P"], a["N"], a["G"], a["K"], a["chunk"], a["dtype"],
                             a["raw"], a["rs"], a["w"], a["b"], a["dtr"], a["dtrs"], a["dtb"], a["A"], a["D"],
                             a["z"], a["zs"], a["doc"], a["len"], a["si"], a["so"], a["h0"], a["hf"], a["act"], a["y"],
                             a["ys"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("over,status,needle", [
    (dict(K=2), 3, "K=2"),
    (dict(len=FAKE, so=FAKE), 2, "lengths cannot be combined with carried states"),
    (dict(chunk=32), 3, "chunk=32"),
    (dict(act=3), 3, "act=3"),
    (dict(raw=None), 1, "xbc_raw is NULL"),
    (dict(dtr=None), 1, "dt_raw is NULL"),
    (dict(w=None), 1, "conv_w is NULL"),
    (dict(A=None), 1, "A is NULL"),
    (dict(rs=1000), 2, "xbc_raw row stride 1000"),
    (dict(dtrs=31, H=32), 2, "dt_raw row stride 31"),
    (dict(dtrs=33), 4, "must be even"),
    (dict(si=FAKE, so=FAKE), 2, "must not overlap"),
    (dict(si=FAKE, so=FAKE + 0x100), 2, "must not overlap"),
    (dict(y=FAKE, hf=FAKE), 2, "y must not alias final_state"),
    (dict(dtype=0, dtrs=32), 5, "fp32 needs a workspace"),
    (dict(dtype=0, dtrs=32, ws=FAKE, wsb=4096), 5, "fp32 needs a workspace"),
    (dict(ws=MIS, wsb=4096), 4, "workspace="),
    (dict(ys=1024), 2, "y row stride 1024"),
])
def test_mixer_refusals(lib, over, status, needle):
    st = call_mixer(lib, **over)
    assert st == status, (st, lib.ssd_last_error())
    assert needle in lib.ssd_last_error().decode()


def test_mixer_workspace_size(lib):
    # the staged plan: conv output (element size of the dtype) and fp32 dt, each padded to 256 bytes, then the
    # scan's split state
    B, L, H, P, N, G = 5, 8192, 32, 64, 64, 8
    C = H * P + 2 * G * N
    r = lambda n: (n + 255) // 256 * 256
    for dtype, es in ((0, 4), (1, 2)):
        assert (lib.ssd_mixer_workspace_size(B, L, H, P, N, G, dtype) ==
                r(B * L * C * es) + r(B * L * H * 4) + lib.ssd_chunk_scan_workspace_size(B, L, H, P, N, G, dtype))
    assert lib.ssd_mixer_workspace_size(0, L, H, P, N, G, 1) == 0


def call_step(lib, **over):
    a = dict(B=4, H=64, P=64, N=128, G=1, K=4, dtype=0, raw=FAKE, dtr=FAKE, z=None, w=FAKE, b=None, dtb=None,
             A=FAKE, D=None, cst=FAKE, sst=FAKE, act=0, y=FAKE, stream=None)
    a.update(over)
    return lib.ssd_step(a["B"], a["H"], a["P"], a["N"], a["G"], a["K"], a["dtype"], a["raw"], a["dtr"], a["z"],
                        a["w"], a["b"], a["dtb"], a["A"], a["D"], a["cst"], a["sst"], a["act"], a["y"], a["stream"])


@pytest.mark.parametrize("over,status,needle", [
    (dict(G=3), 2, "H=64 is not divisible by G=3"),
    (dict(N=256), 3, "N=256"),
    (dict(sst=None), 1, "ssm_state is NULL"),
    (dict(cst=MIS), 4, "conv_state"),
    (dict(z=FAKE + 4), 4, "z="),
    (dict(z=MIS), 4, "z="),
    (dict(H=256, G=1), 3, "64 KiB LDS"),
])
def test_step_refusals(lib, over, status, needle):
    st = call_step(lib, **over)
    assert st == status, (st, lib.ssd_last_error())
    assert needle in lib.ssd_last_error().decode()


def call_resume(lib, **over):
    a = dict(B=4, H=64, P=64, N=128, G=1, K=4, dtype=0, pos=0, n=1, raw=FAKE, dtr=FAKE, z=None, w=FAKE, b=None,
             dtb=None, A=FAKE, D=None, act=0, cst=FAKE, cx=FAKE, cdt=FAKE, cz=None, cs=FAKE, cy=FAKE, y=FAKE,
             stream=None)
    a.update(over)
    return lib.ssd_resume_fwd(a["B"], a["H"], a["P"], a["N"], a["G"], a["K"], a["dtype"], a["pos"], a["n"],
                              a["raw"], a["dtr"], a["z"], a["w"], a["b"], a["dtb"], a["A"], a["D"], a["act"],
                              a["cst"], a["cx"], a["cdt"], a["cz"], a["cs"], a["cy"], a["y"], a["stream"])


@pytest.mark.parametrize("over,status,needle", [
    (dict(pos=64), 2, "pos=64"),
    (dict(pos=60, n=5), 2, "pos + n = 65"),
    (dict(act=2), 3, "act=2"),
    (dict(z=FAKE), 1, "z and chunk_z"),
    (dict(cs=None), 1, "chunk_state is NULL"),
    (dict(H=65536, G=1), 2, "conv_dim=4194560"),
])
def test_resume_refusals(lib, over, status, needle):
    st = call_resume(lib, **over)
    assert st == status, (st, lib.ssd_last_error())
    assert needle in lib.ssd_last_error().decode()


def test_static_scan_refuses_workspace_beyond_static_scratch(lib):
    """ssd_chunk_scan_fwd_static: sizes whose split workspace exceeds SSD_STATIC_SCRATCH_BYTES are refused on
    the host, before any HIP call (the pointers here are never dereferenced)."""
    import selective_state_space_14_amd as ssd
    src = open(HEADER).read()
    assert "#define SSD_STATIC_SCRATCH_BYTES ((size_t)32 << 20)" in src
    assert ssd.SSD_STATIC_SCRATCH_BYTES == 32 << 20
    a = scan_args(B=5, L=8192, H=64, N=128, G=8, xs=4096, bs=1024, cs=1024, dts=64, ys=4096)
    need = lib.ssd_chunk_scan_workspace_size(5, 8192, 64, 64, 128, 8, 1)
    assert need > ssd.SSD_STATIC_SCRATCH_BYTES
    st = lib.ssd_chunk_scan_fwd_static(a["B"], a["L"], a["H"], a["P"], a["N"], a["G"], a["chunk"], a["dtype"],
                                       a["x"], a["xs"], a["Bm"], a["bs"], a["Cm"], a["cs"], a["dt"], a["dts"],
                                       a["dt_softplus"], a["dt_bias"], a["A"], a["D"], a["z"], a["zs"], a["doc"],
                                       a["len"], a["h0"], a["hf"], a["y"], a["ys"], a["stream"])
    assert st == 5, (st, lib.ssd_last_error())
    assert b"static scratch" in lib.ssd_last_error()
    # the same validation as ssd_chunk_scan_fwd runs first
    st = lib.ssd_chunk_scan_fwd_static(a["B"], a["L"], 30, a["P"], a["N"], a["G"], a["chunk"], a["dtype"],
                                       a["x"], a["xs"], a["Bm"], a["bs"], a["Cm"], a["cs"], a["dt"], a["dts"],
                                       a["dt_softplus"], a["dt_bias"], a["A"], a["D"], a["z"], a["zs"], a["doc"],
                                       a["len"], a["h0"], a["hf"], a["y"], a["ys"], a["stream"])
    assert st == 2 and b"H=30" in lib.ssd_last_error()


def test_error_message_cleared_on_success_path_is_thread_local(lib):
    call_scan(lib, scan_args(P=32))
    assert b"P=32" in lib.ssd_last_error()
    import threading
    seen = []
    th = threading.Thread(target=lambda: seen.append(lib.ssd_last_error()))
    th.start()
    th.join()
    assert seen == [b""]


def test_python_binding_refuses_other_dtypes_by_name():
    import torch
    import selective_state_space_14_amd as ssd
    x = torch.zeros(1, 4, 64, dtype=torch.float16)
    with pytest.raises(TypeError, match="float16"):
        ssd.ssd_chunk_scan_fwd(x, x, x, x, x, H=1, P=64, N=16, G=1)


def test_python_binding_refuses_host_tensors():
    import torch
    import selective_state_space_14_amd as ssd
    x = torch.zeros(1, 4, 64, dtype=torch.float32)
    bm = torch.zeros(1, 4, 16)
    with pytest.raises(ValueError, match="GPU tensor"):
        ssd.ssd_chunk_scan_fwd(x, bm, bm, torch.zeros(1, 4, 1), torch.zeros(1), H=1, P=64, N=16, G=1,
                               y=torch.zeros(1, 4, 64))


def s6_args(**over):
    a = dict(B=2, L=128, D=512, N=16, dtype=1, x=FAKE, xs=512, dt=FAKE, dts=512, sp=1, db=None, A=FAKE,
             Bm=FAKE, bs=16, Cm=FAKE, cs=16, Dk=None, z=None, zs=0, doc=None, h0=None, hf=None, y=FAKE, ys=512,
             ws=None, wsb=0, stream=None)
    a.update(over)
    return a


def call_s6(lib, a):
    f = lib.ssd_s6_scan_fwd
    I, P, I64, SZ = ctypes.c_int, ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
    f.restype = I
    f.argtypes = [I, I, I, I, I, P, I64, P, I64, I, P, P, P, I64, P, I64, P, P, I64, P, P, P, P, I64, P, SZ, P]
    return f(a["B"], a["L"], a["D"], a["N"], a["dtype"], a["x"], a["xs"], a["dt"], a["dts"], a["sp"], a["db"],
             a["A"], a["Bm"], a["bs"], a["Cm"], a["cs"], a["Dk"], a["z"], a["zs"], a["doc"], a["h0"], a["hf"],
             a["y"], a["ys"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("over,status,needle", [
    (dict(N=64), 3, "N=64 is not supported"),
    (dict(N=4), 3, "N=4"),
    (dict(dtype=3), 3, "dtype=3"),
    (dict(D=0), 2, "D=0"),
    (dict(B=-2), 2, "B=-2"),
    (dict(L=-1), 2, "L=-1"),
    (dict(x=None), 1, "x is NULL"),
    (dict(dt=None), 1, "dt is NULL"),
    (dict(A=None), 1, "A is NULL"),
    (dict(Bm=None), 1, "Bm is NULL"),
    (dict(y=None), 1, "y is NULL"),
    (dict(xs=500), 2, "x row stride 500"),
    (dict(bs=12), 2, "Bm row stride 12"),
    (dict(Cm=MIS), 4, "Cm=.*not 16-byte aligned"),
    (dict(cs=20), 4, "Cm row stride 20 elements"),
    (dict(z=FAKE, zs=100), 2, "z row stride 100"),
    (dict(h0=MIS), 4, "init_state"),
    (dict(sp=2), 3, "dt_softplus=2"),
    (dict(hf=FAKE), 2, "y must not alias final_state"),
    (dict(L=8192, ws=FAKE, wsb=64), 5, "workspace_bytes=64"),
    (dict(L=8192, ws=MIS, wsb=1 << 40), 4, "workspace=.*not 16-byte aligned"),
])
def test_s6_refusals(lib, over, status, needle):
    st = call_s6(lib, s6_args(**over))
    assert st == status, (st, lib.ssd_last_error())
    assert re.search(needle, lib.ssd_last_error().decode()), lib.ssd_last_error()


def test_s6_workspace_size(lib):
    f = lib.ssd_s6_workspace_size
    f.restype = ctypes.c_size_t
    f.argtypes = [ctypes.c_int] * 5
    assert f(0, 8192, 2048, 16, 1) == 0
    assert f(5, 0, 2048, 16, 1) == 0
    # a short sequence is not split (one superchunk per 64 tokens at most)
    assert f(5, 64, 2048, 16, 1) == 0
    n = f(5, 8192, 2048, 16, 1)
    assert n > 0 and n % 4 == 0
    # hloc + sdt grow with N only through hloc; the initial-state copy is B*D*N floats
    assert f(5, 8192, 2048, 32, 1) > n


def bwd_args(**over):
    a = dict(B=2, L=128, H=8, P=64, N=64, G=2, chunk=64, dtype=1, x=FAKE, xs=512, Bm=FAKE, bs=128, Cm=FAKE, cs=128,
             dt=FAKE, dts=8, sp=1, db=None, A=FAKE, D=None, z=None, zs=0, doc=None, gy=FAKE, gys=512, dx=FAKE,
             dxs=512, dB=FAKE, dBs=128, dC=FAKE, dCs=128, ddt=FAKE, ddts=8, ddb=None, dA=FAKE, dD=None, dz=None, dzs=0,
             ws=FAKE, wsb=1 << 40, stream=None)
    a.update(over)
    return a


def call_bwd(lib, a):
    f = lib.ssd_chunk_scan_bwd
    I, P, I64, SZ = ctypes.c_int, ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
    f.restype = I
    f.argtypes = [I, I, I, I, I, I, I, I, P, I64, P, I64, P, I64, P, I64, I, P, P, P, P, I64, P, P, I64, P, I64, P,
                  I64, P, I64, P, I64, P, P, P, P, I64, P, SZ, P]
    return f(a["B"], a["L"], a["H"], a["P"], a["N"], a["G"], a["chunk"], a["dtype"], a["x"], a["xs"], a["Bm"], a["bs"],
             a["Cm"], a["cs"], a["dt"], a["dts"], a["sp"], a["db"], a["A"], a["D"], a["z"], a["zs"], a["doc"], a["gy"],
             a["gys"], a["dx"], a["dxs"], a["dB"], a["dBs"], a["dC"], a["dCs"], a["ddt"], a["ddts"], a["ddb"], a["dA"],
             a["dD"], a["dz"], a["dzs"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("over,status,needle", [
    (dict(N=256), 3, "N=256"),
    (dict(chunk=32), 3, "chunk=32"),
    (dict(dtype=5), 3, "dtype=5"),
    (dict(gy=None), 1, "grad_y is NULL"),
    (dict(dx=None), 1, "dx is NULL"),
    (dict(ddt=None), 1, "ddt is NULL"),
    (dict(dA=None), 1, "dA is NULL"),
    (dict(dxs=514), 4, "dx row stride 514"),
    (dict(dBs=100), 2, "dB row stride 100"),
    (dict(dz=FAKE, dzs=512), 1, "dz is given but z is NULL"),
    (dict(ws=None, wsb=0), 5, "workspace_bytes=0"),
    (dict(ws=MIS), 4, "workspace=.*not 16-byte aligned"),
    (dict(sp=3), 3, "dt_softplus=3"),
])
def test_scan_bwd_refusals(lib, over, status, needle):
    st = call_bwd(lib, bwd_args(**over))
    assert st == status, (st, lib.ssd_last_error())
    assert re.search(needle, lib.ssd_last_error().decode()), lib.ssd_last_error()


def test_bwd_workspace_sizes(lib):
    I, SZ = ctypes.c_int, ctypes.c_size_t
    for nm in ("ssd_chunk_scan_bwd_workspace_size", "ssd_conv_bwd_workspace_size", "ssd_mixer_bwd_workspace_size"):
        getattr(lib, nm).restype = SZ
        getattr(lib, nm).argtypes = [I] * 7
    s = lib.ssd_chunk_scan_bwd_workspace_size(5, 8192, 32, 64, 64, 8, 1)
    # two [B][H][L/64][N][P] fp32 state arrays dominate
    assert s >= 2 * 5 * 32 * 128 * 64 * 64 * 4
    c = lib.ssd_conv_bwd_workspace_size(5, 8192, 32, 64, 64, 8, 1)
    assert c == 5 * 128 * 3072 * 5 * 4
    m = lib.ssd_mixer_bwd_workspace_size(5, 8192, 32, 64, 64, 8, 1)
    assert m >= s + c + 5 * 8192 * 3072 * (2 + 4)
    assert lib.ssd_chunk_scan_bwd_workspace_size(0, 8192, 32, 64, 64, 8, 1) == 0
