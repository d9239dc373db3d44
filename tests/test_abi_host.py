"""Host-only checks of the C ABI: the library loads, exports every function
that include/bgb.h declares, and rejects bad arguments before touching the
GPU. Nothing here launches a kernel."""
import ctypes
import os
import re

import pytest

from conftest import ROOT

import bit_gemm_binarize_amd as bgb

HDR = os.path.join(ROOT, "include", "bgb.h")

BAD = -1        # BGB_EINVAL
UNSUP = -2      # BGB_EUNSUPPORTED
A = 1 << 20     # a 16-byte aligned, never dereferenced fake device address


def declared_functions():
    src = open(HDR).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    src = re.sub(r"//[^\n]*", "", src)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b([a-z_][a-z0-9_]*)\s*\([^;{]*\)\s*;", src, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(bgb.lib_path()):
        pytest.fail("libbgb.so is not built (python -m bit_gemm_binarize_amd.build)")
    return bgb.load()


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("binarize_pack", "fbi_linear_w1a16", "bitlinear_w1a8", "bgb_workspace_bytes",
              "bgb_packed_bytes", "bgb_status_string", "bgb_last_hip_error", "bgb_version"):
        assert n in names, names


def test_library_exports_every_declared_symbol(lib):
    raw = ctypes.CDLL(bgb.lib_path())
    for n in declared_functions():
        assert hasattr(raw, n), f"{n} declared in bgb.h but not exported"
    assert set(bgb.EXPORTS) <= set(declared_functions())


def test_sizes(lib):
    assert bgb.packed_bytes(32, 5) == 1 * 5 * 16
    assert bgb.packed_bytes(128, 5) == 1 * 5 * 16
    assert bgb.packed_bytes(160, 3) == 2 * 3 * 16
    assert bgb.packed_bytes(4096, 11008) == 5636096
    assert bgb.packed_bytes(31, 5) == 0
    # GEMM path: the activations are read in place; fp32 partial sums
    # [splits][M][N] only when the launch plan splits K (small M x N)
    assert bgb.workspace_bytes(bgb.OP_FBI_LINEAR, 4096, 4096, 11008) == 0
    assert bgb.workspace_bytes(bgb.OP_FBI_LINEAR, 4096, 4000, 11008) == 0
    small = bgb.workspace_bytes(bgb.OP_FBI_LINEAR, 65, 4096, 4096)
    assert small >= 2 * 65 * 4096 * 4 and small % (65 * 4096 * 4) < 256
    assert bgb.workspace_bytes(bgb.OP_BITLINEAR, 4096, 4096, 11008) == bgb.workspace_bytes(bgb.OP_BITLINEAR, 4096, 4096, 0)
    # decode kernels (M <= 64) stage the activations on chip: no workspace,
    # except fp32 sums [splits][M][N] where the K range is split (long K)
    for M, K in ((1, 4096), (1, 16384), (16, 4096), (4, 11008), (64, 2048)):
        assert bgb.workspace_bytes(bgb.OP_FBI_LINEAR, M, K, 4096) == 0
    for M, K, N in ((1, 20000, 4096), (16, 11008, 4096), (64, 5632, 2048), (20, 16416, 70)):
        w = bgb.workspace_bytes(bgb.OP_FBI_LINEAR, M, K, N)
        assert w >= 2 * M * N * 4 and w - (w // (M * N * 4)) * M * N * 4 < 256
    assert bgb.workspace_bytes(bgb.OP_BITLINEAR, 1, 4096, 11008) >= 4096
    assert bgb.workspace_bytes(99, 1, 32, 32) == 0
    assert lib.bgb_version().decode().startswith("bgb")


def test_status_strings(lib):
    for code in (0, -1, -2, -3, -7):
        assert len(lib.bgb_status_string(code)) > 0


def call_pack(lib, W=A, K=64, N=8, mode=0, P=A, alpha=A, adt=0, beta=A, centre=A, ws=A, wsb=1 << 30):
    return lib.binarize_pack(W, K, N, mode, P, alpha, adt, beta, centre, ws, wsb, None)


def test_pack_validation(lib):
    assert call_pack(lib, K=48) == BAD                 # K % 32 != 0
    assert call_pack(lib, K=0) == BAD
    assert call_pack(lib, N=-1) == BAD
    assert call_pack(lib, W=None) == BAD
    assert call_pack(lib, P=A + 4) == BAD              # misaligned
    assert call_pack(lib, mode=5) == UNSUP
    assert call_pack(lib, adt=2) == UNSUP              # bf16 alpha
    assert call_pack(lib, alpha=None) == BAD
    assert call_pack(lib, mode=1, beta=None) == BAD
    assert call_pack(lib, wsb=8) == BAD                # workspace too small
    assert call_pack(lib, N=0) == 0                    # empty: nothing launched


def call_fbi(lib, x=A, xdt=2, M=4, K=64, N=8, P=A, alpha=A, adt=0, y=A, ydt=0, ws=A, wsb=1 << 30):
    return lib.fbi_linear_w1a16(x, xdt, M, K, N, P, alpha, adt, y, ydt, ws, wsb, None)


def test_fbi_linear_validation(lib):
    assert call_fbi(lib, K=40) == BAD
    assert call_fbi(lib, M=-1) == BAD
    assert call_fbi(lib, xdt=0) == UNSUP               # f32 activations are not W1A16
    assert call_fbi(lib, adt=2) == UNSUP
    assert call_fbi(lib, ydt=7) == UNSUP
    assert call_fbi(lib, x=None) == BAD
    assert call_fbi(lib, y=A + 2) == BAD
    need = bgb.workspace_bytes(bgb.OP_FBI_LINEAR, 65, 4096, 4096)   # a GEMM plan that splits K
    assert call_fbi(lib, M=65, K=4096, N=4096, wsb=need - 1) == BAD
    assert call_fbi(lib, M=65, K=4096, N=4096, ws=None) == BAD
    assert call_fbi(lib, M=1 << 25) == BAD
    assert call_fbi(lib, M=0) == 0 and call_fbi(lib, N=0) == 0


def group(specs):
    """specs: (x, P, alpha, y, K, N) per item, fake addresses."""
    arr = (bgb._Item * max(len(specs), 1))()
    for i, sp in enumerate(specs):
        arr[i] = bgb._Item(*sp)
    return arr


def call_group(lib, specs, M=1, xdt=2, adt=1, ydt=2, ws=A, wsb=1 << 30, count=None):
    n = len(specs) if count is None else count
    return lib.fbi_linear_w1a16_group(group(specs), n, M, xdt, adt, ydt, ws, wsb, None)


MB = 1 << 20


def test_group_validation(lib):
    # four independent linears, each on its own megabyte-aligned fake region
    base = [(A + (4 * i) * 64 * MB, A + (4 * i + 1) * 64 * MB, A + (4 * i + 2) * 64 * MB,
             A + (4 * i + 3) * 64 * MB, 4096, 4096) for i in range(4)]
    assert bgb.group_workspace_bytes([], 1) == 0
    assert lib.bgb_group_workspace_bytes(group(base), 4, 1) == 0          # one launch
    assert call_group(lib, [], count=0) == 0
    assert call_group(lib, base, count=bgb.GROUP_MAX + 1) == BAD
    assert call_group(lib, base, count=-1) == BAD
    assert call_group(lib, base, xdt=0) == UNSUP
    assert call_group(lib, base, adt=2) == UNSUP
    assert call_group(lib, base, M=-1) == BAD
    bad = list(base)
    bad[2] = (0,) + bad[2][1:]                                             # null x
    assert call_group(lib, bad) == BAD
    bad = list(base)
    bad[1] = bad[1][:4] + (40, 4096)                                       # K % 32 != 0
    assert call_group(lib, bad) == BAD
    bad = list(base)
    bad[3] = bad[3][:3] + (bad[0][1] + 256,) + bad[3][4:]                  # y inside another item's P
    assert call_group(lib, bad) == BAD
    bad = list(base)
    bad[3] = bad[3][:3] + (bad[0][3] + 4096,) + bad[3][4:]                 # two outputs overlap
    assert call_group(lib, bad) == BAD
    bad = list(base)
    bad[0] = bad[0][:3] + (bad[0][0] + 16,) + bad[0][4:]                   # y over its own x
    assert call_group(lib, bad) == BAD
    empty = list(base)
    empty[1] = (0, 0, 0, 0, 4096, 0)                                        # N = 0: skipped, unchecked
    assert call_group(lib, empty, M=0) == 0
    # several tokens: the items run one after another on the largest item's workspace
    split = [b[:4] + (11008, 4096) for b in base]
    need = lib.bgb_group_workspace_bytes(group(split), 4, 16)
    assert need == max(bgb.workspace_bytes(bgb.OP_FBI_LINEAR, 16, 11008, 4096), 0)
    if need:
        assert call_group(lib, split, M=16, wsb=need - 1) == BAD
        assert call_group(lib, split, M=16, ws=None) == BAD


def call_bwd(lib, dy=A, x=A, dt=2, M=4, K=64, N=64, P=A, PT=A, alpha=A, adt=0, dx=A, dxdt=0, da=A, dw=A, ws=A,
             wsb=1 << 30):
    return lib.fbi_linear_w1a16_backward(dy, x, dt, M, K, N, P, PT, alpha, adt, dx, dxdt, da, dw, ws, wsb, None)


def test_backward_validation(lib):
    assert lib.fbi_pack_transposed(A, 64, 48, A + 64 * MB, None) == BAD          # N % 32 != 0
    assert lib.fbi_pack_transposed(A, 40, 64, A + 64 * MB, None) == BAD          # K % 32 != 0
    assert lib.fbi_pack_transposed(None, 64, 64, A + 64 * MB, None) == BAD
    assert lib.fbi_pack_transposed(A, 64, 64, A + 256, None) == BAD              # PT over P
    assert lib.fbi_pack_transposed(A, 64, 0, A + 64 * MB, None) == 0             # empty
    need = bgb.workspace_bytes(bgb.OP_FBI_BACKWARD, 4, 64, 64)
    assert need >= 4 * 2 * 64 * 2 + 4 * 64 * 4                                     # split gradient + z
    assert call_bwd(lib, N=48) == BAD
    assert call_bwd(lib, K=40) == BAD
    assert call_bwd(lib, dt=0) == UNSUP                                            # f32 gradients not offered
    assert call_bwd(lib, adt=2) == UNSUP
    assert call_bwd(lib, dxdt=7) == UNSUP
    assert call_bwd(lib, dy=None) == BAD
    assert call_bwd(lib, PT=None) == BAD                                           # dx needs the transposed signs
    assert call_bwd(lib, x=None) == BAD                                            # dalpha / dw need x
    assert call_bwd(lib, P=None) == BAD                                            # dalpha needs P
    assert call_bwd(lib, dx=A + 4) == BAD
    assert call_bwd(lib, wsb=need - 1) == BAD
    assert call_bwd(lib, ws=None) == BAD
    assert call_bwd(lib, M=0) == 0 and call_bwd(lib, N=0) == 0
    # dX multiplies by [S^T; S^T], a 2N x K operand: K N < 2^31 but 2 N K > 2^31 - 1
    assert 65536 * 16416 < 2 ** 31 - 1 < 2 * 65536 * 16416
    assert call_bwd(lib, M=1, K=65536, N=16416) == BAD
    assert call_bwd(lib, M=0, K=65536, N=16416) == BAD                            # shapes are checked when empty too
    assert call_bwd(lib, M=0, K=65536, N=16416, dx=None) == 0                     # no dX: that operand is not formed


def call_bl(lib, x=A, xdt=0, M=1, K=64, N=8, P=A, beta=A, qp=None, y=A, xq=None, g=None, acc=None, ws=A,
            wsb=1 << 30):
    return lib.bitlinear_w1a8(x, xdt, M, K, N, P, beta, qp, y, xq, g, acc, ws, wsb, None)


def test_bitlinear_validation(lib):
    assert call_bl(lib, K=33) == BAD
    assert call_bl(lib, xdt=1) == UNSUP                # f16 activations not offered here
    assert call_bl(lib, beta=None) == BAD
    assert call_bl(lib, ws=None) == BAD
    assert call_bl(lib, wsb=16) == BAD
    assert call_bl(lib, xq=A + 1) == BAD
    bad_bits = bgb._QP(1e-5, 9, 1e-3)
    assert call_bl(lib, qp=ctypes.pointer(bad_bits)) == UNSUP
    bad_eps = bgb._QP(1e-5, 8, 2.0)
    assert call_bl(lib, qp=ctypes.pointer(bad_eps)) == BAD
    assert call_bl(lib, qp=ctypes.pointer(bgb._QP(1e-5, 8, 1e-3, 2, 0))) == UNSUP   # round mode
    assert call_bl(lib, qp=ctypes.pointer(bgb._QP(1e-5, 8, 1e-3, 0, 5))) == UNSUP   # gamma scope
    assert call_bl(lib, qp=ctypes.pointer(bgb._QP(1e-5, 8, 1e-3, 0, 0, 2))) == UNSUP   # activation range
    # the non-negative range keeps its row and block minima in the workspace
    assert bgb.workspace_bytes(bgb.OP_BITLINEAR, 100, 4096, 0) >= 100 * 4096 + (100 + 25) * 4
    assert call_bl(lib, M=0) == 0


def test_header_compiles_as_c_and_cpp(tmp_path):
    """The boundary is a C ABI: the header must compile on its own as C and C++."""
    import shutil
    import subprocess
    src = tmp_path / "use.c"
    src.write_text('#include "bgb.h"\nint main(void) { return (int)sizeof(bgb_w1a16_item) + BGB_GROUP_MAX; }\n')
    for exe, lang, std in (("gcc", "c", "-std=c11"), ("g++", "c++", "-std=c++17")):
        if shutil.which(exe) is None:
            pytest.skip(f"{exe} not available")
        r = subprocess.run([exe, "-x", lang, std, "-Wall", "-Wextra", "-Werror", "-fsyntax-only",
                            "-I", os.path.join(ROOT, "include"), str(src)], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr


def test_ceilings_library_exports_and_rejects():
    """libbgb_ceilings.so (measurement kernels) exports what bgb_ceilings.h
    declares; bad arguments return -1 before any launch."""
    path = os.path.join(ROOT, "bit_gemm_binarize_amd", "ceilings", "libbgb_ceilings.so")
    if not os.path.exists(path):
        pytest.fail("libbgb_ceilings.so is not built (python -m bit_gemm_binarize_amd.build)")
    src = open(os.path.join(ROOT, "include", "bgb_ceilings.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = set(re.findall(r"^\s*int\s+([a-z_][a-z0-9_]*)\s*\(", src, flags=re.M))
    assert {"ceil_stream_read", "ceil_empty", "ceil_mfma_bf16", "ceil_mfma_i8", "ceil_last_hip_error"} <= names
    lib = ctypes.CDLL(path)
    for n in names:
        assert hasattr(lib, n), n
    V, SZ, I = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    lib.ceil_stream_read.argtypes = [V, SZ, I, V, V]
    lib.ceil_empty.argtypes = [I, I, V]
    lib.ceil_mfma_bf16.argtypes = [V, I, I, V, V]
    assert lib.ceil_stream_read(None, 1024, 8, A, None) == -1
    assert lib.ceil_stream_read(A + 4, 1024, 8, A, None) == -1          # misaligned
    assert lib.ceil_stream_read(A, 1000, 8, A, None) == -1              # not a multiple of 16
    assert lib.ceil_empty(0, 64, None) == -1
    assert lib.ceil_empty(8, 2048, None) == -1
    assert lib.ceil_mfma_bf16(None, 8, 10, A, None) == -1
    assert lib.ceil_mfma_bf16(A, 8, 0, A, None) == -1


def test_noalloc_rejects_oversize_before_touching_the_gpu(lib):
    """bitlinear_w1a8_noalloc checks its workspace need against the static
    scratch first: a call that does not fit returns BGB_ESCRATCH (-4) with no
    device call (so it runs without a GPU)."""
    assert lib.bgb_noalloc_scratch_bytes() == 64 << 20
    lib.bitlinear_w1a8_noalloc.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
                                           ctypes.c_int64] + [ctypes.c_void_p] * 8
    M, K, N = 8192, 8192, 64
    assert bgb.workspace_bytes(bgb.OP_BITLINEAR, M, K, N) > 64 << 20
    assert lib.bitlinear_w1a8_noalloc(A, 0, M, K, N, A, A, None, A, None, None, None, None) == -4
    assert b"scratch" in lib.bgb_status_string(-4)
    # an empty call is validated and launches nothing
    assert lib.bitlinear_w1a8_noalloc(None, 0, 0, 64, 8, None, None, None, None, None, None, None, None) == 0
    assert lib.bitlinear_w1a8_noalloc(None, 0, 0, 40, 8, None, None, None, None, None, None, None, None) == BAD
