"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments on the host before any launch."""
import ctypes
import os
import re

import pytest

import rotated_runtime_activation_amd as rra

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.skipif(not os.path.exists(rra.LIB_PATH),
                                reason="librrs.so not built (run __graft_entry__.build())")


def header_functions():
    src = open(os.path.join(ROOT, "include", "rrs.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(rrs_[a-z_0-9]+)\s*\(", src)))


def test_header_and_binding_agree():
    assert sorted(rra.EXPORTS) == header_functions()


def test_library_exports_every_header_symbol():
    lib = ctypes.CDLL(rra.LIB_PATH)
    for name in header_functions():
        assert hasattr(lib, name), name


def test_status_strings_and_version():
    assert rra.rrs_status_string(0) == "RRS_OK"
    assert "EINVAL" in rra.rrs_status_string(-1)
    assert "EUNSUPPORTED" in rra.rrs_status_string(-2)
    assert "EHIP" in rra.rrs_status_string(-3)
    assert "ETOOBIG" in rra.rrs_status_string(rra.RRS_ETOOBIG)
    assert "unknown" in rra.rrs_status_string(42)
    assert rra.rrs_version().startswith("rrs-gfx950")


def test_size_queries():
    # weights: N*K/2 codes + 4N scales, each section 256-byte aligned
    assert rra.rrs_weight_bytes(4096, 4096) == 4096 * 2048 + 4096 * 4
    assert rra.rrs_weight_bytes(256, 3) == 512 + 256
    assert rra.rrs_weight_bytes(100, 4) == 0      # K not a power of two
    assert rra.rrs_weight_bytes(32, 4) == 0       # K < 64
    assert rra.rrs_weight_bytes(16384, 4) == 0    # K > 8192
    assert rra.rrs_weight_bytes(256, 0) == 0
    # workspace: sync block + xq + dx + S
    sync = rra.rrs_sync_bytes(4096, 128)
    # 17408 words (control words and a reserved area) + a row of
    # K/G 64-bit tagged maxima for each of 512 workgroups
    assert sync == 4 * (17408 + 2 * 512 * 32) and rra.rrs_sync_bytes(8192, 32) == 4 * (17408 + 2 * 512 * 256)
    assert rra.rrs_sync_bytes(64, 32) == 4 * (17408 + 2 * 512 * 2)
    assert rra.rrs_workspace_bytes(2048, 4096, 128) == sync + 2048 * 2048 + 2048 * 4 + 256
    assert rra.rrs_workspace_bytes(1, 64, 32) == 4 * (17408 + 2048) + 256 + 256 + 256
    assert rra.rrs_workspace_bytes(16, 256, 16) == 0   # G < 32
    assert rra.rrs_workspace_bytes(16, 256, 512) == 0  # G > K
    assert rra.rrs_workspace_bytes(16, 256, 96) == 0   # G not a power of two
    assert rra.rrs_workspace_bytes(-1, 256, 128) == 0
    assert rra.rrs_calibrate_workspace_bytes(8192) == 32768


# Invalid calls return RRS_EINVAL from the host-side checks; nothing is
# launched, so they run without a GPU. Pointers are dummies that would fault
# if ever dereferenced.
DUMMY = ctypes.c_void_p(0x1000)
NULL = None


def _lin(**kw):
    a = dict(X=DUMMY, M=16, K=256, N=256, G=128, perm=DUMMY, wq=DUMMY, Y=DUMMY, ws=DUMMY,
             ws_bytes=1 << 20, s=NULL)
    a.update(kw)
    return rra.lib().rrs_linear(a["X"], a["M"], a["K"], a["N"], a["G"], a["perm"], a["wq"],
                                a["Y"], a["ws"], a["ws_bytes"], a["s"])


@pytest.mark.parametrize("kw", [
    dict(K=100), dict(K=32), dict(K=16384), dict(G=16), dict(G=96), dict(G=512),
    dict(M=-1), dict(N=0), dict(X=NULL), dict(perm=NULL), dict(wq=NULL), dict(Y=NULL),
    dict(ws=NULL), dict(ws_bytes=100),
])
def test_linear_rejects(kw):
    assert _lin(**kw) == rra.RRS_EINVAL


def test_linear_zero_tokens_is_noop():
    assert _lin(M=0, X=NULL, Y=NULL) == rra.RRS_OK


def test_frontend_rejects():
    L = rra.lib()
    ok = dict(X=DUMMY, M=4, K=256, G=64, perm=DUMMY, xq=DUMMY, dx=DUMMY, S=DUMMY, ws=DUMMY,
              ws_bytes=1 << 20, flags=0)

    def call(**kw):
        a = {**ok, **kw}
        return L.rrs_frontend(a["X"], a["M"], a["K"], a["G"], a["perm"], a["xq"], a["dx"], a["S"],
                              a["ws"], a["ws_bytes"], a["flags"], NULL)
    assert call(flags=16) == rra.RRS_EINVAL
    assert call(flags=32 | rra.RRS_FLAG_NO_ROTATE) == rra.RRS_EINVAL
    assert call(ws_bytes=255) == rra.RRS_EINVAL
    assert call(S=NULL) == rra.RRS_EINVAL
    assert call(xq=NULL) == rra.RRS_EINVAL
    assert call(G=512) == rra.RRS_EINVAL
    assert call(M=0, X=NULL, xq=NULL, dx=NULL) == rra.RRS_OK


def test_frontend_passes_rejects():
    L = rra.lib()
    assert L.rrs_frontend_passes(0, 4096, 0) == rra.RRS_EINVAL
    assert L.rrs_frontend_passes(16, 100, 0) == rra.RRS_EINVAL
    assert L.rrs_frontend_passes(16, 4096, 16) == rra.RRS_EINVAL
    # answered without a device when the flags fix the form
    assert L.rrs_frontend_passes(16, 4096, rra.RRS_FLAG_NO_SMOOTH) == 1
    assert L.rrs_frontend_passes(16, 4096, rra.RRS_FLAG_TWO_PASS) == 3


def test_kron_shapes_accepted_and_rejected():
    """K = m 2^k with m in {12, 20, 28} is a valid size (Kronecker rotation);
    other non-powers of two are not, and G must divide K."""
    for K in (768, 1792, 3072, 10240, 12288, 14336):
        assert rra.rrs_weight_bytes(K, 8) > 0, K
        assert rra.rrs_workspace_bytes(4, K, 128) > 0, K
    for K in (100, 11008, 28 * 32, 24576, 28 * 1024, 12 * 32):
        assert rra.rrs_weight_bytes(K, 8) == 0, K
    assert rra.rrs_workspace_bytes(4, 14336, 4096) == 0   # 4096 does not divide 14336
    # layout sync | xq | dx | S | rows: a Kronecker K adds the M x K fp32 row area
    a = lambda n: (n + 255) // 256 * 256
    M, K, G = 2048, 14336, 128
    base = rra.rrs_sync_bytes(K, G) + a(rra.rrs_codes_bytes(M, K)) + a(4 * M) + a(4 * K // G)
    assert rra.rrs_workspace_bytes(M, K, G) == base + a(4 * M * K)
    assert rra.rrs_workspace_bytes(3, 768, 64) == rra.rrs_sync_bytes(768, 64) + a(2 * 2 * 384) + 256 + 256 + a(4 * 3 * 768)
    assert rra.rrs_gemm_form(8, 14336, 4096, 128) == rra.RRS_GEMM_FEW_TOKENS
    assert rra.rrs_gemm_form(8, 14336, 4096, 2048) == rra.RRS_GEMM_TILED
    assert rra.rrs_frontend_passes(8, 14336, 0) == 3
    assert rra.rrs_frontend_passes(8, 14336, rra.RRS_FLAG_NO_SMOOTH) == 1


def test_gemm_form():
    """Few-token kernel for M <= 64 (K split into whole 256-code rounds over
    8 waves, or 7, 6, 5, 4; groups nested in the waves' runs); up to
    M = 512 while its rounds of 256 workgroups (N/32 x M/64 of them) stay
    below the tiled kernel's (N/256 x M/128) times the per-round cost ratio
    (4.8 at K = 8192, 3.6 at 4096, 3 at 2048); tiled otherwise."""
    F, T = rra.RRS_GEMM_FEW_TOKENS, rra.RRS_GEMM_TILED
    assert rra.rrs_gemm_form(64, 8192, 8192, 128) == F
    assert rra.rrs_gemm_form(1, 2048, 1, 64) == F
    assert rra.rrs_gemm_form(1, 8192, 4096, 8192) == F
    assert rra.rrs_gemm_form(64, 1024, 4096, 128) == F      # 4 waves of one round
    assert rra.rrs_gemm_form(64, 512, 4096, 128) == T       # 2 rounds: no wave count divides them
    assert rra.rrs_gemm_form(64, 768, 4096, 64) == T        # 3 rounds
    assert rra.rrs_gemm_form(64, 4096, 4096, 32) == F       # G = 32: two groups per k-step
    # K = m 2^k: a multiple of 2048 with groups nested in the waves' runs of K/8
    assert rra.rrs_gemm_form(64, 14336, 4096, 128) == F     # runs of 1792 codes, groups of 128
    assert rra.rrs_gemm_form(64, 14336, 4096, 256) == F
    assert rra.rrs_gemm_form(64, 14336, 4096, 512) == T     # 512 does not divide 1792
    assert rra.rrs_gemm_form(64, 12288, 4096, 512) == F     # runs of 1536
    assert rra.rrs_gemm_form(64, 10240, 4096, 64) == F
    # other K: 7, 6, 5 or 4 waves of whole rounds (256 codes)
    assert rra.rrs_gemm_form(64, 3072, 4096, 64) == F       # 12 rounds, 6 waves
    assert rra.rrs_gemm_form(64, 5120, 4096, 64) == F       # 20 rounds, 5 waves
    assert rra.rrs_gemm_form(64, 7168, 4096, 256) == F      # 28 rounds, 7 waves
    assert rra.rrs_gemm_form(64, 3072, 4096, 1024) == F     # groups of two waves' runs
    # K = N = 8192: 2 .. 4 rounds against one tiled round (x 4.8); 5 is too many
    assert rra.rrs_gemm_form(65, 8192, 8192, 128) == F
    assert rra.rrs_gemm_form(256, 8192, 8192, 128) == F
    assert rra.rrs_gemm_form(257, 8192, 8192, 128) == T
    # K = N = 4096: up to 3 rounds (x 3.6)
    assert rra.rrs_gemm_form(384, 4096, 4096, 128) == F
    assert rra.rrs_gemm_form(385, 4096, 4096, 128) == T
    # gate/up-sized N: 4 rounds already at M = 65
    assert rra.rrs_gemm_form(65, 4096, 14336, 128) == T
    assert rra.rrs_gemm_form(513, 8192, 64, 128) == T       # past 512 tokens
    L = rra.lib()
    assert L.rrs_gemm_form(0, 4096, 64, 128) == rra.RRS_EINVAL
    assert L.rrs_gemm_form(4, 4096, 64, 8192) == rra.RRS_EINVAL
    assert L.rrs_gemm_form(4, 100, 64, 32) == rra.RRS_EINVAL
    assert L.rrs_gemm_form(4, 4096, 0, 128) == rra.RRS_EINVAL


def test_gemm_and_partials_reject():
    L = rra.lib()
    assert L.rrs_gemm(DUMMY, DUMMY, DUMMY, 4, 256, 0, 128, DUMMY, DUMMY, NULL) == rra.RRS_EINVAL
    assert L.rrs_gemm(DUMMY, DUMMY, NULL, 4, 256, 8, 128, DUMMY, DUMMY, NULL) == rra.RRS_EINVAL
    assert L.rrs_gemm(NULL, NULL, DUMMY, 0, 256, 8, 128, DUMMY, NULL, NULL) == rra.RRS_OK
    # partial windows must lie inside [0, M) x [0, N) and be non-empty
    for m0, m1, n0, n1 in [(0, 5, 0, 4), (2, 2, 0, 4), (0, 4, -1, 4), (0, 4, 0, 9), (3, 1, 0, 4)]:
        assert L.rrs_gemm_partials(DUMMY, 4, 256, 8, 128, DUMMY, m0, m1, n0, n1, DUMMY, NULL) == rra.RRS_EINVAL


def test_weights_calibrate_init_reject():
    L = rra.lib()
    assert L.rrs_prepare_weights(DUMMY, 96, 8, DUMMY, DUMMY, NULL) == rra.RRS_EINVAL
    assert L.rrs_prepare_weights(DUMMY, 256, 0, DUMMY, DUMMY, NULL) == rra.RRS_EINVAL
    assert L.rrs_prepare_weights(DUMMY, 256, 8, NULL, DUMMY, NULL) == rra.RRS_EINVAL
    assert L.rrs_calibrate_perm(DUMMY, 0, 256, DUMMY, DUMMY, 1024, NULL) == rra.RRS_EINVAL
    assert L.rrs_calibrate_perm(DUMMY, 8, 256, DUMMY, DUMMY, 1000, NULL) == rra.RRS_EINVAL
    assert L.rrs_workspace_init(NULL, 1024, NULL) == rra.RRS_EINVAL
    assert L.rrs_workspace_init(DUMMY, 100, NULL) == rra.RRS_EINVAL


def test_misaligned_pointers_rejected():
    """Every device pointer must be 16-byte aligned (the kernels move data in
    16-byte accesses); the host check rejects any other address."""
    L = rra.lib()
    odd = ctypes.c_void_p(0x1004)
    for key in ("X", "perm", "wq", "Y", "ws"):
        assert _lin(**{key: odd}) == rra.RRS_EINVAL, key
    assert L.rrs_gemm(odd, DUMMY, DUMMY, 4, 256, 8, 128, DUMMY, DUMMY, NULL) == rra.RRS_EINVAL
    assert L.rrs_gemm(DUMMY, DUMMY, DUMMY, 4, 256, 8, 128, DUMMY, odd, NULL) == rra.RRS_EINVAL
    assert L.rrs_gemm_partials(DUMMY, 4, 256, 8, 128, odd, 0, 4, 0, 8, DUMMY, NULL) == rra.RRS_EINVAL
    assert L.rrs_frontend(DUMMY, 4, 256, 64, odd, DUMMY, DUMMY, DUMMY, DUMMY, 1 << 20, 0, NULL) == rra.RRS_EINVAL
    assert L.rrs_prepare_weights(odd, 256, 8, DUMMY, DUMMY, NULL) == rra.RRS_EINVAL
    assert L.rrs_calibrate_perm(DUMMY, 8, 256, odd, DUMMY, 1024, NULL) == rra.RRS_EINVAL
    assert L.rrs_workspace_init(odd, 1024, NULL) == rra.RRS_EINVAL


def test_signed_entry_points_reject():
    """The signed entry points need a 16-byte aligned, non-null sign mask,
    and the front end rejects signs without the rotation."""
    L = rra.lib()
    odd = ctypes.c_void_p(0x1004)
    for dsign in (NULL, odd):
        assert L.rrs_linear_signed(DUMMY, 16, 256, 256, 128, DUMMY, dsign, DUMMY, DUMMY, DUMMY, 1 << 20,
                                   NULL) == rra.RRS_EINVAL
        assert L.rrs_prepare_weights_signed(DUMMY, 256, 8, DUMMY, dsign, DUMMY, NULL) == rra.RRS_EINVAL
        assert L.rrs_calibrate_perm_signed(DUMMY, 8, 256, dsign, DUMMY, DUMMY, 1024, NULL) == rra.RRS_EINVAL
        assert L.rrs_frontend_signed(DUMMY, 4, 256, 64, DUMMY, dsign, DUMMY, DUMMY, DUMMY, DUMMY, 1 << 20, 0,
                                     NULL) == rra.RRS_EINVAL
    assert L.rrs_frontend_signed(DUMMY, 4, 256, 64, DUMMY, DUMMY, DUMMY, DUMMY, DUMMY, DUMMY, 1 << 20,
                                 rra.RRS_FLAG_NO_ROTATE, NULL) == rra.RRS_EINVAL
    assert L.rrs_frontend_signed(NULL, 0, 256, 64, DUMMY, DUMMY, NULL, NULL, DUMMY, DUMMY, 1 << 20, 0,
                                 NULL) == rra.RRS_OK
    assert L.rrs_linear_signed(NULL, 0, 256, 256, 128, DUMMY, DUMMY, DUMMY, NULL, DUMMY, 1 << 20,
                               NULL) == rra.RRS_OK


def test_binding_fails_loudly_without_library(monkeypatch):
    monkeypatch.setattr(rra, "_lib", None)
    monkeypatch.setattr(rra, "LIB_PATH", "/nonexistent/librrs.so")
    with pytest.raises(rra.RRSLibraryMissing):
        rra.rrs_weight_bytes(256, 4)


def test_ablation_entry_points_reject():
    """The _ex entry points: weights and calibration accept only
    RRS_FLAG_NO_ROTATE; the layer accepts the front end's flags; a sign mask
    together with RRS_FLAG_NO_ROTATE is rejected everywhere (the signs belong
    to the rotation); M = 0 stays a no-op."""
    L = rra.lib()
    NR = rra.RRS_FLAG_NO_ROTATE
    for flags in (rra.RRS_FLAG_NO_SMOOTH, rra.RRS_FLAG_TWO_PASS, rra.RRS_FLAG_TEST_GIVE_UP, 64):
        assert L.rrs_prepare_weights_ex(DUMMY, 256, 8, DUMMY, NULL, flags, DUMMY, NULL) == rra.RRS_EINVAL
        assert L.rrs_calibrate_perm_ex(DUMMY, 8, 256, NULL, flags, DUMMY, DUMMY, 1024, NULL) == rra.RRS_EINVAL
    assert L.rrs_prepare_weights_ex(DUMMY, 256, 8, DUMMY, DUMMY, NR, DUMMY, NULL) == rra.RRS_EINVAL
    assert L.rrs_calibrate_perm_ex(DUMMY, 8, 256, DUMMY, NR, DUMMY, DUMMY, 1024, NULL) == rra.RRS_EINVAL
    assert L.rrs_linear_ex(DUMMY, 16, 256, 256, 128, DUMMY, DUMMY, NR, DUMMY, DUMMY, DUMMY, 1 << 20,
                           NULL) == rra.RRS_EINVAL
    assert L.rrs_linear_ex(DUMMY, 16, 256, 256, 128, DUMMY, NULL, 64, DUMMY, DUMMY, DUMMY, 1 << 20,
                           NULL) == rra.RRS_EINVAL
    assert L.rrs_linear_ex(DUMMY, 16, 256, 256, 96, DUMMY, NULL, NR, DUMMY, DUMMY, DUMMY, 1 << 20,
                           NULL) == rra.RRS_EINVAL
    assert L.rrs_linear_ex(NULL, 0, 256, 256, 128, DUMMY, NULL, NR, DUMMY, NULL, DUMMY, 1 << 20,
                           NULL) == rra.RRS_OK
    odd = ctypes.c_void_p(0x1004)
    assert L.rrs_linear_ex(DUMMY, 16, 256, 256, 128, DUMMY, odd, 0, DUMMY, DUMMY, DUMMY, 1 << 20,
                           NULL) == rra.RRS_EINVAL


def test_noalloc_rejects_on_host():
    """rrs_linear_noalloc checks its arguments and the scratch capacity on the
    host before touching the device."""
    L = rra.lib()
    assert L.rrs_linear_noalloc(DUMMY, 16, 100, 64, 32, DUMMY, DUMMY, DUMMY, NULL) == rra.RRS_EINVAL
    assert L.rrs_linear_noalloc(DUMMY, 16, 4096, 0, 128, DUMMY, DUMMY, DUMMY, NULL) == rra.RRS_EINVAL
    assert L.rrs_linear_noalloc(DUMMY, 16, 4096, 64, 128, NULL, DUMMY, DUMMY, NULL) == rra.RRS_EINVAL
    assert L.rrs_linear_noalloc(ctypes.c_void_p(0x1004), 16, 4096, 64, 128, DUMMY, DUMMY, DUMMY,
                                NULL) == rra.RRS_EINVAL
    assert L.rrs_linear_noalloc(DUMMY, 12167, 4096, 64, 128, DUMMY, DUMMY, DUMMY, NULL) == rra.RRS_ETOOBIG
    assert L.rrs_linear_noalloc(NULL, 0, 4096, 64, 128, DUMMY, DUMMY, NULL, NULL) == rra.RRS_OK


def test_code_layout_sizes_and_helpers():
    """The stored code layout (row pairs, 64-byte pieces side by side): its
    size query, and the binding's reading and writing helpers against the
    byte-offset formula the header states."""
    import numpy as np
    import torch
    assert rra.rrs_codes_bytes(4, 4096) == 4 * 2048
    assert rra.rrs_codes_bytes(3, 4096) == 4 * 2048     # an odd row count rounds up to a pair
    assert rra.rrs_codes_bytes(5, 64) == 3 * 2 * 64     # K = 64: 32 of each 64-byte piece used
    assert rra.rrs_codes_bytes(1, 14336) == 2 * 7168
    assert rra.rrs_codes_bytes(4, 100) == 0 and rra.rrs_codes_bytes(-1, 256) == 0
    assert rra.rrs_weight_bytes(256, 3) == 512 + 256 and rra.rrs_weight_bytes(64, 5) == 512 + 256  # 384 code bytes, 256-aligned

    def off(r, b, rs):
        return (r // 2) * 2 * rs + (b // 64) * 128 + (r % 2) * 64 + b % 64

    for rows, K in [(5, 64), (6, 128), (7, 1024), (3, 1792), (4, 4096)]:
        kb = K // 2
        rs = (kb + 63) // 64 * 64
        codes = torch.from_numpy(np.random.default_rng(rows + K).integers(0, 256, (rows, kb), dtype=np.uint8))
        buf = rra.codes_buffer(codes, K)
        assert buf.numel() == rra.rrs_codes_bytes(rows, K)
        b = buf.numpy()
        idx = np.array([[off(r, c, rs) for c in range(kb)] for r in range(rows)])
        assert np.array_equal(b[idx], codes.numpy())
        assert torch.equal(rra.codes_matrix(buf, rows, K), codes)
