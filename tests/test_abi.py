"""The C ABI without a GPU: the library loads, exports every entry point
include/fp8q.h declares, and its host-side validation rejects bad
arguments before anything would be enqueued (none of these calls reaches
the HIP runtime)."""
import ctypes
import os
import re
import subprocess

import pytest

from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "fp8q.h")
FAKE = 0x10000  # a 16-byte aligned address that is never dereferenced


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fp8q_\w+)\s*\(", text)))


def test_header_declares_the_binding_symbols(fq):
    assert declared_functions() == sorted(fq.SYMBOLS)


def test_library_exports_every_declared_symbol(fq):
    out = subprocess.run(["nm", "-D", "--defined-only", fq.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\bT (fp8q_\w+)$", out, flags=re.M))
    for name in declared_functions():
        assert name in exported, name
        assert getattr(fq.lib(), name) is not None


def test_version_and_status_strings(fq):
    L = fq.lib()
    assert L.fp8q_version() == 100
    assert L.fp8q_status_string(0) == b"ok"
    for s in range(1, 6):
        assert L.fp8q_status_string(s) not in (b"ok", b"unknown status")
    assert L.fp8q_status_string(99) == b"unknown status"


def test_scaler_struct_layout(fq):
    assert fq.SCALER_BYTES == 1024 * 4 + 10 * 4 + 8
    assert fq.SCALER_SCALE_OFFSET == 1024 * 4 + 6 * 4
    assert fq.Scaler.ema.offset % 8 == 0


def _rc(fq, name, *args):
    rc = getattr(fq.lib(), name)(*args)
    return rc, fq.lib().fp8q_last_error().decode()


def test_scaler_init_stat_validation(fq):
    L = fq.lib()
    f = ctypes.c_float
    assert _rc(fq, "fp8q_delayed_scaler_init_stat", FAKE, 16, f(448.0), f(1e-12), f(1.0), 3, f(0.0), None)[0] == fq.EINVAL
    assert _rc(fq, "fp8q_delayed_scaler_init_stat", FAKE, 16, f(448.0), f(1e-12), f(1.0), 2, f(0.0), None)[0] == fq.EINVAL
    assert _rc(fq, "fp8q_delayed_scaler_init_stat", FAKE, 16, f(448.0), f(1e-12), f(1.0), 2, f(1.5), None)[0] == fq.EINVAL
    assert _rc(fq, "fp8q_delayed_scaler_init_stat", FAKE, 0, f(448.0), f(1e-12), f(1.0), 1, f(0.0), None)[0] == fq.EINVAL
    assert _rc(fq, "fp8q_delayed_scaler_init_stat", FAKE + 4, 16, f(448.0), f(1e-12), f(1.0), 1, f(0.0),
               None)[0] == fq.EALIGN
    assert L.fp8q_delayed_scaler_update(FAKE + 4, FAKE, None) == fq.EALIGN


def test_amax_validation(fq):
    assert _rc(fq, "fp8q_amax", None, 0, 10, FAKE, None)[0] == fq.EINVAL
    assert _rc(fq, "fp8q_amax", FAKE, 0, 10, None, None)[0] == fq.EINVAL
    assert _rc(fq, "fp8q_amax", FAKE, 2, 10, FAKE, None)[0] == fq.EINVAL  # dtype
    assert _rc(fq, "fp8q_amax", FAKE, 0, 0, FAKE, None)[0] == fq.EINVAL
    assert _rc(fq, "fp8q_amax", FAKE + 4, 0, 10, FAKE, None)[0] == fq.EALIGN


def test_quantize_tensor_validation(fq):
    f = "fp8q_quantize_tensor"
    assert _rc(fq, f, FAKE, 0, 10, 0, None, FAKE, None, None)[0] == fq.EINVAL  # scale
    assert _rc(fq, f, FAKE, 0, 10, 7, FAKE, FAKE, None, None)[0] == fq.EINVAL  # format
    assert _rc(fq, f, FAKE, 0, -1, 0, FAKE, FAKE, None, None)[0] == fq.EINVAL
    assert _rc(fq, f, FAKE, 0, 10, 0, FAKE, FAKE + 8, None, None)[0] == fq.EALIGN
    assert _rc(fq, f, FAKE, 0, 10, 0, FAKE, FAKE, FAKE + 2, None)[0] == fq.EALIGN


@pytest.mark.parametrize("fn,br", [("fp8q_quantize_1x128", 1), ("fp8q_quantize_128x128", 128)])
def test_block_quantize_validation(fq, fn, br):
    ok = dict(x=FAKE, dt=0, rows=128, cols=256, ldx=256, f=0, eps=1e-12, q=FAKE, ldq=256, s=FAKE, ld_s=2)

    def call(**kw):
        a = {**ok, **kw}
        return _rc(fq, fn, a["x"], a["dt"], a["rows"], a["cols"], a["ldx"], a["f"], a["eps"], a["q"],
                   a["ldq"], a["s"], a["ld_s"], None)

    assert call(x=None)[0] == fq.EINVAL
    assert call(s=None)[0] == fq.EINVAL
    assert call(dt=3)[0] == fq.EINVAL
    assert call(eps=0.0)[0] == fq.EINVAL
    assert call(eps=float("nan"))[0] == fq.EINVAL
    rc, msg = call(cols=200, ldx=256, ldq=256)
    assert rc == fq.ESHAPE and "multiple of 128" in msg
    assert call(ldx=128)[0] == fq.EINVAL
    assert call(ld_s=1)[0] == fq.EINVAL
    assert call(x=FAKE + 4)[0] == fq.EALIGN
    assert call(ldx=258)[0] == fq.EALIGN
    assert call(ldq=264)[0] == fq.EALIGN
    if br == 128:
        assert call(rows=100)[0] == fq.ESHAPE
    else:
        assert call(rows=0)[0] == fq.EINVAL


def test_transposed_quantize_validation(fq):
    ok = dict(x=FAKE, dt=1, rows=256, cols=128, ldx=128, f=0, eps=1e-12, q=FAKE, ldq=256, s=FAKE, ld_s=2)

    def call(**kw):
        a = {**ok, **kw}
        return _rc(fq, "fp8q_quantize_1x128_t", a["x"], a["dt"], a["rows"], a["cols"], a["ldx"], a["f"],
                   a["eps"], a["q"], a["ldq"], a["s"], a["ld_s"], None)

    assert call(q=None)[0] == fq.EINVAL
    assert call(f=2)[0] == fq.EINVAL
    rc, msg = call(rows=200, ldq=256)
    assert rc == fq.ESHAPE and "multiple of 128" in msg
    rc, msg = call(cols=96, ldx=128)
    assert rc == fq.ESHAPE and "multiple of 64" in msg
    assert call(ldq=128)[0] == fq.EINVAL
    assert call(ld_s=1)[0] == fq.EINVAL
    assert call(ldx=132)[0] == fq.EALIGN
    assert call(ldq=264)[0] == fq.EALIGN


def test_scaler_validation(fq):
    assert _rc(fq, "fp8q_delayed_scaler_init", None, 16, 448.0, 1e-12, 1.0, None)[0] == fq.EINVAL
    assert _rc(fq, "fp8q_delayed_scaler_init", FAKE, 0, 448.0, 1e-12, 1.0, None)[0] == fq.EINVAL
    assert _rc(fq, "fp8q_delayed_scaler_init", FAKE, 1025, 448.0, 1e-12, 1.0, None)[0] == fq.EINVAL
    assert _rc(fq, "fp8q_delayed_scaler_init", FAKE, 16, -1.0, 1e-12, 1.0, None)[0] == fq.EINVAL
    assert _rc(fq, "fp8q_delayed_scaler_init", FAKE, 16, 448.0, 0.0, 1.0, None)[0] == fq.EINVAL
    assert _rc(fq, "fp8q_delayed_scaler_init", FAKE + 1, 16, 448.0, 1e-12, 1.0, None)[0] == fq.EALIGN
    assert _rc(fq, "fp8q_delayed_scaler_update", None, FAKE, None)[0] == fq.EINVAL
    assert _rc(fq, "fp8q_delayed_scaler_update", None, None, None)[0] == fq.EINVAL
    # a NULL amax means the state's own accumulator: alignment is still checked
    assert _rc(fq, "fp8q_delayed_scaler_update", FAKE + 4, None, None)[0] == fq.EALIGN
    assert _rc(fq, "fp8q_delayed_scaler_update", FAKE, FAKE + 2, None)[0] == fq.EALIGN


def test_quantize_tensor_delayed_validation(fq):
    f = "fp8q_quantize_tensor_delayed"
    assert _rc(fq, f, FAKE, 1, 1024, 0, None, FAKE, None, 0, None)[0] == fq.EINVAL      # no state
    assert _rc(fq, f, None, 1, 1024, 0, FAKE, FAKE, None, 0, None)[0] == fq.EINVAL      # no x
    assert _rc(fq, f, FAKE, 7, 1024, 0, FAKE, FAKE, None, 0, None)[0] == fq.EINVAL      # dtype
    assert _rc(fq, f, FAKE, 1, 1024, 3, FAKE, FAKE, None, 0, None)[0] == fq.EINVAL      # format
    assert _rc(fq, f, FAKE, 1, 1024, 0, FAKE, FAKE, FAKE, 9, None)[0] == fq.EINVAL      # round-trip dtype
    assert _rc(fq, f, FAKE, 1, 0, 0, FAKE, FAKE, None, 0, None)[0] == fq.EINVAL         # n
    assert _rc(fq, f, FAKE + 2, 1, 1024, 0, FAKE, FAKE, None, 0, None)[0] == fq.EALIGN  # x
    assert _rc(fq, f, FAKE, 1, 1024, 0, FAKE + 4, FAKE, None, 0, None)[0] == fq.EALIGN  # state
    assert _rc(fq, f, FAKE, 1, 1024, 0, FAKE, FAKE, FAKE + 8, 0, None)[0] == fq.EALIGN  # y


def test_gemm_qt_validation(fq):
    ok = dict(A=FAKE, fa=1, lda=256, sA=FAKE, sA_sm=2, sA_skb=1, B=FAKE, fb=0, ldb=256, sB=FAKE, gb=2, sB_sn=2,
              sB_skb=1, fc=1, eps=1e-12, Ct=FAKE, ldt=256, Cst=FAKE, ld_st=2, Cq=None, ldcq=128, Cs=None, ld_cs=1,
              M=256, N=128, K=256)

    def call(**kw):
        a = {**ok, **kw}
        return _rc(fq, "fp8q_gemm_blockscaled_qt", a["A"], a["fa"], a["lda"], a["sA"], a["sA_sm"], a["sA_skb"],
                   a["B"], a["fb"], a["ldb"], a["sB"], a["gb"], a["sB_sn"], a["sB_skb"], a["fc"],
                   ctypes.c_float(a["eps"]), a["Ct"], a["ldt"], a["Cst"], a["ld_st"], a["Cq"], a["ldcq"], a["Cs"],
                   a["ld_cs"], a["M"], a["N"], a["K"], None)

    assert call(Ct=None)[0] == fq.EINVAL
    assert call(Cst=None)[0] == fq.EINVAL
    assert call(Cq=FAKE)[0] == fq.EINVAL           # Cq without Cs
    assert call(fc=2)[0] == fq.EINVAL
    assert call(eps=0.0)[0] == fq.EINVAL
    rc, msg = call(M=200, ldt=256)
    assert rc == fq.ESHAPE and "multiples of 128" in msg
    assert call(K=200, lda=256, ldb=256)[0] == fq.ESHAPE
    assert call(N=100, Cq=FAKE, Cs=FAKE)[0] == fq.ESHAPE   # the row-wise output needs N % 128 == 0
    assert call(ldt=128)[0] == fq.EINVAL
    assert call(ld_st=1)[0] == fq.EINVAL
    assert call(Cq=FAKE, Cs=FAKE, ldcq=64)[0] == fq.EINVAL
    assert call(Ct=FAKE + 8)[0] == fq.EALIGN
    assert call(ldt=264)[0] == fq.EALIGN
    assert call(Cst=FAKE + 2)[0] == fq.EALIGN


def test_dequantize_validation(fq):
    f = "fp8q_dequantize"
    assert _rc(fq, f, FAKE, 0, 4, 256, 256, FAKE, 5, 2, FAKE, 0, 256, None)[0] == fq.EINVAL  # gran
    assert _rc(fq, f, FAKE, 0, 4, 200, 200, FAKE, 1, 2, FAKE, 0, 200, None)[0] == fq.ESHAPE
    assert _rc(fq, f, FAKE, 0, 4, 256, 256, FAKE, 1, 1, FAKE, 0, 256, None)[0] == fq.EINVAL  # ld_s
    assert _rc(fq, f, FAKE, 0, 4, 256, 258, FAKE, 1, 2, FAKE, 0, 256, None)[0] == fq.EALIGN
    assert _rc(fq, f, FAKE + 4, 0, 4, 256, 256, FAKE, 1, 2, FAKE, 0, 256, None)[0] == fq.EALIGN


def test_gemm_validation(fq):
    ok = dict(A=FAKE, fa=0, lda=256, sA=FAKE, sA_sm=2, sA_skb=1, B=FAKE, fb=0, ldb=256, sB=FAKE, gb=2,
              sB_sn=2, sB_skb=1, C=FAKE, odt=0, ldc=128, M=64, N=128, K=256)

    def call(**kw):
        a = {**ok, **kw}
        return _rc(fq, "fp8q_gemm_blockscaled", a["A"], a["fa"], a["lda"], a["sA"], a["sA_sm"], a["sA_skb"],
                   a["B"], a["fb"], a["ldb"], a["sB"], a["gb"], a["sB_sn"], a["sB_skb"], a["C"], a["odt"],
                   a["ldc"], a["M"], a["N"], a["K"], None)

    assert call(A=None)[0] == fq.EINVAL
    assert call(sB=None)[0] == fq.EINVAL
    assert call(gb=0)[0] == fq.EINVAL
    assert call(fa=2)[0] == fq.EINVAL
    assert call(M=0)[0] == fq.EINVAL
    assert call(K=200, lda=208, ldb=208)[0] == fq.ESHAPE
    assert call(lda=128)[0] == fq.EINVAL
    assert call(ldc=64)[0] == fq.EINVAL
    assert call(sA_sm=-1)[0] == fq.EINVAL
    assert call(A=FAKE + 8)[0] == fq.EALIGN
    assert call(ldb=264)[0] == fq.EALIGN


def test_mx_validation(fq):
    q = "fp8q_quantize_mx"
    assert _rc(fq, q, None, 1, 4, 256, 256, 0, FAKE, 256, FAKE, 8, None)[0] == fq.EINVAL
    assert _rc(fq, q, FAKE, 1, 4, 256, 256, 2, FAKE, 256, FAKE, 8, None)[0] == fq.EINVAL  # format
    rc, msg = _rc(fq, q, FAKE, 1, 4, 240, 256, 0, FAKE, 256, FAKE, 8, None)
    assert rc == fq.ESHAPE and "multiple of 32" in msg
    assert _rc(fq, q, FAKE, 1, 4, 256, 256, 0, FAKE, 256, FAKE, 7, None)[0] == fq.EINVAL  # ld_s
    assert _rc(fq, q, FAKE, 1, 4, 256, 260, 0, FAKE, 256, FAKE, 8, None)[0] == fq.EALIGN  # bf16 rows
    assert _rc(fq, q, FAKE, 1, 4, 256, 256, 0, FAKE + 8, 256, FAKE, 8, None)[0] == fq.EALIGN
    d = "fp8q_dequantize_mx"
    assert _rc(fq, d, FAKE, 0, 4, 256, 256, None, 8, FAKE, 1, 256, None)[0] == fq.EINVAL
    assert _rc(fq, d, FAKE, 0, 4, 96 + 4, 256, FAKE, 8, FAKE, 1, 256, None)[0] == fq.ESHAPE
    assert _rc(fq, d, FAKE, 0, 4, 256, 260, FAKE, 8, FAKE, 1, 256, None)[0] == fq.EALIGN  # ldq % 8
    assert _rc(fq, d, FAKE, 0, 4, 256, 256, FAKE, 8, FAKE, 1, 260, None)[0] == fq.EALIGN  # bf16 rows
    g = "fp8q_gemm_mx"
    okg = dict(A=FAKE, fa=0, lda=256, sA=FAKE, ld_sa=8, B=FAKE, fb=0, ldb=256, sB=FAKE, ld_sb=8, C=FAKE, odt=0,
               ldc=128, M=64, N=128, K=256)

    def call(**kw):
        a = {**okg, **kw}
        return _rc(fq, g, a["A"], a["fa"], a["lda"], a["sA"], a["ld_sa"], a["B"], a["fb"], a["ldb"], a["sB"],
                   a["ld_sb"], a["C"], a["odt"], a["ldc"], a["M"], a["N"], a["K"], None)

    assert call(sB=None)[0] == fq.EINVAL
    assert call(fb=5)[0] == fq.EINVAL
    rc, msg = call(K=224, lda=224, ldb=224, ld_sa=8, ld_sb=8)
    assert rc == fq.ESHAPE and "multiple of 128" in msg
    assert call(ld_sa=4)[0] == fq.EINVAL
    assert call(ld_sb=10)[0] == fq.EALIGN
    assert call(lda=264)[0] == fq.EALIGN
    assert call(sA=FAKE + 2)[0] == fq.EALIGN


def test_gemm_q_validation(fq):
    ok = dict(A=FAKE, fa=0, lda=256, sA=FAKE, sA_sm=2, sA_skb=1, B=FAKE, fb=0, ldb=256, sB=FAKE, gb=2,
              sB_sn=2, sB_skb=1, fc=0, eps=1e-12, Cq=FAKE, ldcq=256, Cs=FAKE, ld_cs=2, M=64, N=256, K=256)

    def call(**kw):
        a = {**ok, **kw}
        return _rc(fq, "fp8q_gemm_blockscaled_q", a["A"], a["fa"], a["lda"], a["sA"], a["sA_sm"], a["sA_skb"],
                   a["B"], a["fb"], a["ldb"], a["sB"], a["gb"], a["sB_sn"], a["sB_skb"], a["fc"],
                   ctypes.c_float(a["eps"]), a["Cq"], a["ldcq"], a["Cs"], a["ld_cs"], a["M"], a["N"], a["K"], None)

    assert call(Cs=None)[0] == fq.EINVAL
    assert call(fc=3)[0] == fq.EINVAL
    assert call(eps=0.0)[0] == fq.EINVAL
    rc, msg = call(N=192, ldcq=192)
    assert rc == fq.ESHAPE and "multiples of 128" in msg
    assert call(ld_cs=1)[0] == fq.EINVAL
    assert call(ldcq=128)[0] == fq.EINVAL
    assert call(Cs=FAKE + 2)[0] == fq.EALIGN


def test_gemm_operand_span_limit(fq):
    """Operands of 4 GiB or more are refused before any launch (the LDS copies
    take 32-bit byte offsets)."""
    M, K = 1 << 20, 8192  # (M - 1) * lda + K > 2^32
    rc, msg = _rc(fq, "fp8q_gemm_blockscaled", FAKE, 0, K, FAKE, K // 128, 1, FAKE, 0, K, FAKE, 2, K // 128, 1,
                  FAKE, 0, 256, M, 256, K, None)
    assert rc == fq.ESHAPE and "4 GiB" in msg
    rc, msg = _rc(fq, "fp8q_gemm_blockscaled_fast", FAKE, 0, K, FAKE, K // 128, 1, FAKE, 0, K, FAKE, 2, K // 128,
                  1, FAKE, 0, M, 256, M, K, None)  # B spans 4 GiB
    assert rc == fq.ESHAPE and "4 GiB" in msg
    rc, msg = _rc(fq, "fp8q_gemm_mx", FAKE, 0, K, FAKE, K // 32, FAKE, 0, K, FAKE, K // 32, FAKE, 0, 256, M, 256, K,
                  None)
    assert rc == fq.ESHAPE and "4 GiB" in msg
    rc, msg = _rc(fq, "fp8q_gemm_blockscaled_q", FAKE, 0, K, FAKE, K // 128, 1, FAKE, 0, K, FAKE, 2, K // 128, 1, 0,
                  ctypes.c_float(1e-12), FAKE, 256, FAKE, 2, M, 256, K, None)
    assert rc == fq.ESHAPE and "4 GiB" in msg
