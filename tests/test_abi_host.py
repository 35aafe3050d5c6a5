"""Host-side checks of the C ABI (no GPU needed, nothing is launched).

* libqlora.so loads and exports every function include/qlora.h declares;
* size arithmetic against sizes printed on the pages (tests/golden);
* argument validation returns the documented status before any launch.
"""

from __future__ import annotations

import ctypes
import os
import re

import pytest

from quantized_frozen_weight_amd import binding as Q

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qlora.h")
PROBE_HEADER = os.path.join(ROOT, "include", "qlora_probe.h")
GOLDEN = os.path.join(ROOT, "tests", "golden", "page_sizes.txt")

FAKE = 0x100000   # aligned, never dereferenced: every call below fails validation


@pytest.fixture(scope="module")
def lib():
    return Q.lib()


def declared_functions(header=HEADER):
    text = open(header).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(qlora_\w+)\s*\(", text, re.M)))


def test_header_declares_the_abi():
    names = declared_functions()
    for n in ("qlora_quantize", "qlora_fwd", "qlora_bwd", "qlora_fwd_workspace",
              "qlora_bwd_workspace", "qlora_weight_bytes", "qlora_status_str",
              "qlora_quantize_rows", "qlora_fwd_acc"):
        assert n in names
    assert set(names) == set(Q.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    for n in declared_functions() + declared_functions(PROBE_HEADER):
        assert hasattr(lib, n), f"{n} not exported"


def test_probe_header_matches_the_binding():
    assert set(declared_functions(PROBE_HEADER)) == set(Q.PROBE_EXPORTS)


def test_loaded_library_is_the_in_tree_build(lib):
    """The binding maps exactly the libqlora.so built next to it."""
    assert os.path.realpath(Q.loaded_path()) == os.path.realpath(Q.LIB_PATH)


def test_backward_kernel_names(lib):
    """The kernel-name query follows the backward's dispatch (and rejects
    what qlora_bwd would reject)."""
    def name(K, N, r, M, dtype):
        v = lib.qlora_bwd_main_kernel(ctypes.byref(_lin(K, N, r)), M, dtype)
        return None if v is None else v.decode()
    assert name(1024, 1024, 8, 1024, Q.QLORA_BF16) == "bwd_pc_kernel"
    assert name(768, 2304, 4, 4096, Q.QLORA_BF16) == "bwd_wide_kernel (128 x 64 tiles)"
    assert name(3072, 768, 4, 4096, Q.QLORA_BF16) == "bwd_wide_kernel"
    assert name(2048, 16384, 8, 512, Q.QLORA_BF16).startswith("bwd_wide_kernel<SPLIT>")
    assert name(256, 256, 4, 64, Q.QLORA_F32) == "gemm_dx_f32_kernel"
    assert name(100, 256, 4, 64, Q.QLORA_BF16) is None      # K % 16 != 0


def test_status_strings(lib):
    for code in range(6):
        assert Q.qlora_status_str(code)
    assert Q.qlora_status_str(99) == "unknown status"


def _golden():
    rows = []
    for line in open(GOLDEN):
        line = line.split("#")[0].strip()
        if line:
            name, K, N, r, val = line.split()
            rows.append((name, int(K), int(N), int(r), float(val)))
    return rows


def test_sizes_match_the_pages(lib):
    for name, K, N, r, val in _golden():
        if name == "fp32_kernel_mib":
            # the frozen kernel the pages list in float32 ...
            assert round(K * N * 4 / 2 ** 20, 3) == val
            # ... is a quarter of that as int8 codes, an eighth as 4-bit
            cb, sb = Q.qlora_weight_bytes(K, N, "w8")
            assert cb * 4 == K * N * 4 and sb == N * 4
            cb4, sb4 = Q.qlora_weight_bytes(K, N, "w4g128")
            assert cb4 * 8 == K * N * 4 and sb4 == N * (K // 128) * 2
        elif name == "fp32_lora_A_mib":
            assert round(K * r * 4 / 2 ** 20, 3) == val
        elif name == "dense_params":
            assert K * N == val
        elif name == "lora_params":
            assert r * (K + N) == val


def test_weight_bytes_rejects_bad_shapes(lib):
    for K, N, fmt in ((8, 16, "w8"), (16, 20, "w8"), (144, 16, "w4g128")):
        with pytest.raises(Q.QloraError) as e:
            Q.qlora_weight_bytes(K, N, fmt)
        assert e.value.status == Q.QLORA_EINVAL


def _lin(K=256, N=256, r=4, fmt=Q.QLORA_W8, ptr=FAKE):
    return Q.qlora_linear(K, N, r, 8.0, fmt, ptr, ptr, ptr, ptr)


def _fwd_ws(lib, lin, M=64, dtype=Q.QLORA_BF16):
    n = ctypes.c_size_t()
    st = lib.qlora_fwd_workspace(ctypes.byref(lin), M, dtype, ctypes.byref(n))
    return st, n.value


def test_workspace_queries(lib):
    st, n = _fwd_ws(lib, _lin())
    assert st == Q.QLORA_OK and n >= 64 * 256 + 64 * 4 + 64 * 4 * 4
    n2 = ctypes.c_size_t()
    assert lib.qlora_bwd_workspace(ctypes.byref(_lin()), 64, Q.QLORA_BF16,
                                   ctypes.byref(n2)) == Q.QLORA_OK
    # t and u [M, r] float32, and one partial sum of dA and of dB per block
    # of 64 rows: [1, r, K + N] float32
    assert n2.value >= 2 * 64 * 4 * 4 + 4 * (256 + 256) * 4
    n3 = ctypes.c_size_t()
    assert lib.qlora_bwd_workspace(ctypes.byref(_lin()), 1000, Q.QLORA_BF16,
                                   ctypes.byref(n3)) == Q.QLORA_OK
    assert n3.value >= 2 * 1000 * 4 * 4 + 16 * 4 * (256 + 256) * 4


def _bwd_ws(lib, lin, M, dtype):
    n = ctypes.c_size_t()
    assert lib.qlora_bwd_workspace(ctypes.byref(lin), M, dtype, ctypes.byref(n)) == Q.QLORA_OK
    return n.value


def test_split_contraction_workspace(lib):
    # 512 rows of a 2048 -> 16384 layer: 4 x 16 output tiles of 128 x 128 over
    # 256 stages of 64 n split 8 ways -> 8 partial products of [512, 2048]
    # float32 plus 8 partial u [512, 8] on top of t, u and the partial sums
    lin = _lin(K=2048, N=16384, r=8)
    bf = _bwd_ws(lib, lin, 512, Q.QLORA_BF16)
    f32 = _bwd_ws(lib, lin, 512, Q.QLORA_F32)
    assert bf - f32 >= 8 * 512 * 2048 * 4 + 8 * 512 * 8 * 4
    assert bf - f32 <= 8 * 512 * 2048 * 4 + 8 * 512 * 8 * 4 + 2 * 256
    # a short contraction does not split (the 1024 x 1024 layers)
    lin = _lin(K=1024, N=1024, r=8)
    assert _bwd_ws(lib, lin, 1024, Q.QLORA_BF16) == _bwd_ws(lib, lin, 1024, Q.QLORA_F32)


def test_split_forward_workspace(lib):
    # 512 rows of a 16384 -> 2048 int8 layer: 4 x 16 output tiles of 128 x 128
    # over 128 stages of 128 k split 8 ways -> 8 int32 partial sums of
    # [512, 2048]; the 4-bit product of the same shape (256 stages of 64 k)
    # splits 8 ways too, into float32 partial sums of the same size
    st, w8 = _fwd_ws(lib, _lin(K=16384, N=2048, r=8), M=512)
    assert st == Q.QLORA_OK
    # codes, scales, t, and the row pass split over 2048-entry slices of k:
    # per row and slice the abs-max bits and r sums, 512 x 8 x (1 + 8) floats
    base = 512 * 16384 + 512 * 4 + 512 * 8 * 4 + 512 * 8 * 9 * 4
    assert w8 >= base + 8 * 512 * 2048 * 4
    assert w8 <= base + 8 * 512 * 2048 * 4 + 5 * 256
    st, w4 = _fwd_ws(lib, _lin(K=16384, N=2048, r=8, fmt=Q.QLORA_W4G128), M=512)
    assert st == Q.QLORA_OK
    assert base + 8 * 512 * 2048 * 4 <= w4 <= base + 8 * 512 * 2048 * 4 + 5 * 256
    # 2048 rows (16 x 16 tiles) do not split: no partial sums
    st, w4 = _fwd_ws(lib, _lin(K=16384, N=2048, r=8, fmt=Q.QLORA_W4G128), M=2048)
    base4 = 2048 * 16384 + 2048 * 4 + 2048 * 8 * 4 + 2048 * 8 * 9 * 4
    assert st == Q.QLORA_OK and base4 <= w4 < base4 + 5 * 256
    # outlier-compensated weights: 4 x 32 tiles of 128 x 64 split 4 ways ->
    # int32 partial sums and float partial corrections, 16 MiB each
    st, w8o = _fwd_ws(lib, _lin(K=16384, N=2048, r=8, fmt=Q.QLORA_W8O), M=512)
    assert st == Q.QLORA_OK
    base_o = base + 512 * 4                            # and the code sums
    assert base_o + 2 * 4 * 512 * 2048 * 4 <= w8o <= base_o + 2 * 4 * 512 * 2048 * 4 + 7 * 256
    # a short contraction does not split
    st, short = _fwd_ws(lib, _lin(K=1024, N=1024, r=8), M=1024)
    assert short < 1024 * 1024 + 1024 * 4 + 1024 * 8 * 4 + 4 * 256


def _w4_split_bytes(M, N, K):
    """Float32 partial sums of the split 4-bit forward, as documented: at
    most 128 tiles of 128 x 128 split (up to 8 ways) while the grid stays
    within 512 blocks and each split keeps at least 8 stages of 64 k."""
    tiles = ((M + 127) // 128) * ((N + 127) // 128)
    nk, sp = K // 64, 1
    if tiles <= 128:
        while sp < 8 and tiles * sp * 2 <= 512 and nk // (sp * 2) >= 8:
            sp *= 2
    if sp == 1:
        return 0
    nks = (nk + sp - 1) // sp
    return ((nk + nks - 1) // nks) * tiles * 128 * 128 * 4


@pytest.mark.parametrize("K,r,slices,R", [(4096, 8, 0, 0), (4224, 8, 3, 8), (8192, 3, 4, 4),
                                          (16384, 1, 8, 1), (16384, 9, 0, 0)])
def test_row_split_workspace(lib, K, r, slices, R):
    # rows of 4097..16384 entries with rank up to 8 add the split row pass's
    # scratch (abs-max bits and R sums per row and 2048-entry slice, R the
    # rank rounded up to a power of two) to the forward workspace and to the
    # backward one (t recomputed from x); other widths add nothing
    M = 100
    extra = M * slices * (1 + R) * 4
    st, f = _fwd_ws(lib, _lin(K=K, N=256, r=r, fmt=Q.QLORA_W4G128), M=M)
    assert st == Q.QLORA_OK
    base = M * K + M * 4 + M * r * 4 + _w4_split_bytes(M, 256, K)
    assert base + extra <= f <= base + extra + 6 * 256
    b = _bwd_ws(lib, _lin(K=K, N=256, r=r), M, Q.QLORA_F32)
    b0 = 2 * M * r * 4 + ((M + 63) // 64) * r * (K + 256) * 4
    assert b0 + extra <= b <= b0 + extra + 7 * 256


@pytest.mark.parametrize("kw,M,dtype,want", [
    (dict(r=0), 64, Q.QLORA_BF16, Q.QLORA_EINVAL),
    (dict(r=33), 64, Q.QLORA_BF16, Q.QLORA_EINVAL),
    (dict(K=200), 64, Q.QLORA_BF16, Q.QLORA_EINVAL),
    (dict(N=8), 64, Q.QLORA_BF16, Q.QLORA_EINVAL),
    (dict(), 0, Q.QLORA_BF16, Q.QLORA_EINVAL),
    (dict(), 64, 7, Q.QLORA_EINVAL),
    (dict(fmt=5), 64, Q.QLORA_BF16, Q.QLORA_EINVAL),
    (dict(fmt=Q.QLORA_W4G128, K=192), 64, Q.QLORA_BF16, Q.QLORA_EINVAL),
    (dict(fmt=Q.QLORA_W4G128), 64, Q.QLORA_F32, Q.QLORA_EUNSUPPORTED),
    (dict(ptr=FAKE + 4), 64, Q.QLORA_BF16, Q.QLORA_EINVAL),
    (dict(ptr=None), 64, Q.QLORA_BF16, Q.QLORA_EINVAL),
    (dict(K=65536, N=65536), 64, Q.QLORA_BF16, Q.QLORA_ERANGE),
])
def test_layer_validation(lib, kw, M, dtype, want):
    st, _ = _fwd_ws(lib, _lin(**kw), M, dtype)
    assert st == want


def test_calls_fail_before_launch(lib):
    lin = _lin()
    st, need = _fwd_ws(lib, lin)
    # workspace too small
    assert lib.qlora_fwd(ctypes.byref(lin), 64, Q.QLORA_BF16, FAKE, FAKE, FAKE, FAKE,
                         need - 1, None) == Q.QLORA_EWORKSPACE
    # null / misaligned data pointers
    assert lib.qlora_fwd(ctypes.byref(lin), 64, Q.QLORA_BF16, None, FAKE, None, FAKE,
                         need, None) == Q.QLORA_EINVAL
    assert lib.qlora_fwd(ctypes.byref(lin), 64, Q.QLORA_BF16, FAKE + 2, FAKE, None, FAKE,
                         need, None) == Q.QLORA_EINVAL
    assert lib.qlora_bwd(ctypes.byref(lin), 64, Q.QLORA_BF16, FAKE, FAKE, None, None,
                         None, FAKE, FAKE, 1 << 30, None) == Q.QLORA_EINVAL
    n = ctypes.c_size_t()
    lib.qlora_bwd_workspace(ctypes.byref(lin), 64, Q.QLORA_BF16, ctypes.byref(n))
    assert lib.qlora_bwd(ctypes.byref(lin), 64, Q.QLORA_BF16, FAKE, FAKE, None, FAKE,
                         FAKE, FAKE, FAKE, n.value - 1, None) == Q.QLORA_EWORKSPACE
    assert lib.qlora_quantize(FAKE, 100, 64, Q.QLORA_W8, FAKE, FAKE, None) == Q.QLORA_EINVAL
    assert lib.qlora_quantize(None, 128, 64, Q.QLORA_W8, FAKE, FAKE, None) == Q.QLORA_EINVAL
    assert lib.qlora_quantize_rows(FAKE, 4, 24, Q.QLORA_BF16, FAKE, FAKE, None) == Q.QLORA_EINVAL
    assert lib.qlora_fwd_acc(ctypes.byref(_lin(fmt=Q.QLORA_W4G128)), 64, Q.QLORA_BF16,
                             FAKE, FAKE, FAKE, 1 << 30, None) == Q.QLORA_EUNSUPPORTED
    # merge: int8 only, outputs must not overlap the inputs
    assert lib.qlora_merge(ctypes.byref(_lin(fmt=Q.QLORA_W4G128)), FAKE + 4096, FAKE + 8192,
                           None) == Q.QLORA_EUNSUPPORTED
    assert lib.qlora_merge(ctypes.byref(lin), FAKE, FAKE + (1 << 20), None) == Q.QLORA_EINVAL
    assert lib.qlora_merge(ctypes.byref(lin), None, FAKE + (1 << 20), None) == Q.QLORA_EINVAL
    # the timed variants need at least one launch of the product kernel
    assert lib.qlora_fwd_timed(ctypes.byref(lin), 64, Q.QLORA_BF16, FAKE, FAKE, None, FAKE,
                               need, None, 0, None, None) == Q.QLORA_EINVAL
    assert lib.qlora_bwd_timed(ctypes.byref(lin), 64, Q.QLORA_BF16, FAKE, FAKE, None, FAKE,
                               FAKE, FAKE, FAKE, n.value, None, 0, None, None) == Q.QLORA_EINVAL
    # the integer 4-bit forward: 4-bit layers only
    assert lib.qlora_fwd_a8w4(ctypes.byref(lin), 64, Q.QLORA_BF16, FAKE, FAKE, None, FAKE,
                              need, None) == Q.QLORA_EUNSUPPORTED
    lin4 = _lin(fmt=Q.QLORA_W4G128)
    st4, need4 = _fwd_ws(lib, lin4)
    assert lib.qlora_fwd_a8w4(ctypes.byref(lin4), 64, Q.QLORA_BF16, FAKE, FAKE, None, FAKE,
                              need4 - 1, None) == Q.QLORA_EWORKSPACE
    assert lib.qlora_fwd_a8w4(ctypes.byref(lin4), 64, Q.QLORA_F32, FAKE, FAKE, None, FAKE,
                              need4, None) == Q.QLORA_EUNSUPPORTED
    assert lib.qlora_fwd_a8w4(ctypes.byref(lin4), 64, Q.QLORA_BF16, None, FAKE, None, FAKE,
                              need4, None) == Q.QLORA_EINVAL
    # multi-head layers: heads must divide N into multiples of 64
    for heads, want in [(-1, Q.QLORA_EINVAL), (3, Q.QLORA_EINVAL), (8, Q.QLORA_EUNSUPPORTED)]:
        lh = Q.qlora_linear(256, 256, 4, 8.0, Q.QLORA_W8, FAKE, FAKE, FAKE, FAKE, heads)
        assert lib.qlora_fwd(ctypes.byref(lh), 64, Q.QLORA_BF16, FAKE, FAKE, None, FAKE,
                             need, None) == want
    lh = Q.qlora_linear(256, 256, 4, 8.0, Q.QLORA_W8, FAKE, FAKE, FAKE, FAKE, 4)
    assert lib.qlora_fwd(ctypes.byref(lh), 64, Q.QLORA_BF16, FAKE, FAKE, None, FAKE,
                         need - 1, None) == Q.QLORA_EWORKSPACE      # valid layout, small ws
    assert lib.qlora_quantize_heads(FAKE, 3, 128, 256, Q.QLORA_W8, FAKE, FAKE, None) == Q.QLORA_EINVAL
    assert lib.qlora_quantize_heads(FAKE, 0, 128, 256, Q.QLORA_W8, FAKE, FAKE, None) == Q.QLORA_EINVAL
    assert lib.qlora_quantize_heads(FAKE, 8, 128, 256, Q.QLORA_W8, FAKE, FAKE, None) == Q.QLORA_EUNSUPPORTED
    # the two halves of the backward validate their own arguments
    assert lib.qlora_bwd_partial(ctypes.byref(lin), 64, Q.QLORA_BF16, None, FAKE, None, FAKE,
                                 FAKE, n.value, None) == Q.QLORA_EINVAL
    assert lib.qlora_bwd_partial(ctypes.byref(lin), 64, Q.QLORA_BF16, FAKE, FAKE, None, FAKE,
                                 FAKE, n.value - 1, None) == Q.QLORA_EWORKSPACE
    assert lib.qlora_bwd_finish(ctypes.byref(lin), 64, Q.QLORA_BF16, None, FAKE, FAKE,
                                n.value, None) == Q.QLORA_EINVAL
    assert lib.qlora_bwd_finish(ctypes.byref(lin), 64, Q.QLORA_BF16, FAKE, FAKE + 2, FAKE,
                                n.value, None) == Q.QLORA_EINVAL
    assert lib.qlora_bwd_finish(ctypes.byref(lin), 64, Q.QLORA_BF16, FAKE, FAKE, FAKE,
                                n.value - 1, None) == Q.QLORA_EWORKSPACE
    assert lib.qlora_bwd_finish(ctypes.byref(lin), 0, Q.QLORA_BF16, FAKE, FAKE, FAKE,
                                n.value, None) == Q.QLORA_EINVAL


@pytest.mark.parametrize("K,N", [(256, 256), (2048, 16384), (16384, 2048), (208, 80)])
def test_outlier_format_sizes(lib, K, N):
    # codes: one byte per weight; the side buffer holds the header, the
    # outlier list (rowptr [K + 1], col [cap], val [cap]) and more, with
    # cap = 2 floor(K N / 1000) + 2 (each tail of the nearest-rank cut holds
    # at most floor(K N / 1000) elements)
    cb, sb = Q.qlora_weight_bytes(K, N, "w8o")
    ro, co, vo, cap = Q.qlora_outlier_layout(K, N)
    assert cb == K * N
    assert cap == 2 * (K * N // 1000) + 2
    assert 16 <= ro and ro + 4 * (K + 1) <= co and co + 4 * cap <= vo
    assert vo + 2 * cap <= sb
    assert ro % 16 == 0 and co % 16 == 0 and vo % 16 == 0


def test_outlier_format_validation(lib):
    lo = _lin(fmt=Q.QLORA_W8O)
    st, need = _fwd_ws(lib, lo)
    assert st == Q.QLORA_OK
    st_w8, need_w8 = _fwd_ws(lib, _lin())
    assert need >= need_w8 + 64 * 4 - 256         # plus the row sums of xq
    assert _fwd_ws(lib, lo, 64, Q.QLORA_F32)[0] == Q.QLORA_EUNSUPPORTED
    assert _fwd_ws(lib, _lin(fmt=Q.QLORA_W8O, N=1 << 24, K=16))[0] == Q.QLORA_EUNSUPPORTED
    # one head only at quantization; merge and the 4-bit forward do not apply
    assert lib.qlora_quantize_heads(FAKE, 4, 128, 256, Q.QLORA_W8O, FAKE, FAKE,
                                    None) == Q.QLORA_EUNSUPPORTED
    assert lib.qlora_quantize(FAKE, 100, 64, Q.QLORA_W8O, FAKE, FAKE, None) == Q.QLORA_EINVAL
    assert lib.qlora_merge(ctypes.byref(lo), FAKE + 4096, FAKE + 8192,
                           None) == Q.QLORA_EUNSUPPORTED
    assert lib.qlora_fwd_a8w4(ctypes.byref(lo), 64, Q.QLORA_BF16, FAKE, FAKE, None, FAKE,
                              need, None) == Q.QLORA_EUNSUPPORTED
    with pytest.raises(Q.QloraError) as e:
        Q.qlora_outlier_layout(100, 64)
    assert e.value.status == Q.QLORA_EINVAL


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(Q, "_lib", None)
    monkeypatch.setattr(Q, "LIB_PATH", str(tmp_path / "absent.so"))
    with pytest.raises(RuntimeError, match="missing"):
        Q.lib()


def test_finish_batch_fails_before_launch(lib):
    # every item is validated before anything is enqueued: an error in the
    # last item launches nothing for the first ones (no GPU is needed here)
    lin, bad = _lin(), _lin(r=0)
    n = ctypes.c_size_t()
    lib.qlora_bwd_workspace(ctypes.byref(lin), 64, Q.QLORA_BF16, ctypes.byref(n))

    def items(*specs):
        arr = (Q.qlora_finish_item * len(specs))()
        for i, (L, ws_bytes, dA) in enumerate(specs):
            arr[i] = Q.qlora_finish_item(ctypes.cast(ctypes.pointer(L), ctypes.c_void_p), 64,
                                         Q.QLORA_BF16, dA, FAKE, FAKE, ws_bytes)
        return arr

    good = (lin, n.value, FAKE)
    assert lib.qlora_bwd_finish_batch(None, 1, None) == Q.QLORA_EINVAL
    assert lib.qlora_bwd_finish_batch(items(good), 0, None) == Q.QLORA_EINVAL
    assert lib.qlora_bwd_finish_batch(items(good, (lin, n.value - 1, FAKE)), 2,
                                      None) == Q.QLORA_EWORKSPACE
    assert lib.qlora_bwd_finish_batch(items(good, good, (bad, n.value, FAKE)), 3,
                                      None) == Q.QLORA_EINVAL
    assert lib.qlora_bwd_finish_batch(items(good, (lin, n.value, FAKE + 4)), 2,
                                      None) == Q.QLORA_EINVAL
    assert lib.qlora_bwd_finish_batch(items(good, (lin, n.value, None)), 2,
                                      None) == Q.QLORA_EINVAL


def test_partials_bytes(lib):
    # the partial sums of dB and dA lead the backward workspace: one per block
    # of 64 rows, [r, N] and [r, K] float32, each rounded up to 256 bytes
    n = ctypes.c_size_t()
    for K, N, r, M in ((256, 256, 4, 64), (1024, 784, 8, 1000), (2048, 16384, 8, 512)):
        lin = _lin(K=K, N=N, r=r)
        assert lib.qlora_bwd_partials_bytes(ctypes.byref(lin), M, Q.QLORA_F32,
                                            ctypes.byref(n)) == Q.QLORA_OK
        up = lambda b: (b + 255) // 256 * 256
        blocks = (M + 63) // 64
        assert n.value == up(blocks * r * N * 4) + up(blocks * r * K * 4)
        assert n.value < _bwd_ws(lib, lin, M, Q.QLORA_F32)
    assert lib.qlora_bwd_partials_bytes(ctypes.byref(_lin(r=0)), 64, Q.QLORA_F32,
                                        ctypes.byref(n)) == Q.QLORA_EINVAL
    assert lib.qlora_bwd_partials_bytes(ctypes.byref(_lin()), 64, Q.QLORA_F32,
                                        None) == Q.QLORA_EINVAL


def test_noalloc_backward_validates_before_any_launch(lib):
    """qlora_bwd_noalloc checks its arguments and the static scratch's size
    on the host, before touching the GPU."""
    call = lambda L, M: lib.qlora_bwd_noalloc(ctypes.byref(L), M, Q.QLORA_BF16, FAKE, FAKE,  # noqa: E731
                                              None, FAKE, FAKE, FAKE, None)
    assert call(_lin(K=100), 64) == Q.QLORA_EINVAL                 # K % 16 != 0
    assert call(_lin(K=2048, N=16384, r=8), 512) == Q.QLORA_EWORKSPACE   # 37 MiB of scratch
    L = _lin(K=2048, N=16384, r=8)
    need = ctypes.c_size_t()
    assert lib.qlora_bwd_workspace(ctypes.byref(L), 512, Q.QLORA_BF16, ctypes.byref(need)) == 0
    assert need.value > Q.QLORA_NOALLOC_SCRATCH_BYTES
