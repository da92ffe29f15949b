"""The C-ABI library loads, exports what include/gemm.h declares, and rejects
bad arguments before any HIP call (CPU only: no compute call is made)."""
import ctypes
import os
import re

import pytest

from fp32_gemm_07_amd import binding, build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gemm.h")


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not os.path.exists(build.LIB_PATH):
        build.build()
    return binding.load()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gemm_\w+)\s*\(", text)))


def test_header_declarations_are_all_exported():
    declared = _declared_functions()
    assert set(declared) == set(binding.EXPORTS)
    lib = ctypes.CDLL(build.LIB_PATH)
    for name in declared:
        assert hasattr(lib, name), name


VP = ctypes.c_void_p


def _st(*args):
    return binding.raw_status("gemm_f32", *args)


def test_negative_dims_rejected():
    a = VP(0x10000)
    assert _st(a, a, VP(0x90000000), -1, 4, 4, None) == binding.GEMM_ERR_INVALID_DIM
    assert _st(a, a, VP(0x90000000), 4, -1, 4, None) == binding.GEMM_ERR_INVALID_DIM
    assert _st(a, a, VP(0x90000000), 4, 4, -1, None) == binding.GEMM_ERR_INVALID_DIM


def test_null_pointers_rejected():
    p = VP(0x7f0000000000)
    q = VP(0x7f1000000000)
    r = VP(0x7f2000000000)
    assert _st(None, q, r, 4, 4, 4, None) == binding.GEMM_ERR_NULL_PTR
    assert _st(p, None, r, 4, 4, 4, None) == binding.GEMM_ERR_NULL_PTR
    assert _st(p, q, None, 4, 4, 4, None) == binding.GEMM_ERR_NULL_PTR


def test_empty_extents_need_no_pointers():
    # M = 0 or N = 0: nothing to do, no pointer needed, no HIP call made
    assert _st(None, None, None, 0, 5, 7, None) == binding.GEMM_OK
    assert _st(None, None, None, 5, 0, 7, None) == binding.GEMM_OK
    # K = 0: A and B are not read, C is (zero-filled)
    assert _st(None, None, None, 5, 3, 0, None) == binding.GEMM_ERR_NULL_PTR


def test_c_overlapping_a_or_b_rejected():
    base = 0x7f0000000000
    A = VP(base)
    B = VP(base + 0x100000)
    assert _st(A, B, VP(base + 16), 4, 4, 4, None) == binding.GEMM_ERR_ALIAS
    assert _st(A, B, VP(base + 0x100000 - 8), 4, 4, 4, None) == binding.GEMM_ERR_ALIAS
    # A and B may overlap each other
    st = binding.raw_status("gemm_f32_ex", A, A, VP(base + 0x200000), 4, 4, 4, None, 0, None)
    assert st != binding.GEMM_ERR_ALIAS


def test_workspace_too_small_rejected():
    M, N, K = 512, 512, 131072
    need = binding.gemm_f32_workspace_bytes(M, N, K)
    assert need == 4 * binding.gemm_f32_plan(M, N, K).split_k * M * N > 0
    A, B, C = VP(0x7f0000000000), VP(0x7f1000000000), VP(0x7f2000000000)
    st = binding.raw_status("gemm_f32_ex", A, B, C, M, N, K, None, 0, None)
    assert st == binding.GEMM_ERR_WORKSPACE
    st = binding.raw_status("gemm_f32_ex", A, B, C, M, N, K, VP(0x7f3000000000), need - 4, None)
    assert st == binding.GEMM_ERR_WORKSPACE


def test_invalid_plans_rejected():
    A, B, C = VP(0x7f0000000000), VP(0x7f1000000000), VP(0x7f2000000000)
    for plan in (binding.make_plan(99, 1), binding.make_plan(binding.GEMM_KERNEL_MFMA_64x64, 0)):
        st = binding.raw_status("gemm_f32_with_plan", A, B, C, 8, 8, 8, ctypes.byref(plan), None, 0,
                                None)
        assert st == binding.GEMM_ERR_INVALID_PLAN
    assert binding.raw_status("gemm_f32_with_plan", A, B, C, 8, 8, 8, None, None, 0, None) == \
        binding.GEMM_ERR_INVALID_PLAN


def test_plan_with_more_workgroups_than_an_int_rejected():
    """16 x 16 tiles of a 2^20 x 2^20 output: 2^32 workgroups, more than the
    device-side ids can count (rejected before any HIP call)."""
    M = N = 1 << 20
    plan = binding.make_plan(binding.GEMM_KERNEL_LADDER_V0, 1)
    assert binding.gemm_f32_plan_workspace_bytes(M, N, 16, plan) == 0
    A, B, C = VP(0x7f0000000000), VP(0x7f1000000000), VP(0x7f2000000000)
    st = binding.raw_status("gemm_f32_with_plan", A, B, C, M, N, 16, ctypes.byref(plan), None, 0,
                            None)
    assert st == binding.GEMM_ERR_INVALID_PLAN


def test_planner_choices_for_standing_workloads():
    p4 = binding.gemm_f32_plan(4096, 4096, 4096)
    assert p4.kernel == binding.GEMM_KERNEL_DMA32_256x256_W8_S3 and p4.split_k == 1
    p5 = binding.gemm_f32_plan(512, 512, 131072)
    assert p5.split_k > 1 and p5.k_chunk * p5.split_k >= 131072
    assert p5.k_chunk % 16 == 0
    # few output tiles and a long K: small tiles, K split
    p = binding.gemm_f32_plan(1024, 1024, 4096)
    assert p.kernel == binding.GEMM_KERNEL_DMA32_64x64_S3
    p = binding.gemm_f32_plan(256, 256, 8192)
    assert p.kernel == binding.GEMM_KERNEL_DMA32_64x64_S3 and p.split_k > 1
    # 24 x 24 tiles of 256 would leave a third round 25% full: 128x128 tiles
    p = binding.gemm_f32_plan(6144, 6144, 6144)
    assert p.kernel == binding.GEMM_KERNEL_DMA32_128x128_W8_S3 and p.split_k == 1
    # one GPU's share of a sharded 4096^3: 512 tiles of 64 x 64, two per CU at
    # once, against 128 tiles of 128 x 128 split in two; the pairs of 64 x 64
    # workgroups keep two waves per SIMD (measured 124.0 against 126.3 us)
    for (M, N, K) in [(512, 4096, 4096), (1024, 2048, 4096)]:
        p = binding.gemm_f32_plan(M, N, K)
        assert p.kernel == binding.GEMM_KERNEL_DMA32_64x64_S3 and p.split_k == 1
    # short K over a large C is bound by the store of C: the 4-wave 128 x 128
    # kernel (two workgroups per CU, one's store under the other's copies);
    # from K ~ 128 (4096^2) on the 256 x 256 kernel again (measured both ways)
    for (M, N, K) in [(8192, 8192, 16), (4096, 4096, 16), (16384, 4096, 16), (8192, 8192, 128)]:
        assert binding.gemm_f32_plan(M, N, K).kernel == binding.GEMM_KERNEL_DMA32_128x128_W4
    for (M, N, K) in [(4096, 4096, 256), (8192, 8192, 256), (4001, 3999, 301)]:
        assert binding.gemm_f32_plan(M, N, K).kernel == binding.GEMM_KERNEL_DMA32_256x256_W8_S3
    # 96 x 96 tiles where they fill the CUs (1536^2: one round), from K = 64
    # on; below that the fill of their stages costs more than it saves
    # (2048 x 16 x 2048: 10.1 against 9.0 us for 128 x 128 tiles)
    for K in (64, 128, 1536):
        assert binding.gemm_f32_plan(1536, 1536, K).kernel == binding.GEMM_KERNEL_DMA16_96x96_S3
    for (M, N, K) in [(2048, 2048, 16), (1024, 1024, 16), (1536, 1536, 32)]:
        assert binding.gemm_f32_plan(M, N, K).kernel != binding.GEMM_KERNEL_DMA16_96x96_S3
    for (M, N, K) in [(128, 112, 96), (1024, 1024, 512), (1001, 777, 513), (1, 1, 1)]:
        p = binding.gemm_f32_plan(M, N, K)
        assert p.split_k >= 1 and p.k_chunk * p.split_k >= K
        assert binding.gemm_kernel_name(p.kernel) != "unknown"


def test_split_tail_plans():
    """Split tail: the planner's plans where 18 x 16 tiles of 64 x 64 leave a
    last round of 32 (1100 x 777 x 1000, split in two) and where 19 x 19 tiles
    of 96 x 96 leave one of 105 (1792^3, split in two: 210 pieces); none where
    16 x 16 tiles of 96 x 96 make exactly one round (1536^3); workspace sizes
    for whole rounds, a partial round and fewer tiles than one round; plans
    the library must reject."""
    p = binding.gemm_f32_plan(1100, 1000, 777)
    assert p.kernel == binding.GEMM_KERNEL_DMA32_64x64_S3
    assert p.split_tail == 1 and p.split_k == 2 and p.k_chunk == 400
    assert binding.gemm_f32_workspace_bytes(1100, 1000, 777) == 4 * 2 * 1100 * 1000
    p = binding.gemm_f32_plan(1792, 1792, 1792)
    assert p.kernel == binding.GEMM_KERNEL_DMA16_96x96_S3
    assert p.split_tail == 1 and p.split_k == 2 and p.k_chunk == 896
    p = binding.gemm_f32_plan(1536, 1536, 1536)
    assert p.kernel == binding.GEMM_KERNEL_DMA16_96x96_S3 and p.split_k == 1
    assert binding.gemm_f32_workspace_bytes(1536, 1536, 1536) == 0
    tail = binding.make_plan(binding.GEMM_KERNEL_DMA32_64x64_S3, 4, True)
    # 16 x 16 = 256 tiles: one whole round, nothing split
    assert binding.gemm_f32_plan_workspace_bytes(1024, 1024, 1024, tail) == 0
    # 17 x 16 tiles: one tile row past a whole round
    assert binding.gemm_f32_plan_workspace_bytes(1088, 1024, 1024, tail) == 4 * 4 * 1088 * 1024
    # 8 x 8 tiles: fewer than a round, every tile split
    assert binding.gemm_f32_plan_workspace_bytes(512, 512, 1024, tail) == 4 * 4 * 512 * 512
    A, B, C = VP(0x7f0000000000), VP(0x7f1000000000), VP(0x7f2000000000)
    bad = (binding.make_plan(binding.GEMM_KERNEL_MFMA_64x64, 2, True),
           binding.make_plan(binding.GEMM_KERNEL_VALU_64x64, 1, True),
           binding.gemm_plan_t(binding.GEMM_KERNEL_DMA32_64x64_S3, 2, 0, 2),
           binding.gemm_plan_t(binding.GEMM_KERNEL_DMA32_64x64_S3, 2, 0, -1))
    for plan in bad:
        st = binding.raw_status("gemm_f32_with_plan", A, B, C, 1536, 1536, 1536,
                                ctypes.byref(plan), None, 0, None)
        assert st == binding.GEMM_ERR_INVALID_PLAN, plan
        assert binding.gemm_f32_plan_workspace_bytes(1536, 1536, 1536, plan) == 0


def test_explicit_split_is_clamped_to_k_steps():
    plan = binding.make_plan(binding.GEMM_KERNEL_MFMA_64x64, 1000)
    # 40 K elements = 3 K steps of 16: at most 3 ranges
    assert binding.gemm_f32_plan_workspace_bytes(8, 8, 40, plan) == 4 * 3 * 8 * 8
    assert binding.gemm_f32_plan_workspace_bytes(8, 8, 40, binding.make_plan(4, 1)) == 0


def test_status_strings_and_names():
    for s in range(0, 8):
        assert binding.gemm_status_string(s) != "unknown status"
    assert binding.gemm_status_string(1234) == "unknown status"
    for name, k in binding.KERNELS.items():
        assert binding.gemm_kernel_name(k) not in ("unknown", "auto")
    assert binding.gemm_kernel_name(0) == "auto"
    assert isinstance(binding.gemm_last_hip_error(), int)


# ---------------------------------------------------------------------------
# gemm_f32_general: argument checks (all before any HIP call).

def _gst(ta, tb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, ws=None, wsb=0):
    f = ctypes.c_float
    return binding.raw_status("gemm_f32_general", ta, tb, M, N, K, f(alpha), A, lda, B, ldb,
                              f(beta), C, ldc, ws, wsb, None)


def test_general_leading_dimensions_checked():
    A, B, C = VP(0x7f0000000000), VP(0x7f1000000000), VP(0x7f2000000000)
    E = binding.GEMM_ERR_INVALID_DIM
    assert _gst(0, 0, 4, 5, 6, 1, A, 5, B, 5, 0, C, 5) == E        # lda < K
    assert _gst(1, 0, 4, 5, 6, 1, A, 3, B, 5, 0, C, 5) == E        # transposed A: lda < M
    assert _gst(0, 0, 4, 5, 6, 1, A, 6, B, 4, 0, C, 5) == E        # ldb < N
    assert _gst(0, 1, 4, 5, 6, 1, A, 6, B, 5, 0, C, 5) == E        # transposed B: ldb < K
    assert _gst(0, 0, 4, 5, 6, 1, A, 6, B, 5, 0, C, 4) == E        # ldc < N
    assert _gst(0, 0, -1, 5, 6, 1, A, 6, B, 5, 0, C, 5) == E
    # a 64-row tile of a K-contiguous A would span 2^31 bytes: rejected
    assert _gst(0, 0, 64, 64, 16, 1, A, 1 << 23, B, 64, 0, C, 64) == E


def test_general_pointer_rules():
    A, B, C = VP(0x7f0000000000), VP(0x7f1000000000), VP(0x7f2000000000)
    assert _gst(0, 0, 4, 5, 6, 1, None, 6, B, 5, 0, C, 5) == binding.GEMM_ERR_NULL_PTR
    assert _gst(0, 0, 4, 5, 6, 1, A, 6, None, 5, 0, C, 5) == binding.GEMM_ERR_NULL_PTR
    assert _gst(0, 0, 4, 5, 6, 1, A, 6, B, 5, 0, None, 5) == binding.GEMM_ERR_NULL_PTR
    # nothing to produce: no pointer needed
    assert _gst(0, 0, 0, 5, 6, 1, None, 6, None, 5, 0, None, 5) == binding.GEMM_OK
    # C's extent (with its stride) overlapping A's
    base = 0x7f0000000000
    st = _gst(0, 0, 4, 4, 4, 1, VP(base), 4, B, 4, 0, VP(base + 4 * 4 * 3), 8)
    assert st == binding.GEMM_ERR_ALIAS


def test_general_workspace_checked():
    M, N, K = 256, 256, 8192
    need = binding.gemm_f32_general_workspace_bytes(0, 0, M, N, K, K, N)
    assert need > 0 and need == binding.gemm_f32_workspace_bytes(M, N, K)
    A, B, C = VP(0x7f0000000000), VP(0x7f1000000000), VP(0x7f2000000000)
    st = _gst(0, 0, M, N, K, 1, A, K, B, N, 0, C, N, VP(0x7f3000000000), need - 4)
    assert st == binding.GEMM_ERR_WORKSPACE
    # transposed operands and strides: workspace is still 4 * S * M * N
    need_t = binding.gemm_f32_general_workspace_bytes(1, 1, M, N, K, M + 3, K + 5)
    assert need_t % (4 * M * N) == 0
    assert binding.gemm_f32_general_workspace_bytes(0, 0, M, N, K, K - 1, N) == 0   # bad lda


def test_binding_kernel_ids_mirror_the_header():
    """Every GEMM_KERNEL_* enumerator of include/gemm.h has the same value in
    the binding, every one but AUTO is in the binding's kernel table, and the
    library names each kernel distinctly."""
    text = open(os.path.join(ROOT, "include", "gemm.h")).read()
    header = {m.group(1): int(m.group(2))
              for m in re.finditer(r"\b(GEMM_KERNEL_\w+)\s*=\s*(\d+)", text)}
    assert len(header) > 20
    for name, value in header.items():
        assert getattr(binding, name) == value, name
    assert sorted(binding.KERNELS.values()) == sorted(v for n, v in header.items()
                                                      if n != "GEMM_KERNEL_AUTO")
    names = [binding.gemm_kernel_name(k) for k in binding.KERNELS.values()]
    assert len(set(names)) == len(names)


def test_plans_follow_the_compute_unit_count():
    """The planner costs rounds of one tile per compute unit. Without a device
    (this host) gemm_f32_plan plans for 256; a device with another count gets
    plans made for its own rounds."""
    for (M, N, K) in [(1536, 1536, 1536), (4096, 4096, 4096), (512, 512, 131072),
                      (1001, 777, 513), (3000, 3000, 3000)]:
        a, b = binding.gemm_f32_plan(M, N, K), binding.gemm_f32_plan_cus(M, N, K, 256)
        assert (a.kernel, a.split_k, a.k_chunk, a.split_tail) == \
            (b.kernel, b.split_k, b.k_chunk, b.split_tail)
    # 288 tiles of 64 x 64: a round + 32 tiles at 256 CUs (split tail),
    # exactly one round at 288 (nothing split)
    p = binding.gemm_f32_plan_cus(1100, 1000, 777, 256)
    assert p.kernel == binding.GEMM_KERNEL_DMA32_64x64_S3 and p.split_tail == 1 and p.split_k == 2
    p = binding.gemm_f32_plan_cus(1100, 1000, 777, 288)
    assert p.kernel == binding.GEMM_KERNEL_DMA32_64x64_S3 and p.split_tail == 0 and p.split_k == 1
    # 1536^3: 256 tiles of 96 x 96, one round at 256 CUs; at 192 a third of
    # them would make a second round, while 576 tiles of 64 x 64 make exactly
    # three
    p = binding.gemm_f32_plan_cus(1536, 1536, 1536, 256)
    assert p.kernel == binding.GEMM_KERNEL_DMA16_96x96_S3 and p.split_k == 1
    p = binding.gemm_f32_plan_cus(1536, 1536, 1536, 192)
    assert p.kernel == binding.GEMM_KERNEL_DMA32_64x64_S3 and p.split_tail == 0 and p.split_k == 1
    # 256 tiles of 256 x 256: one round at 256 CUs, two whole rounds at 128
    for cus in (256, 128):
        p = binding.gemm_f32_plan_cus(4096, 4096, 4096, cus)
        assert p.kernel == binding.GEMM_KERNEL_DMA32_256x256_W8_S3 and p.split_k == 1
    # the long-K product splits K to fill the CUs: fewer CUs, fewer ranges
    assert binding.gemm_f32_plan_cus(512, 512, 131072, 32).split_k < \
        binding.gemm_f32_plan_cus(512, 512, 131072, 256).split_k
    plan = binding.gemm_plan_t()
    assert binding.raw_status("gemm_f32_plan_cus", 64, 64, 64, 0, ctypes.byref(plan)) == \
        binding.GEMM_ERR_INVALID_DIM
    assert binding.raw_status("gemm_f32_plan_cus", 64, 64, 64, 8, None) == binding.GEMM_ERR_NULL_PTR


def test_capturing_status_has_its_own_text():
    text = binding.gemm_status_string(binding.GEMM_ERR_CAPTURING)
    assert "capturing" in text and text != binding.gemm_status_string(99)


REMARKS = """\
gemm_kernels.hpp:191:1: remark: Function Name: _ZN4gemm1aEv [-Rpass-analysis=kernel-resource-usage]
gemm_kernels.hpp:191:1: remark:     VGPRs: 256 [-Rpass-analysis=kernel-resource-usage]
gemm_kernels.hpp:191:1: remark:     AGPRs: 0 [-Rpass-analysis=kernel-resource-usage]
gemm_kernels.hpp:191:1: remark:     ScratchSize [bytes/lane]: 40 [-Rpass-analysis=kernel-resource-usage]
gemm_kernels.hpp:191:1: remark:     SGPRs Spill: 0 [-Rpass-analysis=kernel-resource-usage]
gemm_kernels.hpp:191:1: remark:     VGPRs Spill: 9 [-Rpass-analysis=kernel-resource-usage]
  191 | void a() {
gemm_kernels.hpp:200:1: remark: Function Name: _ZN4gemm1bEv [-Rpass-analysis=kernel-resource-usage]
gemm_kernels.hpp:200:1: remark:     VGPRs: 208 [-Rpass-analysis=kernel-resource-usage]
gemm_kernels.hpp:200:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]
gemm_kernels.hpp:200:1: remark:     SGPRs Spill: 33 [-Rpass-analysis=kernel-resource-usage]
gemm_kernels.hpp:200:1: remark:     VGPRs Spill: 0 [-Rpass-analysis=kernel-resource-usage]
gemm_kernels.hpp:210:1: remark: Function Name: _ZN4gemm1cEv [-Rpass-analysis=kernel-resource-usage]
gemm_kernels.hpp:210:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]
gemm_kernels.hpp:210:1: remark:     VGPRs Spill: 0 [-Rpass-analysis=kernel-resource-usage]
"""


def test_build_refuses_kernels_that_use_scratch_memory():
    """The build reads the compiler's per-kernel resource report: a kernel with
    scratch memory or spilled VGPRs fails it; SGPRs spilled into VGPR lanes
    (no memory) do not."""
    res = build.kernel_resources(REMARKS)
    assert set(res) == {"_ZN4gemm1aEv", "_ZN4gemm1bEv", "_ZN4gemm1cEv"}
    assert res["_ZN4gemm1aEv"]["ScratchSize [bytes/lane]"] == 40
    assert res["_ZN4gemm1bEv"]["SGPRs Spill"] == 33
    assert set(build.spilling_kernels(res)) == {"_ZN4gemm1aEv"}
    assert build.RESOURCE_REMARKS in build.build.__code__.co_consts or \
        "RESOURCE_REMARKS" in build.build.__code__.co_names
