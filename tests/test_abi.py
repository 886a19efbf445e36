"""CPU-side checks of the C ABI: the library loads, exports every declared
symbol, and rejects bad arguments before touching HIP (no GPU needed)."""
import ctypes as C
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "poetx.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(poetx_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def B():
    from orthogonal_equivalence_poet_amd import binding
    if not os.path.exists(binding.LIB_PATH):
        from orthogonal_equivalence_poet_amd import build
        build.build(verbose=False)
    binding.load()
    return binding


def test_every_declared_symbol_is_exported(B):
    names = _declared()
    assert len(names) >= 20
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (poetx_\w+)", out))
    assert set(names) <= exported, set(names) - exported
    assert set(B.EXPORTS) == set(names)
    lib = B.load()
    for n in names:
        getattr(lib, n)


def test_version_and_status_strings(B):
    assert "gfx950" in B.poetx_version()
    lib = B.load()
    assert lib.poetx_status_string(0) == b"ok"
    assert lib.poetx_status_string(4) == b"workspace too small"
    assert lib.poetx_status_string(99) == b"unknown status"


def _d(B, **kw):
    base = dict(T=32, m=64, n=64, b=16, k=3, dtype=B.POETX_F32, variant=B.POETX_FAST)
    base.update(kw)
    return B.desc(**base)


FAKE = 0x1000  # never dereferenced: validation fails before any HIP call


@pytest.mark.parametrize("kw,status", [
    (dict(b=24), 3), (dict(b=8), 3), (dict(b=2048), 3), (dict(b=0), 2),
    (dict(m=72), 2), (dict(n=40), 2), (dict(T=-1), 2),
    (dict(k=0), 3), (dict(k=9), 3), (dict(dtype=7), 1), (dict(variant=5), 1),
])
def test_linear_fwd_rejects_bad_desc(B, kw, status):
    lib = B.load()
    d = _d(B, **kw)
    st = lib.poetx_linear_fwd(C.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, None)
    assert st == status
    assert lib.poetx_linear_fwd_workspace_bytes(C.byref(d)) == 0


def test_null_pointers_and_small_workspace(B):
    lib = B.load()
    d = _d(B)
    need = lib.poetx_linear_fwd_workspace_bytes(C.byref(d))
    assert need > 0
    assert lib.poetx_linear_fwd(C.byref(d), None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need, None) == 1
    # fast needs the saved buffer
    assert lib.poetx_linear_fwd(C.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, need, None) == 1
    assert lib.poetx_linear_fwd(C.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need - 1,
                                None) == 4
    nb = lib.poetx_linear_bwd_workspace_bytes(C.byref(d))
    assert lib.poetx_linear_bwd(C.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE,
                                FAKE, nb, None) == 1
    assert lib.poetx_linear_bwd(C.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                FAKE, nb - 1, None) == 4
    assert lib.poetx_linear_fwd(None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need, None) == 1


def test_misaligned_pointers_are_rejected(B):
    """A contiguous view at an odd element offset is an argument error in the
    layer and group calls (their kernels use 16-byte vector and direct-to-LDS
    accesses), reported before any HIP call."""
    lib = B.load()
    d = _d(B, dtype=B.POETX_BF16)
    nf = lib.poetx_linear_fwd_workspace_bytes(C.byref(d))
    nb = lib.poetx_linear_bwd_workspace_bytes(C.byref(d))
    odd = FAKE + 2   # one bf16 element past an aligned address
    for i in range(9):
        args = [FAKE] * 9
        args[i] = odd
        assert lib.poetx_linear_fwd(C.byref(d), *args, nf, None) == B.POETX_ERR_INVALID_ARG, i
    for i in range(12):
        args = [FAKE] * 12
        args[i] = odd
        assert lib.poetx_linear_bwd(C.byref(d), *args, nb, None) == B.POETX_ERR_INVALID_ARG, i
    g = B.group_desc(32, 64, 16, 3, B.POETX_BF16, B.POETX_FAST, [64, 32])
    gf = lib.poetx_group_fwd_workspace_bytes(C.byref(g))
    gb = lib.poetx_group_bwd_workspace_bytes(C.byref(g))
    for i in range(9):
        args = [FAKE] * 9
        args[i] = odd
        assert lib.poetx_group_fwd(C.byref(g), *args, gf, None) == B.POETX_ERR_INVALID_ARG, i
    for i in range(12):
        args = [FAKE] * 12
        args[i] = odd
        assert lib.poetx_group_bwd(C.byref(g), *args, gb, None) == B.POETX_ERR_INVALID_ARG, i


def test_dense_fold_r_validation(B):
    """The folded dense + R-side product takes bf16 chains with b = 256 only and
    checks shapes and pointers before any HIP call."""
    lib = B.load()
    bf, f32 = B.POETX_BF16, B.POETX_F32
    ok = (2048, 4096, 4096, 256)
    args = [FAKE] * 5 + [None]
    assert lib.poetx_dense_fold_r(f32, *ok, *args) == B.POETX_ERR_UNSUPPORTED
    assert lib.poetx_dense_fold_r(bf, 2048, 4096, 4096, 128, *args) == B.POETX_ERR_UNSUPPORTED
    assert lib.poetx_dense_fold_r(bf, 2048, 4096, 4096, 512, *args) == B.POETX_ERR_UNSUPPORTED
    assert lib.poetx_dense_fold_r(bf, 2048, 4096 + 256, 4096 + 8, 256, *args) == B.POETX_ERR_SHAPE
    assert lib.poetx_dense_fold_r(bf, -1, 4096, 4096, 256, *args) == B.POETX_ERR_SHAPE
    assert lib.poetx_dense_fold_r(bf, 0, 4096, 4096, 256, *args) == B.POETX_OK
    assert lib.poetx_dense_fold_r(7, *ok, *args) == B.POETX_ERR_INVALID_ARG
    for i in range(5):
        a = [FAKE] * 5 + [None]
        a[i] = FAKE + 2
        assert lib.poetx_dense_fold_r(bf, *ok, *a) == B.POETX_ERR_INVALID_ARG, i
    for i in (0, 1, 2, 4):
        a = [FAKE] * 5 + [None]
        a[i] = None
        assert lib.poetx_dense_fold_r(bf, *ok, *a) == B.POETX_ERR_INVALID_ARG, i


def test_noalloc_forward_validation(B):
    """The forward without a workspace refuses a descriptor whose workspace
    exceeds its scratch array, and bad arguments, before any HIP call."""
    lib = B.load()
    big = B.desc(8192, 14336, 4096, 512, 4, B.POETX_BF16, B.POETX_MEM)
    assert lib.poetx_linear_fwd_workspace_bytes(C.byref(big)) > B.POETX_NOALLOC_SCRATCH_BYTES
    assert lib.poetx_linear_fwd_noalloc(C.byref(big), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None,
                                        None) == B.POETX_ERR_WORKSPACE
    d = _d(B)
    assert lib.poetx_linear_fwd_noalloc(C.byref(d), None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                        None) == B.POETX_ERR_INVALID_ARG
    assert lib.poetx_linear_fwd_noalloc(C.byref(d), FAKE + 2, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                        None) == B.POETX_ERR_INVALID_ARG
    assert lib.poetx_linear_fwd_noalloc(C.byref(_d(B, b=24)), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                        None) == B.POETX_ERR_UNSUPPORTED
    # an empty batch returns before anything else
    assert lib.poetx_linear_fwd_noalloc(C.byref(_d(B, T=0)), None, None, None, None, None, None, None, None,
                                        None) == B.POETX_OK


def test_empty_batch_forward_is_a_no_op(B):
    lib = B.load()
    d = _d(B, T=0)
    # returns before any HIP call: nothing to compute
    assert lib.poetx_linear_fwd(C.byref(d), None, None, None, None, None, None, None, None, None, 0, None) == 0


def test_comparison_variant_sizes_and_merge_rejection(B):
    lib = B.load()
    T, m, n, b = 2048, 4096, 1024, 256
    fast = B.desc(T, m, n, b, 3, B.POETX_BF16, B.POETX_FAST)
    four = B.desc(T, m, n, b, 3, B.POETX_BF16, B.POETX_FOUR_PERM)
    wc = B.desc(T, m, n, b, 3, B.POETX_BF16, B.POETX_WEIGHT_CENTRIC)
    # four_perm keeps the same two activations as fast
    assert lib.poetx_linear_saved_bytes(C.byref(four)) == lib.poetx_linear_saved_bytes(C.byref(fast))
    assert lib.poetx_linear_fwd_workspace_bytes(C.byref(four)) == lib.poetx_linear_fwd_workspace_bytes(C.byref(fast))
    # weight-centric keeps dense R, W0 P and W_RP; its backward needs dW_RP, R^T dW_RP, dR and dP
    assert lib.poetx_linear_saved_bytes(C.byref(wc)) == 2 * (m * m + 2 * m * n)
    assert lib.poetx_linear_bwd_workspace_bytes(C.byref(wc)) == 2 * 2 * m * n + 4 * m * m + 4 * n * n
    assert lib.poetx_linear_fwd_workspace_bytes(C.byref(wc)) >= 2 * n * n + 4 * (m + n)
    # the five variant values are accepted, a sixth is not
    assert lib.poetx_linear_saved_bytes(C.byref(B.desc(T, m, n, b, 3, B.POETX_BF16, 5))) == 0
    assert lib.poetx_linear_fwd(C.byref(B.desc(T, m, n, b, 3, B.POETX_BF16, 5)), FAKE, FAKE, FAKE, FAKE, FAKE,
                                FAKE, FAKE, FAKE, FAKE, 1 << 30, None) == B.POETX_ERR_INVALID_ARG
    # saved is required by every variant but mem
    for d in (four, wc):
        need = lib.poetx_linear_fwd_workspace_bytes(C.byref(d))
        assert lib.poetx_linear_fwd(C.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, need,
                                    None) == B.POETX_ERR_INVALID_ARG
        # merge folds into the pre-permuted weight, which these variants do not keep
        assert lib.poetx_merge_workspace_bytes(C.byref(d)) == 0
        assert lib.poetx_merge(C.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30,
                               None) == B.POETX_ERR_UNSUPPORTED


def test_group_desc_layout_sizes_and_validation(B):
    lib = B.load()
    assert C.sizeof(B.GroupDesc) == 3 * 8 + 6 * 4 + 8 * 8
    T, n, b = 2048, 4096, 256
    ms = [4096, 1024, 1024]
    g = B.group_desc(T, n, b, 3, B.POETX_BF16, B.POETX_FAST, ms)
    # FAST keeps the dense outputs [T, sum m] and the gathered inputs [T, count n]
    assert lib.poetx_group_saved_bytes(C.byref(g)) == 2 * T * sum(ms) + 2 * T * 3 * n
    # the same buffers as one chain of that width, plus two index tables
    chain = B.desc(T, sum(ms), 3 * n, b, 3, B.POETX_BF16, B.POETX_FAST)
    assert lib.poetx_group_fwd_workspace_bytes(C.byref(g)) >= lib.poetx_linear_fwd_workspace_bytes(C.byref(chain))
    assert lib.poetx_group_bwd_workspace_bytes(C.byref(g)) >= lib.poetx_linear_bwd_workspace_bytes(C.byref(chain))
    mem = B.group_desc(T, n, b, 3, B.POETX_BF16, B.POETX_MEM, ms)
    assert lib.poetx_group_saved_bytes(C.byref(mem)) == 0

    def fwd(gd, ws_bytes=1 << 40, saved=FAKE):
        return lib.poetx_group_fwd(C.byref(gd), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, saved, FAKE, ws_bytes,
                                   None)

    bad = B.group_desc(T, n, b, 3, B.POETX_BF16, B.POETX_FAST, ms)
    bad.count = 0
    assert fwd(bad) == B.POETX_ERR_SHAPE
    bad.count = 9
    assert fwd(bad) == B.POETX_ERR_SHAPE
    assert fwd(B.group_desc(T, n, b, 3, B.POETX_BF16, B.POETX_FAST, [4096, 1000])) == B.POETX_ERR_SHAPE
    assert fwd(B.group_desc(T, 4000, b, 3, B.POETX_BF16, B.POETX_FAST, ms)) == B.POETX_ERR_SHAPE
    assert fwd(B.group_desc(T, n, 24, 3, B.POETX_BF16, B.POETX_FAST, ms)) == B.POETX_ERR_UNSUPPORTED
    for v in (B.POETX_FOUR_PERM, B.POETX_WEIGHT_CENTRIC, B.POETX_MEM_Q8, 7):
        assert fwd(B.group_desc(T, n, b, 3, B.POETX_BF16, v, ms)) == B.POETX_ERR_INVALID_ARG
    bad = B.group_desc(T, n, b, 3, B.POETX_BF16, B.POETX_FAST, ms)
    bad.reserved = 1
    assert fwd(bad) == B.POETX_ERR_INVALID_ARG
    assert fwd(g, saved=None) == B.POETX_ERR_INVALID_ARG
    assert fwd(g, ws_bytes=lib.poetx_group_fwd_workspace_bytes(C.byref(g)) - 1) == B.POETX_ERR_WORKSPACE
    assert lib.poetx_group_fwd(None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 40,
                               None) == B.POETX_ERR_INVALID_ARG
    nb = lib.poetx_group_bwd_workspace_bytes(C.byref(g))
    assert lib.poetx_group_bwd(C.byref(g), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE,
                               nb, None) == B.POETX_ERR_INVALID_ARG
    assert lib.poetx_group_bwd(C.byref(g), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                               nb - 1, None) == B.POETX_ERR_WORKSPACE
    empty = B.group_desc(0, n, b, 3, B.POETX_BF16, B.POETX_FAST, ms)
    assert lib.poetx_group_fwd(C.byref(empty), None, None, None, None, None, None, None, None, None, 0,
                               None) == B.POETX_OK
    with pytest.raises(ValueError):
        B.group_desc(T, n, b, 3, B.POETX_BF16, B.POETX_FAST, [256] * 9)


def test_quantized_weight_layout_and_validation(B):
    lib = B.load()
    assert lib.poetx_qweight_bytes(4096, 4096) == 4096 * 4096 + 4 * 4096
    assert lib.poetx_qweight_bytes(3, 16) == 256 + 12
    assert lib.poetx_qweight_bytes(0, 16) == 0
    assert lib.poetx_quantize_weight(FAKE, B.POETX_BF16, 8, 40, FAKE, None) == B.POETX_ERR_SHAPE   # n % 16
    assert lib.poetx_quantize_weight(FAKE, 9, 8, 48, FAKE, None) == B.POETX_ERR_INVALID_ARG
    assert lib.poetx_quantize_weight(None, B.POETX_BF16, 8, 48, FAKE, None) == B.POETX_ERR_INVALID_ARG
    assert lib.poetx_quantize_weight(FAKE, B.POETX_BF16, 8, 48, FAKE + 8, None) == B.POETX_ERR_INVALID_ARG
    assert lib.poetx_dequantize_weight(FAKE, -1, 48, FAKE, None) == B.POETX_ERR_SHAPE
    # mem_q8: bf16 only, saves nothing; the layer calls need the mem workspace
    # only (the int8 codes go straight into the dense products), the merge also
    # one bf16 expansion of the weight
    q8 = B.desc(2048, 4096, 1024, 256, 3, B.POETX_BF16, B.POETX_MEM_Q8)
    mem = B.desc(2048, 4096, 1024, 256, 3, B.POETX_BF16, B.POETX_MEM)
    assert lib.poetx_linear_saved_bytes(C.byref(q8)) == 0
    for f in (lib.poetx_linear_fwd_workspace_bytes, lib.poetx_linear_bwd_workspace_bytes):
        assert f(C.byref(q8)) == f(C.byref(mem))
    assert lib.poetx_merge_workspace_bytes(C.byref(q8)) == lib.poetx_merge_workspace_bytes(C.byref(mem)) + \
        2 * 4096 * 1024
    # the int8 products run in 64-k steps over m and n: b % 64 == 0
    for bad_b in (16, 32, 48, 80):
        dbad = B.desc(64, 4 * bad_b, 2 * bad_b, bad_b, 3, B.POETX_BF16, B.POETX_MEM_Q8)
        assert lib.poetx_linear_fwd_workspace_bytes(C.byref(dbad)) == 0
        assert lib.poetx_linear_fwd(C.byref(dbad), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1 << 40,
                                    None) == B.POETX_ERR_SHAPE
    f32 = B.desc(2048, 4096, 1024, 256, 3, B.POETX_F32, B.POETX_MEM_Q8)
    assert lib.poetx_linear_fwd(C.byref(f32), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1 << 40,
                                None) == B.POETX_ERR_UNSUPPORTED
    # no saved buffer needed
    need = lib.poetx_linear_fwd_workspace_bytes(C.byref(q8))
    assert lib.poetx_linear_fwd(C.byref(q8), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, need - 1,
                                None) == B.POETX_ERR_WORKSPACE


def test_cnp_and_skew_validation(B):
    lib = B.load()
    assert lib.poetx_cnp_fwd(FAKE, 4, 24, 3, FAKE, 0, FAKE, 1 << 30, None) == 3
    assert lib.poetx_cnp_fwd(FAKE, 4, 16, 0, FAKE, 0, FAKE, 1 << 30, None) == 3
    assert lib.poetx_cnp_fwd(FAKE, -1, 16, 3, FAKE, 0, FAKE, 1 << 30, None) == 2
    assert lib.poetx_cnp_fwd(FAKE, 4, 16, 3, FAKE, 5, FAKE, 1 << 30, None) == 1
    need = lib.poetx_cnp_fwd_workspace_bytes(4, 16, 3, 0)
    assert need > 0
    assert lib.poetx_cnp_fwd(FAKE, 4, 16, 3, FAKE, 0, FAKE, need - 1, None) == 4
    assert lib.poetx_cnp_fwd(None, 4, 16, 3, FAKE, 0, FAKE, need, None) == 1
    assert lib.poetx_cnp_fwd(None, 0, 16, 3, None, 0, None, 0, None) == 0  # empty batch
    assert lib.poetx_cnp_bwd(FAKE, FAKE, 4, 16, 3, None, 0, FAKE, 1 << 30, None) == 1
    assert lib.poetx_skew_unpack(FAKE, FAKE, 3, 4, 16, None) == 1
    assert lib.poetx_skew_pack(FAKE, FAKE, 4, 0, None) == 2
    assert lib.poetx_permute(FAKE, FAKE, 0, 4, 6, None, None, 0, None) == 2  # 6 f32 columns: not 16-byte rows
    assert lib.poetx_check_perm(FAKE, 10, FAKE, FAKE, 3, None) == 4


def test_workspace_sizes_scale(B):
    lib = B.load()
    d = B.desc(2048, 4096, 4096, 256, 3, B.POETX_BF16, B.POETX_FAST)
    # FAST keeps h2 [T, m] and the gathered input a [T, n] (at a 256-byte boundary)
    assert lib.poetx_linear_saved_bytes(C.byref(d)) == 2048 * 4096 * 2 + 2048 * 4096 * 2
    d3 = B.desc(7, 48, 32, 16, 3, B.POETX_F32, B.POETX_FAST)
    assert lib.poetx_linear_saved_bytes(C.byref(d3)) == (7 * 48 * 4 + 255) // 256 * 256 + 7 * 32 * 4
    dm = B.desc(2048, 4096, 4096, 256, 3, B.POETX_BF16, B.POETX_MEM)
    assert lib.poetx_linear_saved_bytes(C.byref(dm)) == 0
    assert lib.poetx_linear_bwd_workspace_bytes(C.byref(dm)) >= 3 * 2048 * 4096 * 2
    assert lib.poetx_cnp_fwd_workspace_bytes(64, 256, 3, 1) == 2 * lib.poetx_cnp_fwd_workspace_bytes(32, 256, 3, 1)


def test_cnp_saved_validation(B):
    lib = B.load()
    sb = lib.poetx_cnp_saved_bytes(4, 256, 3, 1)
    # k = 3, bf16: Q (float32 and bf16), 2Q + 2S (float32), S and 2Q + S (bf16)
    assert sb >= 4 * 256 * 256 * (4 + 2 + 4 + 2 + 2)
    ws = lib.poetx_cnp_bwd_workspace_bytes(4, 256, 3, 1)
    assert lib.poetx_cnp_fwd_save(FAKE, 4, 256, 3, FAKE, 1, None, sb, FAKE, ws, None) == 1
    assert lib.poetx_cnp_fwd_save(FAKE, 4, 256, 3, FAKE, 1, FAKE, sb - 1, FAKE, ws, None) == 4
    assert lib.poetx_cnp_bwd_saved(FAKE, FAKE, 4, 256, 3, FAKE, 1, None, sb, FAKE, ws, None) == 1
    assert lib.poetx_cnp_bwd_saved(FAKE, FAKE, 4, 256, 3, FAKE, 1, FAKE, sb - 1, FAKE, ws, None) == 4
    assert lib.poetx_cnp_bwd_saved(FAKE, FAKE, 4, 256, 3, FAKE, 1, FAKE, sb, FAKE, 0, None) == 4
    assert lib.poetx_cnp_fwd_save(FAKE, 4, 24, 3, FAKE, 1, FAKE, sb, FAKE, ws, None) == 3
    assert lib.poetx_cnp_saved_bytes(4, 24, 3, 1) == 0


def test_adamw_validation(B):
    lib = B.load()
    ok = B.adamw_params(1e-3)
    fake = 256  # never dereferenced: every case below fails validation or has count == 0
    step = lambda count, t, p: lib.poetx_adamw_step(fake, fake, fake, fake, count, t, C.byref(p) if p else None, None)
    assert lib.poetx_adamw_step(None, None, None, None, 0, 1, C.byref(ok), None) == B.POETX_OK
    assert step(10, 1, None) == B.POETX_ERR_INVALID_ARG
    assert step(10, 0, ok) == B.POETX_ERR_INVALID_ARG
    assert step(-1, 1, ok) == B.POETX_ERR_SHAPE
    assert step(1 << 31, 1, ok) == B.POETX_ERR_SHAPE
    for bad in (dict(beta1=1.0), dict(beta2=-0.1), dict(eps=-1.0), dict(weight_decay=-0.5), dict(lr=float("inf")),
                dict(gamma=float("nan")), dict(beta2=float("nan"))):
        assert step(10, 1, B.adamw_params(**{"lr": 1e-3, **bad})) == B.POETX_ERR_INVALID_ARG, bad
    assert lib.poetx_adamw_step(fake, None, fake, fake, 10, 1, C.byref(ok), None) == B.POETX_ERR_INVALID_ARG
    assert lib.poetx_adamw_reset(None, None, 0, None) == B.POETX_OK
    assert lib.poetx_adamw_reset(fake, None, 4, None) == B.POETX_ERR_INVALID_ARG
    assert lib.poetx_adamw_reset(fake, fake, -2, None) == B.POETX_ERR_SHAPE
