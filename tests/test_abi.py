"""CPU-side checks of the C ABI: the library loads, exports every declared symbol, and the
host-only paths (byte accounting, argument validation) behave as documented.  No call here
launches a kernel: every device call below fails validation before any HIP work."""
import ctypes
import json
import os
import re
import subprocess

import pytest

import weight_only_mixed_amd as q

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qpack.h")
GOLD = json.load(open(os.path.join(ROOT, "tests", "golden", "page_values.json")))


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(q\w+)\s*\(", text, flags=re.M)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert len(names) >= 14
    out = subprocess.run(["nm", "-D", "--defined-only", q._LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (\w+)$", out, flags=re.M))
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    for n in names:
        assert hasattr(q.lib, n)
    assert set(q.EXPORTED) == set(names)


def test_packed_bytes_and_groups():
    for bits in (2, 3, 4, 5, 6):
        d = q.desc(bits, 4096, 4096)
        assert q.qp_packed_bytes(d) == 4096 * 4096 * bits // 8
        assert q.qp_num_groups(d) == 4096 * 32
    assert q.qp_packed_bytes(q.desc(4, 28672, 8192)) == 117_440_512
    assert q.qp_packed_bytes(q.desc(7, 16, 256)) == 0


@pytest.mark.parametrize("c", GOLD["kv_quantized"] + [dict(numel=c["group"], bits=c["bits"], group=c["group"],
                                                             scale_bytes=c["scale_bytes"], zp_bits=c["zp_bits"],
                                                             bpw=c.get("value"))
                                                        for c in GOLD["bits_per_weight"] if "value" in c])
def test_quant_bytes_match_pages(c):
    b = q.qp_quant_bytes(c["numel"], c["bits"], c["group"], c["scale_bytes"], c["zp_bits"])
    if "bpw" in c:
        assert b * 8 / c["group"] == c["bpw"]
    elif "bytes" in c:
        assert b == c["bytes"]
    else:
        assert b == c["bytes_approx"]


def test_outlier_count():
    assert q.qp_outlier_count(28672, 8192, 0.001) == 234_881
    assert q.qp_outlier_count(64, 1024, 0.001) == 65
    assert q.qp_outlier_count(10, 10, 0.0) == 0


FAKE = 0x10000  # an aligned, never-dereferenced address: validation fails before any launch


@pytest.mark.parametrize("d,expect", [
    (q.desc(7, 16, 256), q.QP_ERR_INVALID_ARG),
    (q.desc(1, 16, 256), q.QP_ERR_INVALID_ARG),
    (q.desc(4, 16, 200), q.QP_ERR_INVALID_ARG),
    (q.desc(4, 16, 256, group_size=256), q.QP_ERR_UNSUPPORTED),
    (q.desc(4, 16, 256, group_size=16), q.QP_ERR_UNSUPPORTED),
    (q.desc(4, 15, 256), q.QP_ERR_INVALID_ARG),           # device layout needs n % 16
    (q.desc(4, 16, 384), q.QP_ERR_INVALID_ARG),           # device layout needs k % 256
    (q.desc(4, 0, 256), q.QP_ERR_INVALID_ARG),
])
def test_pack_rejects_bad_descriptors(d, expect):
    assert q.qpack_pack(d, FAKE, FAKE, stream=0, check=False) == expect
    assert q.last_error()


def test_pack_rejects_misaligned_pointers():
    d = q.desc(4, 16, 256)
    assert q.qpack_pack(d, FAKE + 1, FAKE, stream=0, check=False) == q.QP_ERR_INVALID_ARG
    assert q.qpack_pack(d, FAKE, FAKE + 8, stream=0, check=False) == q.QP_ERR_INVALID_ARG
    assert q.qpack_pack(d, None, FAKE, stream=0, check=False) == q.QP_ERR_INVALID_ARG


def test_gemv_validation():
    d = q.desc(4, 256, 512)
    w = q.weight(FAKE, FAKE, FAKE)
    assert q.qlinear_gemv(d, w, FAKE, 512, 17, FAKE, 256, stream=0, check=False) == q.QP_ERR_UNSUPPORTED
    assert q.qlinear_gemv(d, w, FAKE, 512, 0, FAKE, 256, stream=0, check=False) == q.QP_ERR_INVALID_ARG
    assert q.qlinear_gemv(d, w, FAKE, 500, 1, FAKE, 256, stream=0, check=False) == q.QP_ERR_INVALID_ARG
    assert q.qlinear_gemv(d, w, FAKE + 2, 512, 1, FAKE, 256, stream=0, check=False) == q.QP_ERR_INVALID_ARG
    assert q.qlinear_gemv(d, w, FAKE, 512, 1, FAKE, 100, stream=0, check=False) == q.QP_ERR_INVALID_ARG
    canon = q.desc(4, 256, 512, layout=q.QP_LAYOUT_CANONICAL)
    assert q.qlinear_gemv(canon, w, FAKE, 512, 1, FAKE, 256, stream=0, check=False) == q.QP_ERR_UNSUPPORTED
    bad_csr = q.weight(FAKE, FAKE, FAKE, None, None, None, 5)
    assert q.qlinear_gemm(d, bad_csr, FAKE, 512, 64, FAKE, 256, stream=0, check=False) == q.QP_ERR_INVALID_ARG
    assert "csr" in q.last_error().lower()
    csr = q.weight(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 5)
    need = q.qlinear_gemm_workspace_bytes(d, 64, 5)
    assert need == (2 * 512 + 4 * 256) * 128 and q.qlinear_gemm_workspace_bytes(d, 64, 0) == 0
    assert q.qlinear_gemm(d, csr, FAKE, 512, 64, FAKE, 256, FAKE, need - 1, stream=0,
                          check=False) == q.QP_ERR_WORKSPACE


def test_gemv_batch_validation():
    d = q.desc(4, 256, 512)
    w = q.weight(FAKE, FAKE, FAKE)
    good = q.gemv_problem(d, w, FAKE, 512, 1, FAKE, 256)
    assert q.qlinear_gemv_batch([], stream=0, check=False) == q.QP_ERR_INVALID_ARG
    assert q.qlinear_gemv_batch([good] * 9, stream=0, check=False) == q.QP_ERR_INVALID_ARG
    bad_ldx = q.gemv_problem(d, w, FAKE, 500, 1, FAKE, 256)
    assert q.qlinear_gemv_batch([good, bad_ldx], stream=0, check=False) == q.QP_ERR_INVALID_ARG
    assert "ldx" in q.last_error()
    big_m = q.gemv_problem(d, w, FAKE, 512, 17, FAKE, 256)
    assert q.qlinear_gemv_batch([good, big_m], stream=0, check=False) == q.QP_ERR_UNSUPPORTED
    canon = q.gemv_problem(q.desc(4, 256, 512, layout=q.QP_LAYOUT_CANONICAL), w, FAKE, 512, 1, FAKE, 256)
    assert q.qlinear_gemv_batch([canon], stream=0, check=False) == q.QP_ERR_UNSUPPORTED


def test_quantize_validation():
    d = q.desc(4, 64, 1024)
    st, nnz = q.qpack_quantize(d, FAKE, 1024, 0.001, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 10, FAKE, 1 << 20,
                               stream=0, check=False)
    assert st == q.QP_ERR_WORKSPACE and nnz == 65          # CSR capacity too small
    st, _ = q.qpack_quantize(d, FAKE, 1024, 0.001, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 65, FAKE, 16,
                             stream=0, check=False)
    assert st == q.QP_ERR_WORKSPACE                         # workspace too small
    st, _ = q.qpack_quantize(d, FAKE, 1023, 0.0, FAKE, FAKE, FAKE, stream=0, check=False)
    assert st == q.QP_ERR_INVALID_ARG                       # odd / short ldw
    st, _ = q.qpack_quantize(d, FAKE, 1024, 1.5, FAKE, FAKE, FAKE, stream=0, check=False)
    assert st == q.QP_ERR_INVALID_ARG
    assert q.qpack_quantize_workspace_bytes(d, 0.0) == 0
    assert q.qpack_quantize_workspace_bytes(d, 0.001) > 32768 * 4


def test_zero_mode_validation():
    """QP_ZERO_MIDPOINT descriptors are valid at every bit width and need no zero points;
    unknown modes are rejected; QP_ZERO_STORED still needs them (all checked before any
    device work)."""
    for bits in (2, 3, 4, 5, 6):
        assert q.qp_packed_bytes(q.desc(bits, 64, 1024, zero_mode=q.QP_ZERO_MIDPOINT)) == 64 * 1024 * bits // 8
    assert q.qp_packed_bytes(q.desc(4, 64, 1024, zero_mode=3)) == 0
    assert q.qp_packed_bytes(q.desc(4, 64, 1024, zero_mode=-1)) == 0
    d = q.desc(4, 64, 1024)
    st, _ = q.qpack_quantize(d, FAKE, 1024, 0.0, FAKE, FAKE, None, stream=0, check=False)
    assert st == q.QP_ERR_INVALID_ARG                       # stored zero points need a buffer
    w = q.weight(FAKE, FAKE, None)
    assert q.qlinear_gemv(d, w, FAKE, 1024, 1, FAKE, 64, stream=0, check=False) == q.QP_ERR_INVALID_ARG
    bad = q.desc(4, 64, 1024, zero_mode=3)
    assert q.qlinear_gemv(bad, q.weight(FAKE, FAKE, FAKE), FAKE, 1024, 1, FAKE, 64, stream=0,
                          check=False) == q.QP_ERR_INVALID_ARG


def test_group_size_validation():
    """Groups of 32, 64 and 128 are valid descriptors (k a multiple of 128); other sizes are
    not built; the int8-activation GEMM takes only 128; a GEMV batch takes one group size."""
    for g in (32, 64, 128):
        assert q.qp_num_groups(q.desc(2, 64, 1024, group_size=g)) == 64 * 1024 // g
    assert q.qp_num_groups(q.desc(2, 64, 1024, group_size=256)) == 0
    assert q.qp_num_groups(q.desc(2, 64, 1088, group_size=32)) == 0     # k not a multiple of 128
    d32 = q.desc(2, 256, 512, group_size=32)
    w = q.weight(FAKE, FAKE, FAKE)
    assert q.qlinear_gemm_a8(d32, w, FAKE, FAKE, 64, FAKE, 256, stream=0, check=False) == q.QP_ERR_UNSUPPORTED
    p32 = q.gemv_problem(d32, w, FAKE, 512, 1, FAKE, 256)
    p128 = q.gemv_problem(q.desc(2, 256, 512), w, FAKE, 512, 1, FAKE, 256)
    assert q.qlinear_gemv_batch([p32, p128], stream=0, check=False) == q.QP_ERR_UNSUPPORTED


def test_grouped_and_moe_validation():
    d = q.desc(4, 256, 512)
    w = q.weight(FAKE, FAKE, FAKE)
    assert q.qlinear_grouped_gemm(d, [w] * 65, FAKE, 512, FAKE, FAKE, 10, 0, FAKE, 256, stream=0,
                                  check=False) == q.QP_ERR_INVALID_ARG
    assert q.qlinear_grouped_gemm(d, [w], FAKE, 512, FAKE, FAKE, 10, 9, FAKE, 256, stream=0,
                                  check=False) == q.QP_ERR_INVALID_ARG
    d48 = q.desc(4, 48, 512)
    assert q.qlinear_grouped_gemm(d48, [w], FAKE, 512, FAKE, FAKE, 10, q.QP_EPI_SWIGLU, FAKE, 24, stream=0,
                                  check=False) == q.QP_ERR_INVALID_ARG
    assert q.qmoe_dispatch(FAKE, FAKE, 40000, 2, 16, FAKE, FAKE, FAKE, FAKE, stream=0,
                           check=False) == q.QP_ERR_INVALID_ARG
    assert q.qmoe_dispatch(FAKE, FAKE, 128, 2, 65, FAKE, FAKE, FAKE, FAKE, stream=0,
                           check=False) == q.QP_ERR_INVALID_ARG
    gu, dn = q.desc(4, 2 * 14336, 4096), q.desc(4, 4096, 14336)
    need = q.qmoe_ffn_workspace_bytes(128, 2, 16, 4096, 14336)
    assert need > 256 * 14336 * 2
    assert q.qmoe_ffn(gu, [w] * 16, dn, [w] * 16, FAKE, 4096, 128, FAKE, FAKE, 2, FAKE, 4096, FAKE, need - 1,
                      stream=0, check=False) == q.QP_ERR_WORKSPACE


def test_grouped_rejects_more_row_tiles_than_the_grid_holds():
    """The grouped launch's second grid dimension counts 32-row tiles of routed rows: more than
    65535 of them is refused before any launch."""
    d = q.desc(4, 256, 256)
    w = q.weight(FAKE, FAKE, FAKE)
    rows = 65536 * 32
    assert q.qlinear_grouped_gemm(d, [w], FAKE, 256, FAKE, FAKE, rows, q.QP_EPI_NONE, FAKE, 256, stream=0,
                                  check=False) == q.QP_ERR_UNSUPPORTED
    assert "65535" in q.last_error()


def test_moe_ffn_rejects_intermediate_beyond_2gib():
    """The fp16 intermediate [tokens*topk][d_ff] is read through one 2 GiB buffer range: 65536
    routed rows at d_ff = 16384 (2 GiB exactly) must be refused before any launch."""
    w = q.weight(FAKE, FAKE, FAKE)
    gu, dn = q.desc(4, 2 * 16384, 4096), q.desc(4, 4096, 16384)
    need = q.qmoe_ffn_workspace_bytes(32768, 2, 16, 4096, 16384)
    assert q.qmoe_ffn(gu, [w] * 16, dn, [w] * 16, FAKE, 4096, 32768, FAKE, FAKE, 2, FAKE, 4096, FAKE, need,
                      stream=0, check=False) == q.QP_ERR_UNSUPPORTED
    assert "2 GiB" in q.last_error()


def test_status_message_is_thread_local_text():
    q.qpack_pack(q.desc(9, 16, 256), FAKE, FAKE, stream=0, check=False)
    assert "bits=9" in q.last_error()


# ---- quantized KV cache ----------------------------------------------------------------

def _kv_layer_bytes(d):
    return sum(q.qkv_cache_bytes(d, w) + 4 * q.qkv_scale_count(d, w) for w in (q.QKV_K, q.QKV_V))


@pytest.mark.parametrize("heads,group,mib", [(32, 64, 288), (32, 128, 272), (4, 64, 36)])
def test_kv_cache_sizes_match_page(heads, group, mib):
    """KV page s3.1-s3.2: 32 layers, 2048 tokens, INT4 K and V with FP32 scales."""
    d = q.kv_desc(1, heads, heads, 2048, 4, 4, group, group)
    assert 32 * _kv_layer_bytes(d) == mib * 2 ** 20


def test_kv_mixed_precision_size():
    """KV page s2.3: INT4 K with INT8 V leaves 0.375 GB of the 1 GB fp16 cache."""
    c = GOLD["kv_mixed_k4_v8"]
    d = q.kv_desc(1, c["kv_heads"], c["kv_heads"], c["tokens"], c["k_bits"], c["v_bits"])
    assert c["layers"] * (q.qkv_cache_bytes(d, q.QKV_K) + q.qkv_cache_bytes(d, q.QKV_V)) == c["bytes"]


def test_kv_workspace():
    assert q.qattn_decode_workspace_bytes(q.kv_desc(64, 32, 32, 128)) == 0     # one chunk each
    d = q.kv_desc(1, 32, 8, 32768)
    ws = q.qattn_decode_workspace_bytes(d)
    assert ws > 0 and ws % (32 * (128 * 4 + 8)) == 0


FAKE = 1 << 20  # a 16-byte aligned address; never dereferenced (validation fails first)


@pytest.mark.parametrize("field,value,status", [
    ("head_dim", 64, q.QP_ERR_UNSUPPORTED), ("k_bits", 2, q.QP_ERR_UNSUPPORTED), ("v_bits", 6, q.QP_ERR_UNSUPPORTED),
    ("k_group", 16, q.QP_ERR_UNSUPPORTED), ("v_group", 256, q.QP_ERR_UNSUPPORTED),
    ("q_heads", 12, q.QP_ERR_INVALID_ARG), ("q_heads", 8 * 17, q.QP_ERR_UNSUPPORTED),
    ("capacity", 48, q.QP_ERR_INVALID_ARG), ("capacity", 0, q.QP_ERR_INVALID_ARG), ("batch", 0, q.QP_ERR_INVALID_ARG)])
def test_kv_desc_validation(field, value, status):
    d = q.kv_desc(2, 16, 8, 256)
    setattr(d, field, value)
    assert q.qkv_cache_bytes(d, q.QKV_K) == 0 and q.qkv_scale_count(d, q.QKV_V) == 0
    assert q.qkv_quantize(d, q.QKV_K, FAKE, 128, FAKE, 4, FAKE, FAKE, check=False) == status
    assert q.qattn_decode(d, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0.1, FAKE, FAKE, 1 << 30, check=False) == status
    assert q.last_error()


def test_kv_call_validation():
    d = q.kv_desc(2, 16, 8, 256)
    E = q.QP_ERR_INVALID_ARG
    assert q.qkv_quantize(d, 2, FAKE, 128, FAKE, 4, FAKE, FAKE, check=False) == E
    assert q.qkv_quantize(d, q.QKV_V, FAKE + 2, 128, FAKE, 4, FAKE, FAKE, check=False) == E   # x misaligned
    assert q.qkv_quantize(d, q.QKV_V, FAKE, 120, FAKE, 4, FAKE, FAKE, check=False) == E       # ldx < 128
    assert q.qkv_quantize(d, q.QKV_V, FAKE, 128, None, 4, FAKE, FAKE, check=False) == E       # slots NULL
    assert q.qkv_quantize(d, q.QKV_V, FAKE, 128, FAKE, -1, FAKE, FAKE, check=False) == E
    assert q.qkv_quantize(d, q.QKV_V, FAKE, 128, FAKE, 4, FAKE + 8, FAKE, check=False) == E   # codes misaligned
    assert q.qattn_decode(d, FAKE + 2, FAKE, FAKE, FAKE, FAKE, FAKE, 0.1, FAKE, check=False) == E
    assert q.qattn_decode(d, FAKE, None, FAKE, FAKE, FAKE, FAKE, 0.1, FAKE, check=False) == E
    assert q.qattn_decode(d, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0.1, FAKE, check=False) == E
    assert q.qattn_decode(d, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, float("nan"), FAKE, check=False) == E
    big = q.kv_desc(1, 8, 8, 32768)
    need = q.qattn_decode_workspace_bytes(big)
    assert need > 0
    assert q.qattn_decode(big, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0.1, FAKE, FAKE, need - 1,
                          check=False) == q.QP_ERR_WORKSPACE
    assert q.qattn_decode(big, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0.1, FAKE, None, 0,
                          check=False) == q.QP_ERR_WORKSPACE


def test_packed_zero_points():
    """QP_ZERO_PACKED: zero points in b bits per group, rows padded to 32-bit words; every
    matmul checks their alignment, a GEMV batch does not mix them with byte zero points;
    qpack_pack_zeros checks its mode and pointers (all before any device work)."""
    for bits in (2, 3, 4, 5, 6):
        for g in (32, 64, 128):
            for k in (1024, 1280, 11008 // 128 * 128):
                G = k // g
                d = q.desc(bits, 64, k, group_size=g, zero_mode=q.QP_ZERO_PACKED)
                assert q.qp_zero_bytes(d) == 64 * 4 * ((G * bits + 31) // 32)
                assert q.qp_zero_bytes(q.desc(bits, 64, k, group_size=g)) == 64 * G
                assert q.qp_zero_bytes(q.desc(bits, 64, k, group_size=g, zero_mode=q.QP_ZERO_MIDPOINT)) == 0
    d = q.desc(2, 256, 1024, group_size=128, zero_mode=q.QP_ZERO_PACKED)
    w = q.weight(FAKE, FAKE, FAKE)
    U, E = q.QP_ERR_UNSUPPORTED, q.QP_ERR_INVALID_ARG
    misaligned = q.weight(FAKE, FAKE, FAKE + 2)                  # packed zeros need 4-byte alignment
    assert q.qlinear_gemv(d, misaligned, FAKE, 1024, 1, FAKE, 256, stream=0, check=False) == E
    assert q.qlinear_gemm(d, misaligned, FAKE, 1024, 64, FAKE, 256, stream=0, check=False) == E
    assert q.qlinear_grouped_gemm(d, [misaligned], FAKE, 1024, FAKE, FAKE, 64, q.QP_EPI_NONE, FAKE, 256, stream=0,
                                  check=False) == E
    assert q.qlinear_gemm_a8(d, misaligned, FAKE, FAKE, 64, FAKE, 256, stream=0, check=False) == E
    ds = q.desc(2, 256, 1024, group_size=128)
    probs = [q.gemv_problem(d, w, FAKE, 1024, 1, FAKE, 256), q.gemv_problem(ds, w, FAKE, 1024, 1, FAKE, 256)]
    assert q.qlinear_gemv_batch(probs, stream=0, check=False) == U
    assert q.qpack_pack_zeros(ds, FAKE, FAKE, stream=0, check=False) == E      # mode must be packed
    assert q.qpack_pack_zeros(d, FAKE + 1, FAKE, stream=0, check=False) == E
    assert q.qpack_pack_zeros(d, FAKE, FAKE + 2, stream=0, check=False) == E


def test_attention_noalloc_rejects_scratch_beyond_its_limit():
    """16 query heads per kv head over 16 kv heads split into 16 chunks needs 4096 partials
    (2,129,920 bytes), above the fixed 2 MiB: refused before any device call."""
    d = q.kv_desc(1, 256, 16, 32768, 4, 8, 64, 64)
    need = q.qattn_decode_workspace_bytes(d)
    assert need == 4096 * (128 * 4 + 8) > q.QATTN_NOALLOC_SCRATCH_BYTES
    st = q.qattn_decode_noalloc(d, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0.1, FAKE, stream=0, check=False)
    assert st == q.QP_ERR_WORKSPACE and "2097152" in q.last_error()
    # within the limit: the benchmarked 4 x 8K GQA layer (2048 partials)
    assert 0 < q.qattn_decode_workspace_bytes(q.kv_desc(4, 64, 8, 8192)) <= q.QATTN_NOALLOC_SCRATCH_BYTES


def test_int8_path_validation():
    """qact_quantize / qlinear_gemm_a8 reject what the kernels do not handle, before any launch."""
    assert q.qact_quantize(FAKE, 256, 4, 200, FAKE, FAKE, stream=0, check=False) == q.QP_ERR_INVALID_ARG  # k % 128
    assert q.qact_quantize(FAKE, 100, 4, 128, FAKE, FAKE, stream=0, check=False) == q.QP_ERR_INVALID_ARG  # ldx < k
    assert q.qact_quantize(FAKE + 8, 128, 4, 128, FAKE, FAKE, stream=0, check=False) == q.QP_ERR_INVALID_ARG
    assert q.qact_quantize(FAKE, 128, 0, 128, FAKE, FAKE, stream=0, check=False) == q.QP_ERR_INVALID_ARG
    assert q.qact_quantize(FAKE, 128, 4, 128, FAKE + 4, FAKE, stream=0, check=False) == q.QP_ERR_INVALID_ARG
    d = q.desc(4, 256, 512)
    w = q.weight(FAKE, FAKE, FAKE)
    ok = dict(stream=0, check=False)
    assert q.qlinear_gemm_a8(d, w, FAKE, FAKE, 0, FAKE, 256, **ok) == q.QP_ERR_INVALID_ARG
    assert q.qlinear_gemm_a8(d, w, FAKE + 8, FAKE, 4, FAKE, 256, **ok) == q.QP_ERR_INVALID_ARG
    assert q.qlinear_gemm_a8(d, w, FAKE, FAKE, 4, FAKE, 100, **ok) == q.QP_ERR_INVALID_ARG
    assert q.qlinear_gemm_a8(d, w, FAKE, FAKE, (1 << 31) // 512, FAKE, 256, **ok) == q.QP_ERR_UNSUPPORTED
    csr = q.weight(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 5)
    assert q.qlinear_gemm_a8(d, csr, FAKE, FAKE, 4, FAKE, 256, **ok) == q.QP_ERR_UNSUPPORTED
    assert "outlier" in q.last_error()
    d64 = q.desc(4, 256, 512, group_size=64)
    assert q.qlinear_gemm_a8(d64, w, FAKE, FAKE, 4, FAKE, 256, **ok) == q.QP_ERR_UNSUPPORTED
    canon = q.desc(4, 256, 512, layout=q.QP_LAYOUT_CANONICAL)
    assert q.qlinear_gemm_a8(canon, w, FAKE, FAKE, 4, FAKE, 256, **ok) == q.QP_ERR_UNSUPPORTED


def test_fp8_scale_validation():
    """QP_SCALE_FP8 (8-bit float scales with an fp16 fallback, mixed-bit page s2.3): only the
    fp8 quantizer writes it; the GEMVs (device and host), the layer GEMM, the int8-activation
    GEMM, the grouped GEMM and the expert FFN read it; the blob refuses it, and the fp8 calls
    check their buffers before any launch (no call here gets past validation: every weight or
    shape is malformed)."""
    ok = dict(stream=0, check=False)
    f8 = q.desc(2, 256, 512, group_size=32, zero_mode=q.QP_ZERO_MIDPOINT, scale_format=q.QP_SCALE_FP8)
    fp16 = q.desc(2, 256, 512, group_size=32, zero_mode=q.QP_ZERO_MIDPOINT)
    assert q.qp_packed_bytes(q.desc(2, 256, 512, scale_format=7)) == 0
    assert q.qp_packed_bytes(f8) == 256 * 512 // 4
    assert q.qp_packed_bytes(q.desc(2, 256, 512, zero_mode=q.QP_ZERO_PACKED, scale_format=q.QP_SCALE_FP8)) == 0
    # the fp8 quantizer
    args = (FAKE, 512, FAKE, FAKE, FAKE, FAKE, FAKE, 8, FAKE)
    assert q.qpack_quantize_fp8(fp16, *args, **ok) == q.QP_ERR_INVALID_ARG
    assert q.qpack_quantize_fp8(f8, FAKE, 512, FAKE, None, FAKE, FAKE, FAKE, 8, FAKE, **ok) == q.QP_ERR_INVALID_ARG
    assert q.qpack_quantize_fp8(f8, FAKE, 512, FAKE, FAKE, FAKE, FAKE, FAKE, 129, FAKE, **ok) == q.QP_ERR_INVALID_ARG
    assert q.qpack_quantize_fp8(f8, FAKE, 512, FAKE, FAKE, FAKE, FAKE, None, 8, FAKE, **ok) == q.QP_ERR_INVALID_ARG
    assert q.qpack_quantize_fp8(f8, FAKE, 510, FAKE, FAKE, FAKE, FAKE, FAKE, 8, FAKE, **ok) == q.QP_ERR_INVALID_ARG
    assert q.qpack_quantize_fp8(f8, FAKE, 512, FAKE, FAKE, FAKE, FAKE + 2, FAKE, 8, FAKE, **ok) == q.QP_ERR_INVALID_ARG
    stored = q.desc(2, 256, 512, group_size=32, scale_format=q.QP_SCALE_FP8)
    assert q.qpack_quantize_fp8(stored, FAKE, 512, FAKE, FAKE, None, FAKE, FAKE, 8, FAKE, **ok) == q.QP_ERR_INVALID_ARG
    wide = q.desc(2, 16, 524416, layout=q.QP_LAYOUT_CANONICAL, group_size=32,
                  scale_format=q.QP_SCALE_FP8)  # 16388 groups per row
    assert q.qpack_quantize_fp8(wide, FAKE, 524416, *args[2:], **ok) == q.QP_ERR_UNSUPPORTED
    st, _ = q.qpack_quantize(f8, FAKE, 512, 0.0, FAKE, FAKE, FAKE, **ok)
    assert st == q.QP_ERR_UNSUPPORTED
    # the GEMV checks the fp8 buffers
    good = q.weight_fp8(FAKE, FAKE, FAKE, FAKE, 8)
    bad = q.weight_fp8(FAKE, None, FAKE, FAKE, 8)
    assert q.qlinear_gemv(f8, q.weight_fp8(FAKE, None, FAKE, FAKE, 8), FAKE, 512, 1, FAKE, 256, **ok) == q.QP_ERR_INVALID_ARG
    assert q.qlinear_gemv(f8, q.weight_fp8(FAKE, FAKE, None, FAKE, 8), FAKE, 512, 1, FAKE, 256, **ok) == q.QP_ERR_INVALID_ARG
    assert q.qlinear_gemv(f8, q.weight_fp8(FAKE, FAKE, FAKE, None, 8), FAKE, 512, 1, FAKE, 256, **ok) == q.QP_ERR_INVALID_ARG
    assert q.qlinear_gemv(f8, q.weight_fp8(FAKE, FAKE, FAKE, FAKE, 129), FAKE, 512, 1, FAKE, 256, **ok) == q.QP_ERR_INVALID_ARG
    assert q.qlinear_gemv(f8, q.weight_fp8(FAKE, FAKE + 1, FAKE, FAKE, 8), FAKE, 512, 1, FAKE, 256, **ok) == q.QP_ERR_INVALID_ARG
    assert q.qlinear_gemv(f8, good, FAKE, 512, 17, FAKE, 256, **ok) == q.QP_ERR_UNSUPPORTED
    with_csr = q.weight_fp8(FAKE, FAKE, FAKE, FAKE, 8)
    with_csr.csr_rowptr, with_csr.csr_col, with_csr.csr_val, with_csr.nnz = FAKE, FAKE, FAKE, 5
    assert q.qlinear_gemv(f8, with_csr, FAKE, 512, 1, FAKE, 256, **ok) == q.QP_ERR_UNSUPPORTED
    # the batched GEMV checks every problem's fp8 buffers and takes one scale format per batch
    assert q.qlinear_gemv_batch([q.gemv_problem(f8, good, FAKE, 512, 1, FAKE, 256),
                                 q.gemv_problem(f8, bad, FAKE, 512, 1, FAKE, 256)], **ok) == q.QP_ERR_INVALID_ARG
    f16 = q.desc(2, 256, 512, group_size=32, zero_mode=q.QP_ZERO_MIDPOINT)
    w16 = q.qp_weight(FAKE, FAKE, None, None, None, None, 0)
    assert q.qlinear_gemv_batch([q.gemv_problem(f8, good, FAKE, 512, 1, FAKE, 256),
                                 q.gemv_problem(f16, w16, FAKE, 512, 1, FAKE, 256)], **ok) == q.QP_ERR_UNSUPPORTED
    # the layer GEMM reads them too (validation only here: a malformed weight is refused)
    assert q.qlinear_gemm(f8, q.weight_fp8(FAKE, None, FAKE, FAKE, 8), FAKE, 512, 64, FAKE, 256, **ok) == \
        q.QP_ERR_INVALID_ARG
    assert q.qlinear_gemm(f8, with_csr, FAKE, 512, 64, FAKE, 256, **ok) == q.QP_ERR_UNSUPPORTED
    # the grouped GEMM and the expert FFN check every expert's fp8 buffers
    assert q.qlinear_grouped_gemm(f8, [good, bad], FAKE, 512, FAKE, FAKE, 10, 0, FAKE, 256, **ok) == q.QP_ERR_INVALID_ARG
    assert q.qlinear_grouped_gemm(f8, [good, q.weight_fp8(FAKE, FAKE, FAKE, FAKE, 129)], FAKE, 512, FAKE, FAKE, 10, 0,
                                  FAKE, 256, **ok) == q.QP_ERR_INVALID_ARG
    assert q.qlinear_grouped_gemm(f8, [with_csr], FAKE, 512, FAKE, FAKE, 10, 0, FAKE, 256, **ok) == q.QP_ERR_UNSUPPORTED
    f8_128 = q.desc(4, 256, 512, zero_mode=q.QP_ZERO_MIDPOINT, scale_format=q.QP_SCALE_FP8)
    assert q.qlinear_gemm_a8(f8_128, bad, FAKE, FAKE, 4, FAKE, 256, **ok) == q.QP_ERR_INVALID_ARG
    assert q.qlinear_gemm_a8(f8_128, with_csr, FAKE, FAKE, 4, FAKE, 256, **ok) == q.QP_ERR_UNSUPPORTED
    gu = q.desc(4, 2 * 1024, 512, scale_format=q.QP_SCALE_FP8)
    dn = q.desc(4, 512, 1024, scale_format=q.QP_SCALE_FP8)
    assert q.qmoe_ffn(gu, [good] * 4, dn, [good] * 3 + [bad], FAKE, 512, 8, FAKE, FAKE, 2, FAKE, 512, FAKE, 1 << 30,
                      **ok) == q.QP_ERR_INVALID_ARG
    assert q.qmoe_ffn(gu, [good] * 3 + [bad], dn, [good] * 4, FAKE, 512, 8, FAKE, FAKE, 2, FAKE, 512, FAKE, 1 << 30,
                      **ok) == q.QP_ERR_INVALID_ARG
    canon8 = q.desc(2, 256, 512, layout=q.QP_LAYOUT_CANONICAL, group_size=32, zero_mode=q.QP_ZERO_MIDPOINT,
                    scale_format=q.QP_SCALE_FP8)
    # the host GEMV reads fp8 scales too (validation only here: every weight is malformed)
    assert q.lib.qlinear_gemv_host(ctypes.byref(canon8), ctypes.byref(bad), FAKE, 512, 1, FAKE, 256, 1) == \
        q.QP_ERR_INVALID_ARG
    assert q.lib.qlinear_gemv_host(ctypes.byref(canon8), ctypes.byref(q.weight_fp8(FAKE, FAKE, FAKE, None, 8)), FAKE,
                                   512, 1, FAKE, 256, 1) == q.QP_ERR_INVALID_ARG
    assert q.lib.qlinear_gemv_host(ctypes.byref(canon8), ctypes.byref(with_csr), FAKE, 512, 1, FAKE, 256, 1) == \
        q.QP_ERR_UNSUPPORTED
    assert q.qp_blob_bytes(canon8, 0) == 0
    assert q.lib.qp_blob_write(ctypes.byref(canon8), ctypes.byref(good), FAKE, 1 << 20) == q.QP_ERR_UNSUPPORTED
