"""CPU checks of the C-ABI library: it loads, exports every function the
header declares, and its host-side validation returns the documented status
codes before any device work (no compute call is made here)."""

import ctypes
import os
import re

import pytest

from tests.conftest import ROOT

HEADER = os.path.join(ROOT, "include", "pdakv.h")


@pytest.fixture(scope="module")
def P():
    from paged_decode_attention_kv_amd import _lib as lib_mod
    return lib_mod


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", src, flags=re.M)))


def test_library_exports_every_declared_function(P):
    names = _declared_functions()
    assert len(names) == 23, names
    for n in names:
        assert hasattr(P._lib, n), n
    assert set(names) == set(P.EXPORTED)


# the calls of the boundary as the scope table names them: the two writers,
# the INT8 decode and its FP16-KV control, and the sizing queries
BOUNDARY_CALLS = {
    "pdakv_page_bytes": "size_t pdakv_page_bytes(int kv_format, int block_size, "
                        "int num_kv_heads, int head_dim)",
    "pdakv_capabilities": "int pdakv_capabilities(uint32_t* flags_out)",
    "paged_attn_decode_workspace_bytes": "size_t paged_attn_decode_workspace_bytes(int num_seqs, "
                                         "int num_q_heads, int head_dim, int max_context_len)",
    "kv_quant_int8_sym_write": None, "kv_write_16bit": None,
    "paged_attn_decode_int8": None, "paged_attn_decode_fp16": None,
}


def _flat_header():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return re.sub(r"\s+", " ", src)


def test_boundary_calls_are_declared_with_their_signatures(P):
    flat = _flat_header()
    for name, sig in BOUNDARY_CALLS.items():
        assert name in _declared_functions(), name
        assert hasattr(P._lib, name), name
        if sig is not None:
            assert sig + ";" in flat, sig
    # the writers and decodes share one argument list per kind
    for a, b in (("kv_quant_int8_sym_write", "kv_write_16bit"),
                 ("paged_attn_decode_int8", "paged_attn_decode_fp16")):
        args = [re.search(r"\b" + n + r"\((.*?)\);", flat).group(1) for n in (a, b)]
        assert args[0] == args[1]


@pytest.mark.parametrize("B,hq,d,L", [(64, 32, 128, 8193), (8, 32, 128, 32768),
                                      (32, 14, 64, 4105), (1, 32, 128, 2048), (3, 16, 64, 40),
                                      (2, 48, 128, 100)])
def test_any_kv_heads_workspace_is_the_largest_over_kv_heads(P, B, hq, d, L):
    """paged_attn_decode_workspace_bytes(B, Hq, D, L) is the largest
    pdakv_decode_workspace_bytes over the KV-head counts Hq allows."""
    sizes = [P.pdakv_decode_workspace_bytes(B, hq, hkv, d, L)
             for hkv in range(1, hq + 1) if hq % hkv == 0 and hq // hkv <= 16]
    assert P.paged_attn_decode_workspace_bytes(B, hq, d, L) == max(sizes) > 0
    assert P.paged_attn_decode_workspace_bytes(0, hq, d, L) == 0
    assert P.paged_attn_decode_workspace_bytes(B, hq, d, 0) == 0
    assert P.paged_attn_decode_workspace_bytes(B, 0, d, L) == 0


def test_version_and_status_strings(P):
    assert P.pdakv_version() >= 100
    for code in (0, -1, -2, -3, -4, -5, -6):
        s = P.pdakv_status_string(code)
        assert s and s != "unknown status"
    assert P.pdakv_status_string(-99) == "unknown status"


def test_page_bytes_match_the_printed_totals(P, golden):
    (row,) = golden("page_bytes.txt")
    bs, hkv, d, i8, f16, ratio = row[0].split()
    assert P.pdakv_page_bytes(P.KV_INT8_SYM, int(bs), int(hkv), int(d)) == int(i8)
    assert P.pdakv_page_bytes(P.KV_16BIT, int(bs), int(hkv), int(d)) == int(f16)
    assert P.pdakv_page_bytes(P.KV_INT8_SYM, 16, 2, 64) == 4224
    assert P.pdakv_page_bytes(7, 16, 8, 128) == 0
    assert P.pdakv_page_bytes(P.KV_INT8_SYM, 15, 8, 128) == 0
    # static scales: codes only, half the 16-bit page
    assert P.pdakv_page_bytes(P.KV_INT8_STATIC, 16, 8, 128) == 32768
    assert P.pdakv_page_bytes(P.KV_INT8_STATIC, 16, 2, 64) == 4096


def test_page_bytes_agree_with_oracle(P):
    import oracle
    for fmt in (P.KV_INT8_SYM, P.KV_16BIT, P.KV_INT8_STATIC):
        for hkv in (1, 2, 8, 32):
            for d in (64, 128):
                assert P.pdakv_page_bytes(fmt, 16, hkv, d) == oracle.page_bytes(fmt, 16, hkv, d)


MIN_PPW = 2  # fewest pages a decode wave is given (one page pair)


@pytest.mark.parametrize("B,hkv,L", [(1, 8, 256), (1, 8, 2048), (64, 8, 8193), (8, 8, 32768),
                                     (32, 2, 4104), (8, 8, 8192), (3, 1, 0), (1, 32, 1),
                                     (256, 8, 131072)])
@pytest.mark.parametrize("D", [64, 128])
def test_decode_plan_is_consistent(P, B, hkv, L, D):
    items = B * hkv * -(-L // 16)
    for fmt in (P.KV_INT8_SYM, P.KV_16BIT, P.KV_INT8_STATIC):
        # one wave per SIMD (1,024 on 256 CUs) where a KV head's page block
        # holds 4 KB or more and that round holds the items at <= 128 each,
        # else two
        block = 16 * 2 * D * (2 if fmt == P.KV_16BIT else 1)
        resident = 1024 if block >= 4096 and items <= 1024 * 128 else 2048
        waves, ppw = P.pdakv_decode_plan(fmt, B, hkv, D, L)
        assert waves >= 4 and waves % 4 == 0
        assert MIN_PPW <= ppw <= 128 and ppw == max(MIN_PPW, -(-items // waves))
        # one resident round unless the items need more than 128 per wave;
        # never more waves than MIN_PPW-page shares (rounded to whole workgroups)
        want = min(max(resident, -(-items // 128)), -(-items // MIN_PPW))
        assert waves == max(4, -(-max(want, 1) // 4) * 4)


@pytest.mark.parametrize("B,hkv,L", [(1, 8, 2048), (64, 8, 8193), (8, 8, 32768), (3, 1, 1),
                                     (500, 2, 700), (8, 8, 0)])
def test_workspace_holds_every_plan(P, B, hkv, L):
    """The workspace holds the partial slots (wave + unit) of every format's
    plan, whichever format a call then decodes: it is sized with the most
    waves any of them plans (a workspace sized for fewer waves than a launch
    uses would be written past its end)."""
    wmax = max(P.pdakv_decode_plan(f, B, hkv, 128, L)[0]
               for f in (P.KV_INT8_SYM, P.KV_16BIT, P.KV_INT8_STATIC))
    ws = P.pdakv_decode_workspace_bytes(B, 4 * hkv, hkv, 128, L)
    partials = -(-(wmax + B * hkv) * 4 * 130 * 4 // 16) * 16
    # sized for two waves per SIMD (the kernels' occupancy), which no plan exceeds
    full = -(-(_plan_waves(2, B, hkv, L) + B * hkv) * 4 * 130 * 4 // 16) * 16
    assert ws == (0 if L == 0 else full + B * hkv * 8)
    assert ws == 0 or ws >= partials + B * hkv * 8


def test_decode_plan_rejects_bad_arguments(P):
    assert P._lib.pdakv_decode_plan(7, 1, 8, 128, 16, None, None) == P.ERR_INVALID_ARG
    assert P._lib.pdakv_decode_plan(P.KV_INT8_SYM, -1, 8, 128, 16, None, None) == P.ERR_INVALID_ARG
    assert P._lib.pdakv_decode_plan(P.KV_INT8_SYM, 1, 0, 128, 16, None, None) == P.ERR_INVALID_ARG
    assert P._lib.pdakv_decode_plan(P.KV_INT8_SYM, 1, 8, 96, 16, None, None) == P.ERR_UNSUPPORTED
    # more than 2^30 (sequence, KV head, page) items
    assert (P._lib.pdakv_decode_plan(P.KV_INT8_SYM, 4096, 64, 128, 1 << 17, None, None) ==
            P.ERR_UNSUPPORTED)


def test_capabilities_without_device(P):
    flags = ctypes.c_uint32(123)
    assert P._lib.pdakv_capabilities(None) == P.ERR_INVALID_ARG
    st = P._lib.pdakv_capabilities(ctypes.byref(flags))
    assert st in (P.OK, P.ERR_NO_DEVICE)


FAKE = 0x10000  # a non-null, 16-byte aligned pointer value that is never dereferenced


def _write_args(**kw):
    a = dict(k=FAKE, v=FAKE, dtype=1, T=4, hkv=8, d=128, kst=1024, ksh=128, ksd=1, vst=1024,
             vsh=128, vsd=1, slots=FAKE, pool=FAKE, nblk=4, bs=16, err=None, stream=None)
    a.update(kw)
    return list(a.values())


@pytest.mark.parametrize("fn", ["kv_quant_int8_sym_write", "kv_write_16bit"])
@pytest.mark.parametrize("change,status", [
    (dict(dtype=0), -3), (dict(dtype=5), -3), (dict(T=-1), -1), (dict(hkv=0), -1),
    (dict(d=96), -2), (dict(bs=32), -2), (dict(ksd=-1), -1), (dict(vst=-4), -1),
    (dict(k=None), -1), (dict(slots=None), -1), (dict(pool=FAKE + 4), -1),
    (dict(nblk=-1), -1), (dict(nblk=2 ** 28), -2), (dict(T=0, k=None), 0),
])
def test_write_validation(P, fn, change, status):
    assert getattr(P._lib, fn)(*_write_args(**change)) == status


def _decode_args(**kw):
    a = dict(out=FAKE, odt=0, oss=4096, osh=128, q=FAKE, qdt=1, qss=4096, qsh=128, pool=FAKE,
             nblk=16, bs=16, bt=FAKE, bts=16, ctx=FAKE, B=1, hq=32, hkv=8, d=128, maxL=256,
             sm=0.088, ws=None, wsb=0, err=None, stream=None)
    a.update(kw)
    return list(a.values())


@pytest.mark.parametrize("fn", ["paged_attn_decode_int8", "paged_attn_decode_fp16"])
@pytest.mark.parametrize("change,status", [
    (dict(qdt=0), -3), (dict(odt=9), -3), (dict(hq=30), -2), (dict(hq=8 * 17), -2),
    (dict(d=256), -2), (dict(bs=8), -2), (dict(bts=15), -1), (dict(maxL=-1), -1),
    (dict(B=-1), -1), (dict(q=None), -1), (dict(bt=None), -1), (dict(ctx=None), -1),
    (dict(out=None), -1), (dict(pool=FAKE + 8), -1), (dict(sm=float("nan")), -1),
    (dict(oss=-1), -1), (dict(maxL=2048, bts=128), -4),
    (dict(maxL=2048, bts=128, ws=FAKE, wsb=16), -4), (dict(B=0), 0),
    (dict(maxL=2048, bts=128, ws=FAKE + 8, wsb=1 << 30), -1),
    (dict(B=65536, maxL=32784, bts=2050), -2), (dict(nblk=0), -1), (dict(nblk=0, B=0), 0),
])
def test_decode_validation(P, fn, change, status):
    assert getattr(P._lib, fn)(*_decode_args(**change)) == status


def _append_args(**kw):
    a = dict(out=FAKE, odt=0, oss=4096, osh=128, q=FAKE, qdt=1, qss=4096, qsh=128, kn=FAKE,
             vn=FAKE, kst=1024, ksh=128, ksd=1, vst=1024, vsh=128, vsd=1, pool=FAKE, nblk=16,
             bs=16, bt=FAKE, bts=16, ctx=FAKE, B=1, hq=32, hkv=8, d=128, maxL=256, sm=0.088,
             ws=FAKE, wsb=1 << 30, err=None, stream=None)
    a.update(kw)
    return list(a.values())


@pytest.mark.parametrize("fn", ["paged_attn_decode_int8_append", "paged_attn_decode_fp16_append"])
@pytest.mark.parametrize("change,status", [
    (dict(kn=None), -1), (dict(vn=None), -1), (dict(ksd=-1), -1), (dict(vst=-2), -1),
    (dict(qdt=0), -3), (dict(d=96), -2), (dict(maxL=2048, bts=128, ws=None, wsb=0), -4),
    (dict(B=0), 0),
    (dict(B=0, kn=None, vn=None), 0),
])
def test_append_validation(P, fn, change, status):
    assert getattr(P._lib, fn)(*_append_args(**change)) == status


# ---- static scales --------------------------------------------------------

def _with_scales(args, at, ks=0.05, vs=0.07):
    return args[:at] + [ks, vs] + args[at:]


BAD_SCALES = [(0.0, 1.0), (1.0, 0.0), (-0.5, 1.0), (1.0, -2.0), (float("nan"), 1.0),
              (1.0, float("inf"))]


@pytest.mark.parametrize("change,status", [
    (dict(dtype=0), -3), (dict(d=96), -2), (dict(k=None), -1), (dict(pool=FAKE + 4), -1),
    (dict(T=0, k=None), 0),
])
def test_static_write_validation(P, change, status):
    assert P._lib.kv_quant_int8_static_write(*_with_scales(_write_args(**change), 12)) == status


@pytest.mark.parametrize("ks,vs", BAD_SCALES)
def test_static_write_rejects_bad_scales(P, ks, vs):
    assert P._lib.kv_quant_int8_static_write(*_with_scales(_write_args(), 12, ks, vs)) == -1


@pytest.mark.parametrize("change,status", [
    (dict(qdt=0), -3), (dict(hq=30), -2), (dict(d=256), -2), (dict(bts=15), -1),
    (dict(q=None), -1), (dict(pool=FAKE + 8), -1), (dict(maxL=2048, bts=128), -4),
    (dict(B=0), 0),
])
def test_static_decode_validation(P, change, status):
    assert P._lib.paged_attn_decode_int8_static(*_with_scales(_decode_args(**change), 20)) == status


@pytest.mark.parametrize("ks,vs", BAD_SCALES + [(3e38, 1.0)])
def test_static_decode_rejects_bad_scales(P, ks, vs):
    # (3e38 * sm_scale * log2(e) is beyond the float range: rejected too)
    args = _with_scales(_decode_args(sm=1.0, ws=FAKE, wsb=1 << 30), 20, ks, vs)
    assert P._lib.paged_attn_decode_int8_static(*args) == -1
    args = _with_scales(_append_args(sm=1.0), 28, ks, vs)
    assert P._lib.paged_attn_decode_int8_static_append(*args) == -1


@pytest.mark.parametrize("change,status", [
    (dict(kn=None), -1), (dict(ksd=-1), -1), (dict(qdt=0), -3),
    (dict(maxL=2048, bts=128, ws=None, wsb=0), -4), (dict(B=0, kn=None, vn=None), 0),
])
def test_static_append_validation(P, change, status):
    args = _with_scales(_append_args(**change), 28)
    assert P._lib.paged_attn_decode_int8_static_append(*args) == status


# ---- several query tokens ---------------------------------------------------

def _multi_args(**kw):
    a = dict(out=FAKE, odt=0, oss=4 * 4096, ost=4096, osh=128, q=FAKE, qdt=1, qss=4 * 4096,
             qst=4096, qsh=128, T=4, pool=FAKE, nblk=16, bs=16, bt=FAKE, bts=16, ctx=FAKE, B=1,
             hq=32, hkv=8, d=128, maxL=256, sm=0.088, ws=FAKE, wsb=1 << 30, err=None,
             stream=None)
    a.update(kw)
    return list(a.values())


@pytest.mark.parametrize("fn", ["paged_attn_decode_int8_multi", "paged_attn_decode_fp16_multi"])
@pytest.mark.parametrize("change,status", [
    (dict(T=0), -1), (dict(T=-2), -1), (dict(ost=-1), -1), (dict(qst=-8), -1), (dict(qdt=0), -3),
    (dict(hq=30), -2), (dict(d=96), -2), (dict(q=None), -1), (dict(ws=None, wsb=0), -4),
    (dict(ws=FAKE, wsb=64), -4), (dict(B=0), 0), (dict(ws=FAKE + 4), -1),
])
def test_multi_validation(P, fn, change, status):
    assert getattr(P._lib, fn)(*_multi_args(**change)) == status


def _plan_waves(waves_per_simd, B, heads, L):
    """The decode grid's wave count (256 CUs x 4 SIMDs resident per wave per
    SIMD; at most 128 and at least MIN_PPW items per wave; a multiple of 4)."""
    items = B * heads * -(-L // 16)
    v = max(256 * 4 * waves_per_simd, -(-items // 128))
    v = max(min(v, -(-items // MIN_PPW)), 1)
    return -(-v // 4) * 4


@pytest.mark.parametrize("B,T,hq,hkv,L", [(64, 1, 32, 8, 8193), (64, 4, 32, 8, 8193),
                                          (8, 8, 32, 8, 32768), (32, 3, 14, 2, 4104),
                                          (1, 16, 8, 8, 100), (3, 2, 16, 1, 40),
                                          (4, 128, 32, 8, 3000), (2, 256, 14, 2, 4000),
                                          (5, 11, 32, 8, 900)])
def test_multi_workspace_formula(P, B, T, hq, hkv, L):
    """Units of a KV head: its T * G query columns in tiles of 16, all of
    them in one unit up to 4 tiles, else units of 4. Workspace:
    [waves + B * units][min(T * G, 16 * tiles per unit)][D + 2] floats
    (16-byte padded), then B * units records; the waves are those of the
    INT8 plan with units as heads (two waves per SIMD up to two tiles per
    unit, one beyond). T = 1 is the one-token workspace."""
    G = hq // hkv
    cols = T * G
    tiles = -(-cols // 16)
    per_unit = min(tiles, 4)
    vh = hkv * -(-tiles // per_unit)
    waves = _plan_waves(2 if per_unit <= 2 else 1, B, vh, L)
    if per_unit == 1:  # the one-token plan never has more waves
        assert waves >= P.pdakv_decode_plan(P.KV_INT8_SYM, B, vh, 128, L)[0]
    partials = -(-(waves + B * vh) * min(cols, 16 * per_unit) * 130 * 4 // 16) * 16
    assert P.pdakv_decode_multi_workspace_bytes(B, T, hq, hkv, 128, L) == partials + B * vh * 8
    if T == 1:
        assert (P.pdakv_decode_multi_workspace_bytes(B, 1, hq, hkv, 128, L) ==
                P.pdakv_decode_workspace_bytes(B, hq, hkv, 128, L))
    assert P.pdakv_decode_multi_workspace_bytes(B, 0, hq, hkv, 128, L) == 0


# ---- page lifecycle ---------------------------------------------------------

def _swap_args(**kw):
    a = dict(pool=FAKE, nblk=16, pb=33280, ids=FAKE, n=4, dst=FAKE, err=None, stream=None)
    a.update(kw)
    return list(a.values())


@pytest.mark.parametrize("change,status", [
    (dict(pb=33281), -1), (dict(pb=0), -1), (dict(n=-1), -1), (dict(nblk=-1), -1),
    (dict(ids=None), -1), (dict(dst=None), -1), (dict(dst=FAKE + 8), -1),
    (dict(pool=FAKE + 4), -1), (dict(n=0, ids=None, dst=None), 0), (dict(n=1 << 31), -2),
])
def test_swap_validation(P, change, status):
    assert P._lib.kv_pages_swap_out(*_swap_args(**change)) == status
    a = dict(zip(["pool", "nblk", "pb", "ids", "n", "dst", "err", "stream"], _swap_args(**change)))
    assert P._lib.kv_pages_swap_in(a["dst"], a["n"], a["ids"], a["pool"], a["nblk"], a["pb"],
                                   None, None) == status


def _trim_args(**kw):
    a = dict(fmt=1, pool=FAKE, nblk=64, bs=16, hkv=8, d=128, bt=FAKE, bts=8, ctx=FAKE,
             trim=FAKE, B=2, keep=4, new=FAKE, err=None, stream=None)
    a.update(kw)
    return list(a.values())


@pytest.mark.parametrize("change,status", [
    (dict(fmt=0), -1), (dict(fmt=4), -1), (dict(keep=-1), -1), (dict(B=-1), -1),
    (dict(hkv=0), -1), (dict(d=96), -2), (dict(bs=32), -2), (dict(bts=-1), -1),
    (dict(trim=None), -1), (dict(new=None), -1), (dict(ctx=None), -1), (dict(pool=FAKE + 4), -1),
    (dict(B=0, pool=None), 0), (dict(nblk=1 << 28), -2),
])
def test_trim_validation(P, change, status):
    assert P._lib.kv_trim_keep_sink(*_trim_args(**change)) == status


# ---- the Python binding rejects wrong dtypes, devices, layouts and sizes ----
# (CPU tensors: every check runs before the library is called)

def _t(*shape, dtype=None):
    import torch
    return torch.zeros(shape, dtype=dtype or torch.float16)


def test_binding_rejects_a_wrong_slot_mapping_dtype(P):
    import torch
    k = _t(4, 8, 128)
    pool = _t(4, 33280, dtype=torch.uint8)
    with pytest.raises(ValueError, match="slot_mapping must be int32"):
        P.kv_quant_int8_sym_write(k, k, _t(4, dtype=torch.int64), pool, 4)
    with pytest.raises(ValueError, match="slot_mapping must be a GPU tensor"):
        P.kv_quant_int8_sym_write(k, k, _t(4, dtype=torch.int32), pool, 4)


def test_binding_rejects_wrong_table_and_length_dtypes(P):
    import torch
    q, out = _t(2, 32, 128), _t(2, 32, 128, dtype=torch.float32)
    pool = _t(4, 33280, dtype=torch.uint8)
    with pytest.raises(ValueError, match="block_tables must be int32"):
        P.paged_attn_decode_int8(out, q, pool, 4, _t(2, 4, dtype=torch.int64),
                                 _t(2, dtype=torch.int32), 8, 64, 0.088)
    with pytest.raises(ValueError, match="block_tables must be a GPU tensor"):
        P.paged_attn_decode_int8(out, q, pool, 4, _t(2, 4, dtype=torch.int32),
                                 _t(2, dtype=torch.int64), 8, 64, 0.088)
    with pytest.raises(ValueError, match="context_lens must be int32"):
        P.kv_trim_keep_sink(P.KV_INT8_SYM, pool, 4, 8, 128, _t(2, 4, dtype=torch.int32),
                            _t(2, dtype=torch.int64), _t(2, dtype=torch.int32), 4,
                            _t(2, dtype=torch.int32))
    with pytest.raises(ValueError, match="block_ids must be int32"):
        P.kv_pages_swap_out(pool, 4, _t(2, dtype=torch.int64), _t(2, 33280, dtype=torch.uint8))


def test_binding_checks_pools_and_tables(P):
    """Layout and size checks, with the dtype and device checks out of the way."""
    import torch
    from paged_decode_attention_kv_amd import _lib

    class Dev:  # a stand-in that passes the device checks
        def __init__(self, t):
            self.t = t
            self.is_cuda = True
            self.dtype, self.shape = t.dtype, t.shape

        def __getattr__(self, n):
            return getattr(self.t, n)

    bt = Dev(_t(4, 3, dtype=torch.int32).t())  # transposed: stride(1) != 1
    with pytest.raises(ValueError, match="unit stride"):
        _lib._need_block_tables(bt, 2)
    with pytest.raises(ValueError, match="rows"):
        _lib._need_block_tables(Dev(_t(1, 4, dtype=torch.int32)), 2)
    pool = Dev(_t(3, 33280, dtype=torch.uint8))
    with pytest.raises(ValueError, match="kv_pool holds"):
        _lib._need_pool(pool, 4, 33280)
    _lib._need_pool(pool, 3, 33280)
    with pytest.raises(ValueError, match="kv_pool holds"):
        _lib._need_pool(pool, 3, 0)
    with pytest.raises(ValueError, match="entries"):
        _lib._need_int32("context_lens", Dev(_t(1, dtype=torch.int32)), 2)


# ---- the decode entry point without a workspace -----------------------------

def _noalloc_args(**kw):
    a = _decode_args(**kw)
    return a[:20] + a[22:]  # no workspace, workspace_bytes


@pytest.mark.parametrize("change,status", [
    (dict(qdt=0), -3), (dict(hq=30), -2), (dict(d=96), -2), (dict(bts=15), -1),
    (dict(q=None), -1), (dict(pool=FAKE + 8), -1), (dict(B=0), 0),
    # a workspace beyond the 32 MiB scratch: refused before any device call
    (dict(B=512, maxL=32768, bts=2048), -4),
])
def test_noalloc_validation(P, change, status):
    assert P._lib.paged_attn_decode_int8_noalloc(*_noalloc_args(**change)) == status


def test_noalloc_scratch_size_is_the_header_constant(P):
    m = re.search(r"#define PDAKV_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", open(HEADER).read())
    assert m and int(m.group(1)) << int(m.group(2)) == P.NOALLOC_SCRATCH_BYTES
    # the batched step and the 32K workload fit; 512 sequences at 32K do not
    assert P.pdakv_decode_workspace_bytes(64, 32, 8, 128, 8193) <= P.NOALLOC_SCRATCH_BYTES
    assert P.pdakv_decode_workspace_bytes(8, 32, 8, 128, 32768) <= P.NOALLOC_SCRATCH_BYTES
    assert P.pdakv_decode_workspace_bytes(512, 32, 8, 128, 32768) > P.NOALLOC_SCRATCH_BYTES
