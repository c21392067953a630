"""The C ABI without a GPU: exports, status strings, host-side checks and plans,
and the kernels' fp8 encoder (same source, built for the host) against the oracle."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import paged_kv_decode_mapping_amd as pa
from paged_kv_decode_mapping_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pa.h")


@pytest.fixture(scope="module")
def lib():
    # These tests pass fake device addresses that the library must reject
    # before launching anything; where a GPU is visible a check that let one
    # through would launch against it, so they run only without one.
    import torch
    if torch.cuda.is_available():
        pytest.skip("host-only ABI checks (fake device addresses): run where no GPU is visible")
    if not os.path.exists(pa.LIB_PATH):
        pytest.fail("libpa.so is not built (python -m paged_kv_decode_mapping_amd.build)")
    return pa.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pa_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_function_is_exported(lib):
    names = declared_functions()
    assert {"pa_cache_write", "pa_decode", "pa_decode_workspace_size", "pa_strerror"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_binding_constants_match_the_header():
    text = open(HEADER).read()
    defs = dict((n, int(v)) for n, v in re.findall(r"#define (PA_[A-Z0-9_]+)\s+\(?(-?\d+)\)?", text))
    assert len(defs) >= 14
    for name, value in defs.items():
        if name.startswith(("PA_OK", "PA_ERR_", "PA_DTYPE_", "PA_VARIANT_")):
            assert getattr(pa, name) == value, name


def test_status_strings(lib):
    for code in range(0, -12, -1):
        s = pa.strerror(code)
        assert s and s != "unknown status"
    assert pa.strerror(-99) == "unknown status"
    assert lib.pa_version() >= 100


def test_host_fp8_encoder_matches_oracle_on_all_bf16_values(lib):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    x = W.bf16_bits_to_f32(bits)
    got = pa.fp8_encode_host(x)
    want = oracle.f32_to_e4m3fn(x)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("scale", [1.0, 4.7 / 448, 0.0123, 3.0e-3, 17.0])
def test_host_fp8_quantiser_matches_oracle(lib, scale):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    with np.errstate(all="ignore"):
        y = W.bf16_bits_to_f32(bits) / np.float32(scale)  # IEEE float32 division
    assert np.array_equal(pa.fp8_encode_host(y), oracle.quantize_bf16(bits, scale))


# Fake, never-dereferenced device addresses for argument checks that must
# fail before anything is launched.
A = 0x10000
BF16, FP8, I32, I64 = pa.PA_DTYPE_BF16, pa.PA_DTYPE_FP8_E4M3FN, pa.PA_DTYPE_I32, pa.PA_DTYPE_I64


def T(shape, dtype=BF16, stride=None, data=A):
    """A pa_tensor at a fake address (contiguous unless strides are given)."""
    d = pa.desc(pa.TensorSpec(tuple(shape), dtype, None if stride is None else tuple(stride)))
    d.data = data
    return d


def _ref(d):
    return ctypes.byref(d) if d is not None else None


def _decode_args(S=4, Hq=8, Hkv=2, D=64, bs=16, MB=7, N=32, kvd=BF16):
    return dict(q=T((S, Hq, D)), k=T((N, bs, Hkv, D), kvd), v=T((N, bs, Hkv, D), kvd), bt=T((S, MB), I32),
                cl=T((S,), I32), scale=0.125, out=T((S, Hq, D)), ks=1.0, vs=1.0, ws=None, wsb=0,
                opts=pa._opts(partition_tokens=-1, schedule=-1))


def _decode(lib, **kw):
    sizes = {k: kw.pop(k) for k in ("S", "Hq", "Hkv", "D", "bs", "MB", "N", "kvd") if k in kw}
    args = _decode_args(**sizes)
    args.update(kw)
    o = args["opts"]
    return lib.pa_decode(_ref(args["q"]), _ref(args["k"]), _ref(args["v"]), _ref(args["bt"]), _ref(args["cl"]),
                         args["scale"], _ref(args["out"]), args["ks"], args["vs"], args["ws"], args["wsb"],
                         ctypes.byref(o) if o is not None else None, None)


def _reserved(v):
    o = pa._opts(partition_tokens=-1, schedule=-1)
    o.reserved = v
    return o


def _with(d, **kw):
    """A copy of descriptor d with fields replaced (data, dtype, ndim, shape, stride)."""
    e = pa.pa_tensor()
    ctypes.pointer(e)[0] = d
    for k, v in kw.items():
        if k in ("shape", "stride"):
            for i, x in enumerate(v):
                getattr(e, k)[i] = x
        else:
            setattr(e, k, v)
    return e


@pytest.mark.parametrize("kw,code", [
    (dict(D=96), -3), (dict(D=256), -3), (dict(Hq=6, Hkv=4), -2), (dict(Hq=2050, Hkv=2), -3),
    (dict(Hq=64, Hkv=2, opts=pa._opts(variant="valu")), -3),
    (dict(bs=8), -3), (dict(bs=24), -3), (dict(kvd=7), -5), (dict(MB=0), -2),
    (dict(N=0), -2), (dict(q=None), -1), (dict(bt=None), -1), (dict(kvd=2, ks=0.0), -5),
    (dict(kvd=2, vs=float("nan")), -5), (dict(scale=float("inf")), -2),
    (dict(opts=pa._opts(partition_tokens=24)), -2), (dict(opts=pa._opts(waves=3)), -2),
    (dict(opts=pa._opts(partition_tokens=32, schedule=-1)), -6), (dict(opts=pa._opts(prefetch=4)), -2),
    (dict(opts=pa._opts(prefetch=-1)), -2), (dict(Hq=16, Hkv=2, opts=pa._opts(variant="valu")), -3),
    (dict(opts=pa._opts(partition_tokens=32, schedule=-1), ws=A, wsb=16), -6),
    (dict(opts=pa._opts(partition_tokens=-1, schedule=1)), -6), (dict(opts=pa._opts(partition_tokens=-1, schedule=3)), -2),
    (dict(opts=pa._opts(partition_tokens=-1, schedule=1), ws=A + 16, wsb=1 << 20), -4),
    (dict(opts=_reserved(1)), -2), (dict(opts=_reserved(-1)), -2),
    (dict(opts=pa._opts(partition_tokens=-1, heads_per_tile=3)), -2),
    (dict(opts=pa._opts(partition_tokens=-1, heads_per_tile=8)), -2),
    (dict(Hkv=1, Hq=4, opts=pa._opts(partition_tokens=-1, variant="mfma", heads_per_tile=2)), -3),
    (dict(Hq=16, Hkv=2, opts=pa._opts(partition_tokens=-1, heads_per_tile=4)), -3),
    (dict(opts=pa._opts(partition_tokens=-1, variant="valu", heads_per_tile=2)), -3),
])
def test_decode_rejects_bad_arguments_without_launching(lib, kw, code):
    assert _decode(lib, **kw) == code


def test_decode_rejects_bad_tensors_without_launching(lib):
    a = _decode_args()
    cases = [
        ("q", _with(a["q"], data=A + 8), -4), ("out", _with(a["out"], data=A + 8), -4),
        ("k", _with(a["k"], data=A + 2), -4), ("bt", _with(a["bt"], data=A + 2), -4),
        ("cl", _with(a["cl"], data=A + 2), -4),
        ("q", _with(a["q"], data=None), -1), ("cl", _with(a["cl"], data=None), -1),
        ("q", _with(a["q"], dtype=I32), -5), ("k", _with(a["k"], dtype=I32), -5), ("bt", _with(a["bt"], dtype=I64), -5),
        ("cl", _with(a["cl"], dtype=I64), -5), ("v", _with(a["v"], dtype=FP8), -5), ("out", _with(a["out"], dtype=FP8), -5),
        ("q", _with(a["q"], ndim=2), -2), ("k", _with(a["k"], ndim=3), -2), ("bt", _with(a["bt"], ndim=1), -2),
        ("q", _with(a["q"], shape=(5, 8, 64)), -2), ("cl", _with(a["cl"], shape=(3,)), -2),
        ("out", _with(a["out"], shape=(3, 8, 64)), -2), ("v", _with(a["v"], shape=(31, 16, 2, 64)), -2),
        ("bt", _with(a["bt"], shape=(3, 7)), -2), ("q", _with(a["q"], shape=(4, 8, -1)), -2),
    ]
    for name, d, code in cases:
        assert _decode(lib, **{name: d}) == code, (name, code)


@pytest.mark.parametrize("name,stride,code", [
    ("q", (512, 64, 2), -10),            # innermost dimension not contiguous
    ("q", (512, 60, 1), -10),            # head stride not a multiple of 16 bytes
    ("q", (-512, 64, 1), -10),           # negative stride
    ("out", (512, 32, 1), -10),          # written rows overlap (heads 32 elements apart, 64 wide)
    ("out", (0, 64, 1), -10),            # every sequence writes the same row
    ("k", (2048, 64, 1024, 1), -10),     # head-major K with a standard V
    ("k", (2048, 64, 64, 1), -10),       # heads overlap
    ("k", (2048, 128, 64, 2), -10),
    ("k", (2048, 132, 64, 1), -10),      # token stride not a multiple of 16 bytes
    ("bt", (5, 1), -10),                 # table rows narrower than the table
    ("bt", (7, 2), -10),
    ("cl", (2,), -10),                   # 1-D index arrays contiguous
])
def test_decode_rejects_bad_strides(lib, name, stride, code):
    a = _decode_args()
    d = _with(a[name], stride=stride)
    # (2048, 64, 1024, 1) is a valid layout for K alone, but V keeps the
    # standard one: K and V must share it
    assert _decode(lib, **{name: d}) == code


def test_decode_accepts_strided_views_and_head_major_pools(lib):
    """Layouts the rules allow get a plan (the call fails only later, at the
    workspace it lacks): padded rows, a table row stride wider than the row,
    and a head-major pool [N, Hkv, bs, D] described as [N, bs, Hkv, D]."""
    N, bs, Hkv, D = 32, 16, 2, 64
    hm = pa.head_major_strides(N, bs, Hkv, D)
    opts = pa._opts(partition_tokens=32, schedule=1)  # needs a workspace: -6 means every check passed
    for kw in [dict(q=T((4, 8, 64), stride=(8 * 80, 80, 1))),
               dict(out=T((4, 8, 64), stride=(1024, 64, 1))),
               dict(bt=T((4, 7), I32, stride=(11, 1))),
               dict(k=T((N, bs, Hkv, D), stride=hm), v=T((N, bs, Hkv, D), stride=hm)),
               dict(k=T((N, bs, Hkv, D), stride=(bs * Hkv * 128, Hkv * 128, 128, 1)),
                    v=T((N, bs, Hkv, D), stride=(bs * Hkv * 128, Hkv * 128, 128, 1)))]:
        assert _decode(lib, opts=opts, **kw) == -6, kw
    # a head-major pool never packs two KV heads into one matrix tile
    q, kc, bt = pa.decode_specs(4, 16, 2, 64, 16, 7, head_major=True, num_blocks=32)
    assert pa.pa_decode_get_plan(q, kc, bt, partition_tokens=-1, variant="mfma")["heads_per_tile"] == 1
    q, kc, bt = pa.decode_specs(4, 16, 2, 64, 16, 7, num_blocks=32)
    assert pa.pa_decode_get_plan(q, kc, bt, partition_tokens=-1, variant="mfma")["heads_per_tile"] == 2
    with pytest.raises(pa.PAError) as e:
        q, kc, bt = pa.decode_specs(4, 16, 2, 64, 16, 7, head_major=True, num_blocks=32)
        pa.pa_decode_get_plan(q, kc, bt, partition_tokens=-1, variant="mfma", heads_per_tile=2)
    assert e.value.status == -3


def test_decode_zero_sequences_is_a_no_op(lib):
    a = _decode_args(S=0)
    assert _decode(lib, S=0, q=_with(a["q"], data=None), out=_with(a["out"], data=None)) == 0


def _align(x, a=256):
    return -(-x // a) * a


def _plan(S, Hq, Hkv, D, bs, MB, **kw):
    return pa.pa_decode_get_plan(*pa.decode_specs(S, Hq, Hkv, D, bs, MB, num_blocks=64), **kw)


def test_plan_with_explicit_partitions(lib):
    S, Hq, Hkv, D = 128, 32, 8, 128
    p = _plan(S, Hq, Hkv, D, 16, 256, partition_tokens=512, variant="valu", waves=4, schedule=-1)
    assert p["num_partitions"] == 8 and p["partition_tokens"] == 512 and not p["scheduled"]
    assert p["num_workgroups"] == S * Hkv * 8
    rows = S * Hq * 8
    assert p["workspace_bytes"] == _align(rows * 8) + rows * D * 4
    assert p["variant"] == "valu" and p["prefetch_tiles"] == 2
    # longest-first items (the default when contexts are split), found by
    # each workgroup when the grid is small (S * partitions <= 1024): no
    # list in the workspace
    ps = _plan(S, Hq, Hkv, D, 16, 256, partition_tokens=512, variant="valu", waves=4, schedule=2)
    assert ps["scheduled"] and ps["self_scheduled"] and ps["num_workgroups"] == S * Hkv * 8
    assert ps["workspace_bytes"] == _align(rows * 8) + rows * D * 4
    # the device-built list: a 256-byte header and the item list come first
    pl = _plan(S, Hq, Hkv, D, 16, 256, partition_tokens=512, variant="valu", waves=4, schedule=1)
    assert pl["scheduled"] and not pl["self_scheduled"] and pl["num_workgroups"] == S * Hkv * 8
    assert pl["workspace_bytes"] == 256 + _align(S * Hkv * 8 * 16) + _align(rows * 8) + rows * D * 4
    assert _plan(S, Hq, Hkv, D, 16, 256, partition_tokens=512, variant="valu", waves=4)["self_scheduled"]
    assert not _plan(S, Hq, Hkv, D, 16, 512, partition_tokens=512, variant="valu", waves=4)["self_scheduled"]
    # more sequences than one wave ranks: the list by default, and beyond
    # what a workgroup ranks, only the list
    assert _plan(256, Hq, Hkv, D, 16, 64, partition_tokens=256, variant="valu", waves=4)["self_scheduled"]
    p257 = _plan(257, Hq, Hkv, D, 16, 64, partition_tokens=256, variant="valu", waves=4)
    assert p257["scheduled"] and not p257["self_scheduled"]
    assert _plan(4096, Hq, Hkv, D, 16, 256, partition_tokens=512, variant="valu", waves=4,
                 schedule=2)["self_scheduled"]
    pb = _plan(4097, Hq, Hkv, D, 16, 256, partition_tokens=512, variant="valu", waves=4)
    assert pb["scheduled"] and not pb["self_scheduled"]
    with pytest.raises(pa.PAError) as e:
        _plan(4097, Hq, Hkv, D, 16, 256, partition_tokens=512, variant="valu", waves=4, schedule=2)
    assert e.value.status == pa.PA_ERR_UNSUPPORTED
    p1 = _plan(4, 8, 2, 64, 16, 7, partition_tokens=-1, prefetch=3, schedule=-1)
    assert p1["num_partitions"] == 1 and p1["workspace_bytes"] == 0 and p1["prefetch_tiles"] == 3
    assert p1["variant"] == "mfma" and p1["partition_tokens"] == 112
    p1d = _plan(4, 8, 2, 64, 16, 7, partition_tokens=-1)
    assert not p1d["scheduled"] and p1d["workspace_bytes"] == 0
    p1s = _plan(4, 8, 2, 64, 16, 7, partition_tokens=-1, schedule=1)
    assert p1s["scheduled"] and p1s["workspace_bytes"] == 256 + _align(4 * 2 * 16)
    p1t = _plan(4, 8, 2, 64, 16, 7, partition_tokens=-1, schedule=2)
    assert p1t["self_scheduled"] and p1t["workspace_bytes"] == 0
    # a partition longer than the longest possible context is no split
    p2 = _plan(4, 8, 2, 64, 16, 7, partition_tokens=4096)
    assert p2["num_partitions"] == 1
    assert pa.pa_decode_workspace_size(*pa.decode_specs(S, Hq, Hkv, D, 16, 256, num_blocks=64),
                                       partition_tokens=512, variant="valu", waves=4) == ps["workspace_bytes"]


def _cw_args(T_=4, Hkv=2, D=64, bs=16, N=32, kvd=BF16):
    return dict(k=T((T_, Hkv, D)), v=T((T_, Hkv, D)), slots=T((T_,), I64), kc=T((N, bs, Hkv, D), kvd),
                vc=T((N, bs, Hkv, D), kvd), ks=1.0, vs=1.0)


def _cw(lib, **kw):
    sizes = {k: kw.pop(k) for k in ("T_", "Hkv", "D", "bs", "N", "kvd") if k in kw}
    args = _cw_args(**sizes)
    args.update(kw)
    return lib.pa_cache_write(_ref(args["k"]), _ref(args["v"]), _ref(args["slots"]), _ref(args["kc"]),
                              _ref(args["vc"]), args["ks"], args["vs"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(N=0), -2), (dict(kvd=3), -5), (dict(D=80), -3),
    (dict(bs=12), -3), (dict(bs=8), -3), (dict(bs=2048), -3),  # the block sizes pa_decode reads: 16..1024
    (dict(k=None), -1), (dict(slots=None), -1),
    (dict(kvd=2, ks=-1.0), -5), (dict(kvd=2, vs=float("inf")), -5),
    (dict(T_=(1 << 32) // 8 // 2, Hkv=2, D=64), -3),
])
def test_cache_write_rejects_bad_arguments(lib, kw, code):
    assert _cw(lib, **kw) == code


def test_cache_write_rejects_bad_tensors(lib):
    a = _cw_args()
    cases = [
        ("kc", _with(a["kc"], data=A + 4), -4), ("slots", _with(a["slots"], data=A + 4), -4),
        ("k", _with(a["k"], data=A + 8), -4), ("slots", _with(a["slots"], dtype=I32), -5),
        ("k", _with(a["k"], shape=(4, 3, 64)), -2), ("v", _with(a["v"], shape=(5, 2, 64)), -2),
        ("kc", _with(a["kc"], stride=(2048, 64, 64, 1)), -10),   # cache rows overlap
        ("kc", _with(a["kc"], stride=(1024, 128, 64, 1)), -10),  # blocks overlap
        ("k", _with(a["k"], stride=(128, 64, 2)), -10), ("slots", _with(a["slots"], stride=(2,)), -10),
    ]
    for name, d, code in cases:
        assert _cw(lib, **{name: d}) == code, (name, code)
    hm = pa.head_major_strides(32, 16, 2, 64)
    assert _cw(lib, T_=0, k=_with(a["k"], data=None, shape=(0, 2, 64)), v=_with(a["v"], data=None, shape=(0, 2, 64)),
               slots=_with(a["slots"], data=None, shape=(0,)), kc=T((32, 16, 2, 64), stride=hm),
               vc=T((32, 16, 2, 64), stride=hm)) == 0


def test_cache_write_zero_tokens_is_a_no_op(lib):
    a = _cw_args(T_=0)
    assert _cw(lib, k=_with(a["k"], data=None), v=_with(a["v"], data=None), slots=_with(a["slots"], data=None)) == 0


def test_check_argument_errors(lib):
    """The precondition checks validate their own arguments before touching the device."""
    kc = T((32, 16, 2, 64))
    assert lib.pa_check_cache_write_inputs(None, _ref(kc), None) == -1
    assert lib.pa_check_cache_write_inputs(_ref(T((4,), I32)), _ref(kc), None) == -5
    assert lib.pa_check_cache_write_inputs(_ref(T((0,), I64, data=None)), _ref(kc), None) == 0
    assert lib.pa_check_cache_write_inputs(_ref(T((4,), I64)), _ref(T((0, 16, 2, 64))), None) == -2
    bt, cl = T((4, 7), I32), T((4,), I32)
    assert lib.pa_check_decode_inputs(None, _ref(cl), _ref(kc), None) == -1
    assert lib.pa_check_decode_inputs(_ref(bt), None, _ref(kc), None) == -1
    assert lib.pa_check_decode_inputs(_ref(bt), _ref(T((3,), I32)), _ref(kc), None) == -2
    assert lib.pa_check_decode_inputs(_ref(T((0, 7), I32, data=None)), _ref(T((0,), I32, data=None)), _ref(kc),
                                      None) == 0
    assert lib.pa_check_multi_inputs(_ref(bt), _ref(cl), _ref(T((4,), I32)), 4, _ref(kc), None) == -2
    assert lib.pa_check_multi_inputs(_ref(bt), _ref(cl), _ref(T((5,), I32)), -1, _ref(kc), None) == -2
    assert lib.pa_check_cascade_inputs(None, None, None, 0, 4, _ref(kc), None) == 0
    assert lib.pa_check_cascade_inputs(None, None, None, -1, 4, _ref(kc), None) == -2
    pt = T((1, 1), I32)
    assert lib.pa_check_cascade_inputs(_ref(pt), None, None, 1, 4, _ref(kc), None) == -1
    assert lib.pa_check_cascade_inputs(_ref(pt), _ref(T((2,), I32)), _ref(T((2,), I32)), 1, 4, _ref(kc), None) == -2


def _multi_args(S=4, Tq=10, Hq=8, Hkv=2, D=64, bs=16, MB=7, N=32, kvd=BF16):
    return dict(q=T((Tq, Hq, D)), k=T((N, bs, Hkv, D), kvd), v=T((N, bs, Hkv, D), kvd), bt=T((S, MB), I32),
                cl=T((S,), I32), qs=T((S + 1,), I32), scale=0.125, out=T((Tq, Hq, D)), maxq=4, ks=1.0, vs=1.0,
                ws=None, wsb=0, part=-1)


def _multi(lib, **kw):
    sizes = {k: kw.pop(k) for k in ("S", "Tq", "Hq", "Hkv", "D", "bs", "MB", "N", "kvd") if k in kw}
    args = _multi_args(**sizes)
    args.update(kw)
    r = lambda n: _ref(args[n])
    return lib.pa_decode_multi(r("q"), r("k"), r("v"), r("bt"), r("cl"), r("qs"), args["scale"], r("out"),
                               args["maxq"], args["ks"], args["vs"], args["ws"], args["wsb"], args["part"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(D=96), -3), (dict(Hq=6, Hkv=4), -2), (dict(maxq=-2), -2), (dict(qs=None), -1),
    (dict(kvd=2, ks=0.0), -5), (dict(part=24), -2),
    (dict(part=32), -6), (dict(part=32, ws=A + 16, wsb=1 << 24), -4), (dict(bs=8), -3), (dict(N=0), -2),
])
def test_multi_rejects_bad_arguments_without_launching(lib, kw, code):
    assert _multi(lib, **kw) == code


def test_multi_rejects_bad_tensors(lib):
    a = _multi_args()
    for name, d, code in [("out", _with(a["out"], data=A + 8), -4), ("qs", _with(a["qs"], data=A + 2), -4),
                          ("qs", _with(a["qs"], shape=(4,)), -2), ("out", _with(a["out"], shape=(9, 8, 64)), -2),
                          ("out", _with(a["out"], stride=(512, 0, 1)), -10)]:
        assert _multi(lib, **{name: d}) == code, (name, code)


def test_multi_nothing_to_do_is_a_no_op(lib):
    assert _multi(lib, S=0) == 0  # no sequences: nothing launched, whatever the query rows hold
    a = _multi_args(Tq=0)
    assert _multi(lib, Tq=0, q=_with(a["q"], data=None), out=_with(a["out"], data=None)) == 0


def test_multi_workspace_size(lib):
    """Unsplit: nothing. Split: the split-K partials, after a header (item
    count) and the work list of (sequence, KV head, partition) items when
    the batch is too large for the workgroups to rank their items
    themselves (more than 256 sequences)."""
    S, Tq, Hq, Hkv, D = 4, 10, 8, 2, 64
    q, kc, bt = pa.TensorSpec((Tq, Hq, D), BF16), pa.TensorSpec((32, 16, Hkv, D), BF16), pa.TensorSpec((S, 7), I32)
    assert pa.pa_decode_multi_workspace_size(q, kc, bt, 4, partition_tokens=-1) == 0
    n = pa.pa_decode_multi_workspace_size(q, kc, bt, 4, partition_tokens=32)
    P = -(-7 * 16 // 32)
    assert n == _align(Tq * Hq * P * 2 * 4) + Tq * Hq * P * D * 4
    S, Tq = 300, 600
    q, bt = pa.TensorSpec((Tq, Hq, D), BF16), pa.TensorSpec((S, 7), I32)
    n = pa.pa_decode_multi_workspace_size(q, kc, bt, 4, partition_tokens=32)
    assert n == 256 + _align(S * Hkv * P * 16) + _align(Tq * Hq * P * 2 * 4) + Tq * Hq * P * D * 4


def _cascade_args(S=4, Hq=8, Hkv=2, D=64, bs=16, MB=7, N=32, kvd=BF16):
    return dict(q=T((S, Hq, D)), k=T((N, bs, Hkv, D), kvd), v=T((N, bs, Hkv, D), kvd), bt=T((S, MB), I32),
                cl=T((S,), I32), pt=None, pl=None, gs=None, scale=0.125, out=T((S, Hq, D)), maxg=0, ks=1.0,
                vs=1.0, ws=A, wsb=1 << 20, opts=pa._opts(partition_tokens=-1))


def _cascade(lib, **kw):
    sizes = {k: kw.pop(k) for k in ("S", "Hq", "Hkv", "D", "bs", "MB", "N", "kvd") if k in kw}
    args = _cascade_args(**sizes)
    args.update(kw)
    r = lambda n: _ref(args[n])
    o = args["opts"]
    return lib.pa_decode_cascade(r("q"), r("k"), r("v"), r("bt"), r("cl"), r("pt"), r("pl"), r("gs"),
                                 args["scale"], r("out"), args["maxg"], args["ks"], args["vs"], args["ws"],
                                 args["wsb"], ctypes.byref(o) if o is not None else None, None)


@pytest.mark.parametrize("kw,code", [
    (dict(maxg=-1, pt=T((1, 1), I32), pl=T((1,), I32), gs=T((2,), I32)), -2),
    (dict(pt=T((1, 1 << 27), I32), pl=T((1,), I32), gs=T((2,), I32), maxg=1), -3),
    (dict(pt=T((2, 1), I32), pl=T((1,), I32), gs=T((3,), I32), maxg=1), -2),
    (dict(pt=T((1, 1), I32), pl=T((1,), I32), gs=T((1,), I32), maxg=1), -2),
    (dict(Hq=64, Hkv=2), -3), (dict(D=96), -3),
    (dict(kvd=9), -5), (dict(N=0), -2), (dict(scale=float("nan")), -2), (dict(q=None), -1), (dict(cl=None), -1),
    (dict(ws=None), -6), (dict(wsb=256), -6), (dict(ws=A + 16), -4),
    (dict(kvd=2, ks=-1.0), -5), (dict(opts=pa._opts(partition_tokens=24)), -2),
])
def test_cascade_rejects_bad_arguments_without_launching(lib, kw, code):
    """Checks that precede the device query (no groups, or sizes already
    invalid); the group arrays' own checks run in the GPU tests."""
    assert _cascade(lib, **kw) == code


def test_cascade_zero_sequences_is_a_no_op(lib):
    a = _cascade_args(S=0)
    assert _cascade(lib, S=0, q=_with(a["q"], data=None), out=_with(a["out"], data=None), ws=None, wsb=0) == 0


def test_cascade_workspace_without_groups(lib):
    """No groups: header + the suffix pass's work list + its partial states,
    which a cascade keeps even when contexts are not split."""
    S, Hq, Hkv, D, MB = 4, 8, 2, 64, 7
    specs = pa.decode_specs(S, Hq, Hkv, D, 16, MB, num_blocks=32)
    units = Hkv // pa.pa_decode_get_plan(*specs, partition_tokens=-1)["heads_per_tile"]
    n = pa.pa_decode_cascade_workspace_size(*specs, None, 0, partition_tokens=-1)
    P = 1
    assert n == 256 + _align(S * units * P * 16) + _align(S * Hq * P * 2 * 4) + _align(S * Hq * P * D * 4)
    n2 = pa.pa_decode_cascade_workspace_size(*specs, None, 0, partition_tokens=32)
    P = -(-MB * 16 // 32)
    assert n2 == 256 + _align(S * units * P * 16) + _align(S * Hq * P * 2 * 4) + _align(S * Hq * P * D * 4)
    wide = pa.decode_specs(S, 64, 2, D, 16, MB, num_blocks=32)
    assert pa.pa_decode_cascade_workspace_size(*wide, None, 0, partition_tokens=-1) == 0


def _copy(lib, **kw):
    sizes = {k: kw.pop(k) for k in ("n", "Hkv", "D", "bs", "N", "kvd") if k in kw}
    n, Hkv, D, bs, N, kvd = (sizes.get(k, v) for k, v in (("n", 4), ("Hkv", 2), ("D", 64), ("bs", 16), ("N", 32),
                                                          ("kvd", BF16)))
    args = dict(k=T((N, bs, Hkv, D), kvd), v=T((N, bs, Hkv, D), kvd), m=T((n, 2), I64))
    args.update(kw)
    return lib.pa_copy_blocks(_ref(args["k"]), _ref(args["v"]), _ref(args["m"]), None)


@pytest.mark.parametrize("kw,code", [
    (dict(N=0), -2), (dict(kvd=5), -5), (dict(D=32), -3),
    (dict(bs=24), -3), (dict(k=None), -1), (dict(m=None), -1), (dict(v=T((32, 16, 2, 64), data=A + 4)), -4),
    (dict(m=T((4, 2), I64, data=A + 4)), -4), (dict(m=T((4, 3), I64)), -2), (dict(m=T((4, 2), I32)), -5),
    (dict(m=T((4, 2), I64, stride=(4, 1))), -10),
    (dict(n=1 << 31), -3), (dict(n=1 << 24), -3),
    # blocks that are not one dense range: padded rows
    (dict(k=T((32, 16, 2, 64), stride=(16 * 256, 256, 64, 1)), v=T((32, 16, 2, 64), stride=(16 * 256, 256, 64, 1))), -10),
])
def test_copy_blocks_rejects_bad_arguments(lib, kw, code):
    assert _copy(lib, **kw) == code


def test_copy_blocks_zero_pairs_is_a_no_op(lib):
    hm = pa.head_major_strides(32, 16, 2, 64)  # head-major blocks are dense ranges too
    assert _copy(lib, n=0, m=T((0, 2), I64, data=None), k=T((32, 16, 2, 64), stride=hm),
                 v=T((32, 16, 2, 64), stride=hm)) == 0


@pytest.mark.parametrize("args,code", [
    ((A, 24, 1, A), -2), ((A, -16, 1, A), -2), ((None, 32, 1, A), -1), ((A, 32, 0, None), -1),
    ((A + 8, 32, 1, A), -4), ((A, 32, 1, A + 2), -4), ((None, 0, 1, None), 0),
])
def test_probe_rejects_bad_arguments(lib, args, code):
    assert lib.pa_probe_stream_read(*args, None) == code


@pytest.mark.parametrize("S,Hq,Hkv,kw", [
    (1 << 22, 8, 8, dict()),                       # VALU, 8 waves: 2^25 workgroups x 512 threads
    (1 << 23, 32, 8, dict(heads_per_tile=2)),      # MFMA, 4 waves: 2^25 x 256
    (1 << 20, 4096, 4, dict(partition_tokens=-1)),  # MQA-like groups on the multi-row kernel
])
def test_plans_refuse_grids_beyond_32_bit_work_items(lib, S, Hq, Hkv, kw):
    """A dispatch counts work-items in 32 bits: such plans are refused before
    any launch instead of wrapping."""
    kw = dict(dict(partition_tokens=-1), **kw)
    with pytest.raises(pa.PAError) as e:
        _plan(S, Hq, Hkv, 64, 16, 7, **kw)
    assert e.value.status == -3


def test_split_plan_refuses_grids_beyond_32_bit_work_items(lib):
    # 2^24 sequences x 64 heads, 2 partitions: 2^31 decode workgroups, and
    # 2^30 merge rows of up to 512 threads each
    with pytest.raises(pa.PAError) as e:
        _plan(1 << 24, 64, 64, 64, 16, 8, partition_tokens=64, variant="mfma", heads_per_tile=1)
    assert e.value.status == -3
    # the largest grids that fit are still planned
    p = _plan(1 << 16, 8, 2, 64, 16, 7, partition_tokens=-1)
    assert p["num_workgroups"] * 64 * p["waves_per_group"] < 1 << 32
