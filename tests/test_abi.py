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
        if name.startswith(("PA_OK", "PA_ERR_", "PA_KV_", "PA_VARIANT_")):
            assert getattr(pa, name) == value, name


def test_status_strings(lib):
    for code in range(0, -10, -1):
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


def _decode(lib, **kw):
    args = dict(q=A, k=A, v=A, bt=A, cl=A, scale=0.125, out=A, S=4, Hq=8, Hkv=2, D=64, bs=16, MB=7, N=32,
                kvd=1, ks=1.0, vs=1.0, ws=None, wsb=0, opts=pa._opts(partition_tokens=-1, schedule=-1))
    args.update(kw)
    o = args["opts"]
    return lib.pa_decode(args["q"], args["k"], args["v"], args["bt"], args["cl"], args["scale"], args["out"],
                         args["S"], args["Hq"], args["Hkv"], args["D"], args["bs"], args["MB"], args["N"],
                         args["kvd"], args["ks"], args["vs"], args["ws"], args["wsb"],
                         ctypes.byref(o) if o is not None else None, None)


def _reserved(v):
    o = pa._opts(partition_tokens=-1, schedule=-1)
    o.reserved = v
    return o


@pytest.mark.parametrize("kw,code", [
    (dict(D=96), -3), (dict(D=256), -3), (dict(Hq=6, Hkv=4), -2), (dict(Hq=2050, Hkv=2), -3), (dict(Hq=64, Hkv=2, opts=pa._opts(variant="valu")), -3),
    (dict(bs=8), -3), (dict(bs=24), -3), (dict(kvd=7), -5), (dict(MB=0), -2), (dict(S=-1), -2),
    (dict(N=0), -2), (dict(q=None), -1), (dict(bt=None), -1), (dict(out=A + 8), -4), (dict(k=A + 2), -4),
    (dict(kvd=2, ks=0.0), -5), (dict(kvd=2, vs=float("nan")), -5), (dict(scale=float("inf")), -2),
    (dict(opts=pa._opts(partition_tokens=24)), -2), (dict(opts=pa._opts(waves=3)), -2),
    (dict(opts=pa._opts(partition_tokens=32, schedule=-1)), -6), (dict(opts=pa._opts(prefetch=4)), -2),
    (dict(opts=pa._opts(prefetch=-1)), -2), (dict(Hq=16, Hkv=2, opts=pa._opts(variant="valu")), -3),
    (dict(opts=pa._opts(partition_tokens=32, schedule=-1), ws=A, wsb=16), -6),
    (dict(opts=pa._opts(partition_tokens=-1, schedule=1)), -6), (dict(opts=pa._opts(partition_tokens=-1, schedule=2)), -2),
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


def test_decode_zero_sequences_is_a_no_op(lib):
    assert _decode(lib, S=0, q=None, out=None) == 0


def _align(x, a=256):
    return -(-x // a) * a


def test_plan_with_explicit_partitions(lib):
    S, Hq, Hkv, D = 128, 32, 8, 128
    p = pa.pa_decode_get_plan(S, Hq, Hkv, D, 16, 256, partition_tokens=512, variant="valu", waves=4, schedule=-1)
    assert p["num_partitions"] == 8 and p["partition_tokens"] == 512 and not p["scheduled"]
    assert p["num_workgroups"] == S * Hkv * 8
    rows = S * Hq * 8
    assert p["workspace_bytes"] == _align(rows * 8) + rows * D * 4
    assert p["variant"] == "valu" and p["prefetch_tiles"] == 2
    # scheduled (the default when contexts are split): a 256-byte header and
    # the item list come first
    ps = pa.pa_decode_get_plan(S, Hq, Hkv, D, 16, 256, partition_tokens=512, variant="valu", waves=4)
    assert ps["scheduled"] and ps["num_workgroups"] == S * Hkv * 8
    assert ps["workspace_bytes"] == 256 + _align(S * Hkv * 8 * 16) + _align(rows * 8) + rows * D * 4
    p1 = pa.pa_decode_get_plan(4, 8, 2, 64, 16, 7, partition_tokens=-1, prefetch=3, schedule=-1)
    assert p1["num_partitions"] == 1 and p1["workspace_bytes"] == 0 and p1["prefetch_tiles"] == 3
    assert p1["variant"] == "mfma" and p1["partition_tokens"] == 112
    p1d = pa.pa_decode_get_plan(4, 8, 2, 64, 16, 7, partition_tokens=-1)
    assert not p1d["scheduled"] and p1d["workspace_bytes"] == 0
    p1s = pa.pa_decode_get_plan(4, 8, 2, 64, 16, 7, partition_tokens=-1, schedule=1)
    assert p1s["scheduled"] and p1s["workspace_bytes"] == 256 + _align(4 * 2 * 16)
    # a partition longer than the longest possible context is no split
    p2 = pa.pa_decode_get_plan(4, 8, 2, 64, 16, 7, partition_tokens=4096)
    assert p2["num_partitions"] == 1


def _cw(lib, **kw):
    args = dict(k=A, v=A, slots=A, kc=A, vc=A, T=4, Hkv=2, D=64, bs=16, N=32, kvd=1, ks=1.0, vs=1.0)
    args.update(kw)
    return lib.pa_cache_write(args["k"], args["v"], args["slots"], args["kc"], args["vc"], args["T"], args["Hkv"],
                              args["D"], args["bs"], args["N"], args["kvd"], args["ks"], args["vs"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(T=-1), -2), (dict(Hkv=0), -2), (dict(N=0), -2), (dict(kvd=3), -5), (dict(D=80), -3),
    (dict(bs=12), -3), (dict(k=None), -1), (dict(slots=None), -1), (dict(kc=A + 4), -4),
    (dict(slots=A + 4), -4), (dict(kvd=2, ks=-1.0), -5), (dict(kvd=2, vs=float("inf")), -5),
    (dict(T=1 << 62, Hkv=1 << 30, D=128), -3), (dict(T=(1 << 32) // 8 // 2, Hkv=2, D=64), -3),
])
def test_cache_write_rejects_bad_arguments(lib, kw, code):
    assert _cw(lib, **kw) == code


def test_cache_write_zero_tokens_is_a_no_op(lib):
    assert _cw(lib, T=0, k=None, v=None, slots=None) == 0


@pytest.mark.parametrize("args,code", [
    ((None, 4, 16, 32), -1), ((A, -1, 16, 32), -2), ((A, 4, 0, 32), -2), ((A, 4, 16, 0), -2),
    ((None, 0, 16, 32), 0),
])
def test_cache_write_check_argument_errors(lib, args, code):
    """The precondition check validates its own arguments before touching the device."""
    assert lib.pa_check_cache_write_inputs(*args, None) == code


@pytest.mark.parametrize("args,code", [
    ((None, A, 4, 16, 7, 32), -1), ((A, None, 4, 16, 7, 32), -1), ((A, A, -1, 16, 7, 32), -2),
    ((A, A, 4, 16, 0, 32), -2), ((A, A, 4, 16, 7, 0), -2), ((None, None, 0, 16, 7, 32), 0),
])
def test_decode_check_argument_errors(lib, args, code):
    assert lib.pa_check_decode_inputs(*args, None) == code


def _multi(lib, **kw):
    args = dict(q=A, k=A, v=A, bt=A, cl=A, qs=A, scale=0.125, out=A, S=4, Tq=10, maxq=4, Hq=8, Hkv=2, D=64,
                bs=16, MB=7, N=32, kvd=1, ks=1.0, vs=1.0, ws=None, wsb=0, part=-1)
    args.update(kw)
    return lib.pa_decode_multi(args["q"], args["k"], args["v"], args["bt"], args["cl"], args["qs"], args["scale"],
                               args["out"], args["S"], args["Tq"], args["maxq"], args["Hq"], args["Hkv"], args["D"],
                               args["bs"], args["MB"], args["N"], args["kvd"], args["ks"], args["vs"], args["ws"],
                               args["wsb"], args["part"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(D=96), -3), (dict(Hq=6, Hkv=4), -2), (dict(Tq=-1), -2), (dict(maxq=-2), -2), (dict(qs=None), -1),
    (dict(out=A + 8), -4), (dict(qs=A + 2), -4), (dict(kvd=2, ks=0.0), -5), (dict(part=24), -2),
    (dict(part=32), -6), (dict(part=32, ws=A + 16, wsb=1 << 24), -4), (dict(bs=8), -3), (dict(N=0), -2),
])
def test_multi_rejects_bad_arguments_without_launching(lib, kw, code):
    assert _multi(lib, **kw) == code


def test_multi_nothing_to_do_is_a_no_op(lib):
    assert _multi(lib, S=0, q=None, out=None) == 0
    assert _multi(lib, Tq=0, q=None, out=None) == 0


def test_multi_workspace_size(lib):
    """Unsplit: nothing. Split: header (item count) + the work list of
    (sequence, KV head, partition) items, then the split-K partials."""
    S, Tq, Hq, Hkv, D = 4, 10, 8, 2, 64
    assert pa.pa_decode_multi_workspace_size(S, Tq, 4, Hq, Hkv, D, 16, 7, partition_tokens=-1) == 0
    n = pa.pa_decode_multi_workspace_size(S, Tq, 4, Hq, Hkv, D, 16, 7, partition_tokens=32)
    P = -(-7 * 16 // 32)
    assert n == 256 + _align(S * Hkv * P * 16) + _align(Tq * Hq * P * 2 * 4) + Tq * Hq * P * D * 4


def _cascade(lib, **kw):
    args = dict(q=A, k=A, v=A, bt=A, cl=A, pt=None, pl=None, gs=None, scale=0.125, out=A, S=4, Hq=8, Hkv=2,
                D=64, bs=16, MB=7, N=32, G=0, maxg=0, PMB=1, kvd=1, ks=1.0, vs=1.0, ws=A, wsb=1 << 20,
                opts=pa._opts(partition_tokens=-1))
    args.update(kw)
    o = args["opts"]
    return lib.pa_decode_cascade(args["q"], args["k"], args["v"], args["bt"], args["cl"], args["pt"], args["pl"],
                                 args["gs"], args["scale"], args["out"], args["S"], args["Hq"], args["Hkv"],
                                 args["D"], args["bs"], args["MB"], args["N"], args["G"], args["maxg"],
                                 args["PMB"], args["kvd"], args["ks"], args["vs"], args["ws"], args["wsb"],
                                 ctypes.byref(o) if o is not None else None, None)


@pytest.mark.parametrize("kw,code", [
    (dict(G=-1), -2), (dict(maxg=-1), -2), (dict(PMB=-1), -2), (dict(Hq=64, Hkv=2), -3), (dict(D=96), -3),
    (dict(kvd=9), -5), (dict(N=0), -2), (dict(scale=float("nan")), -2), (dict(q=None), -1), (dict(cl=None), -1),
    (dict(out=A + 8), -4), (dict(bt=A + 2), -4), (dict(ws=None), -6), (dict(wsb=256), -6), (dict(ws=A + 16), -4),
    (dict(kvd=2, ks=-1.0), -5), (dict(PMB=1 << 27), -3), (dict(opts=pa._opts(partition_tokens=24)), -2),
])
def test_cascade_rejects_bad_arguments_without_launching(lib, kw, code):
    """Checks that precede the device query (no groups, or sizes already
    invalid); the group arrays' own checks run in the GPU tests."""
    assert _cascade(lib, **kw) == code


def test_cascade_zero_sequences_is_a_no_op(lib):
    assert _cascade(lib, S=0, q=None, out=None, ws=None, wsb=0) == 0


def test_cascade_workspace_without_groups(lib):
    """No groups: header + the suffix pass's work list + its partial states,
    which a cascade keeps even when contexts are not split."""
    S, Hq, Hkv, D, MB = 4, 8, 2, 64, 7
    units = Hkv // pa.pa_decode_get_plan(S, Hq, Hkv, D, 16, MB, partition_tokens=-1)["heads_per_tile"]
    n = pa.pa_decode_cascade_workspace_size(S, Hq, Hkv, D, 16, MB, 0, 0, 1, partition_tokens=-1)
    P = 1
    assert n == 256 + _align(S * units * P * 16) + _align(S * Hq * P * 2 * 4) + _align(S * Hq * P * D * 4)
    n2 = pa.pa_decode_cascade_workspace_size(S, Hq, Hkv, D, 16, MB, 0, 0, 1, partition_tokens=32)
    P = -(-MB * 16 // 32)
    assert n2 == 256 + _align(S * units * P * 16) + _align(S * Hq * P * 2 * 4) + _align(S * Hq * P * D * 4)
    assert pa.pa_decode_cascade_workspace_size(S, 64, 2, D, 16, MB, 0, 0, 1, partition_tokens=-1) == 0


@pytest.mark.parametrize("args,code", [
    ((None, None, None, 0, 0, 0, 4, 16, 32), 0), ((None, None, None, -1, 0, 0, 4, 16, 32), -2),
    ((None, None, None, 1, 1, 1, 4, 16, 32), -1), ((A, A, A, 1, 1, 1, 4, 0, 32), -2),
    ((A, A, A, 1, 1, 1, 4, 16, 0), -2),
])
def test_cascade_check_argument_errors(lib, args, code):
    assert lib.pa_check_cascade_inputs(*args, None) == code


def _copy(lib, **kw):
    args = dict(k=A, v=A, m=A, n=4, Hkv=2, D=64, bs=16, N=32, kvd=1)
    args.update(kw)
    return lib.pa_copy_blocks(args["k"], args["v"], args["m"], args["n"], args["Hkv"], args["D"], args["bs"],
                              args["N"], args["kvd"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(n=-1), -2), (dict(Hkv=0), -2), (dict(N=0), -2), (dict(kvd=5), -5), (dict(D=32), -3),
    (dict(bs=24), -3), (dict(k=None), -1), (dict(m=None), -1), (dict(v=A + 4), -4), (dict(m=A + 4), -4),
    (dict(n=1 << 31), -3), (dict(n=1 << 24), -3),
])
def test_copy_blocks_rejects_bad_arguments(lib, kw, code):
    assert _copy(lib, **kw) == code


def test_copy_blocks_zero_pairs_is_a_no_op(lib):
    assert _copy(lib, n=0, k=None, v=None, m=None) == 0


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
        pa.pa_decode_get_plan(S, Hq, Hkv, 64, 16, 7, **kw)
    assert e.value.status == -3


def test_split_plan_refuses_grids_beyond_32_bit_work_items(lib):
    # 2^24 sequences x 64 heads, 2 partitions: 2^31 decode workgroups, and
    # 2^30 merge rows of up to 512 threads each
    with pytest.raises(pa.PAError) as e:
        pa.pa_decode_get_plan(1 << 24, 64, 64, 64, 16, 8, partition_tokens=64, variant="mfma", heads_per_tile=1)
    assert e.value.status == -3
    # the largest grids that fit are still planned
    p = pa.pa_decode_get_plan(1 << 16, 8, 2, 64, 16, 7, partition_tokens=-1)
    assert p["num_workgroups"] * 64 * p["waves_per_group"] < 1 << 32
