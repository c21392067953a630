"""GPU parity of pa_decode_cascade (shared-prefix decode) against the oracle.

The oracle is the plain decode definition gathered through the table that
the cascade's reading rule composes (oracle.cascade_decode): group members
take their prefix tokens from the group's prefix table, everything else
from their own rows. In most cases here the members' own rows name a NaN
block where the prefix lies, so an output is finite and right only if the
kernels read the prefix through the prefix table. Tolerances as for
pa_decode: max 1e-2 / mean 1e-3 (bf16 KV), 5e-2 / 5e-3 (fp8 KV).
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_decode_mapping_amd as pa
from paged_kv_decode_mapping_amd import workloads as W

from _gpu_util import DeviceWorkload, compare, dev_bf16, dev_u8, host_bits, note

pytestmark = pytest.mark.gpu

BF16_TOL = (1e-2, 1e-3)
FP8_TOL = (5e-2, 5e-3)


@pytest.fixture(scope="module")
def lib(gpu):
    return pa.load_library()


def _poison_member_prefix(b):
    """Members' own rows name the poison block where their prefix lies."""
    t = b.block_tables.copy()
    for k in range(b.num_groups):
        nb = int(b.prefix_lens[k]) // b.block_size
        t[b.group_start[k]:b.group_start[k + 1], :nb] = b.poison_block
    return t


class DeviceCascade:
    def __init__(self, b, tables=None, fp8_scales=None):
        self.b = b
        self.fp8 = fp8_scales is not None
        kc, vc = b.k_cache, b.v_cache
        if self.fp8:
            self.ks, self.vs = fp8_scales
            kc, vc = oracle.quantize_pool(kc, self.ks), oracle.quantize_pool(vc, self.vs)
        else:
            self.ks = self.vs = 1.0
        self.kc_host, self.vc_host = kc, vc
        self.tables_host = b.block_tables if tables is None else tables
        self.q = dev_bf16(b.q)
        self.k_cache = dev_u8(kc) if self.fp8 else dev_bf16(kc)
        self.v_cache = dev_u8(vc) if self.fp8 else dev_bf16(vc)
        self.block_tables = torch.from_numpy(np.ascontiguousarray(self.tables_host)).cuda()
        self.context_lens = torch.from_numpy(b.context_lens).cuda()
        self.prefix_tables = torch.from_numpy(b.prefix_tables).cuda()
        self.prefix_lens = torch.from_numpy(b.prefix_lens).cuda()
        self.group_start = torch.from_numpy(b.group_start).cuda()

    def cascade(self, max_group_size=None, partition_tokens=0):
        """One call on a workspace filled with NaN bytes, so that a state the
        merge reads but no pass wrote shows up in the output."""
        b = self.b
        mg = b.max_group_size if max_group_size is None else max_group_size
        need = pa.pa_decode_cascade_workspace_size(self.q, self.k_cache, self.block_tables, self.prefix_tables, mg,
                                                   partition_tokens=partition_tokens)
        assert need > 0
        ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")
        return pa.pa_decode_cascade(self.q, self.k_cache, self.v_cache, self.block_tables, self.context_lens,
                                    self.prefix_tables, self.prefix_lens, self.group_start, b.scale,
                                    max_group_size=mg, k_scale=self.ks, v_scale=self.vs, workspace=ws,
                                    partition_tokens=partition_tokens)

    def reference(self, max_group_size=None, units=None):
        b = self.b
        return oracle.cascade_decode(b.q, self.kc_host, self.vc_host, self.tables_host, b.context_lens,
                                     b.prefix_tables, b.prefix_lens, b.group_start, b.scale,
                                     max_group_size=max_group_size or b.max_group_size, units=units,
                                     kv_dtype=oracle.KV_FP8_E4M3FN if self.fp8 else oracle.KV_BF16,
                                     k_scale=self.ks, v_scale=self.vs)


GROUPS = [(64, [64, 100, 30, 200, 0]), (160, [500, 160, 1]), (32, []), (0, [50, 0]), (48, [49, 17, 300])]
LEAD, TAIL = [5, 0], [17, 300, 1]

SHAPES = [  # (Hq, Hkv, D): VALU g = 1, 2; MFMA g = 4; two KV heads per tile at g = 8; D 64 and 128
    (4, 4, 64), (8, 4, 128), (8, 2, 64), (32, 8, 128), (16, 2, 128),
]


@pytest.mark.parametrize("Hq,Hkv,D", SHAPES)
@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_cascade_groups_agree_with_oracle(lib, Hq, Hkv, D, kv):
    b = W.make_prefix_groups(num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, block_size=16, groups=GROUPS,
                             lead=LEAD, tail=TAIL, seed=11)
    scales = None
    if kv == "fp8":
        amax = lambda x: float(np.abs(W.bf16_bits_to_f32(x[np.isfinite(W.bf16_bits_to_f32(x))])).max())
        scales = (float(np.float32(amax(b.k_cache)) / np.float32(448.0)),
                  float(np.float32(amax(b.v_cache)) / np.float32(448.0)))
    d = DeviceCascade(b, tables=_poison_member_prefix(b), fp8_scales=scales)
    ref = d.reference()
    tol = FP8_TOL if kv == "fp8" else BF16_TOL
    for part in (0, -1, 48):
        note(f"cascade Hq={Hq} Hkv={Hkv} D={D} kv={kv} partition={part}")
        got = host_bits(d.cascade(partition_tokens=part))
        compare(got, ref, *tol)
        assert np.all(got[[1, 6, 11]] == 0)  # empty contexts: one ungrouped, two members


def test_cascade_large_groups_and_many_groups(lib):
    """A group wider than one workgroup's rows (40 members x 4 heads: two row
    blocks of 8 waves), and 64 small groups (enough workgroups that the prefix
    is not split), against the oracle."""
    big = W.make_prefix_groups(num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
                               groups=[(96, list(range(1, 400, 10)))], tail=[33, 2], seed=12)
    many = W.make_prefix_groups(num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
                                groups=[(32, [40 + k, 20 + 3 * k]) for k in range(64)], seed=13)
    for name, b in (("one group of 40", big), ("64 groups", many)):
        d = DeviceCascade(b, tables=_poison_member_prefix(b))
        note(f"cascade {name}")
        compare(host_bits(d.cascade()), d.reference(), *BF16_TOL)


def test_cascade_group_size_cap_and_block_size_128(lib):
    """max_group_size below a group's size: its later members read through
    their own rows (intact here); block size 128 with a 256-token prefix."""
    b = W.make_prefix_groups(num_q_heads=8, num_kv_heads=2, head_dim=128, block_size=128,
                             groups=[(256, [300, 256, 100, 700, 1000])], lead=[129], seed=14)
    d = DeviceCascade(b)
    for cap in (5, 3, 1):
        note(f"cascade max_group_size={cap} bs=128")
        compare(host_bits(d.cascade(max_group_size=cap)), d.reference(max_group_size=cap), *BF16_TOL)


def test_cascade_equals_decode_on_the_mixed_batch(lib):
    """The mixed batch (half the sequences share a 512-token prefix), reduced,
    reordered with its sharers first: the cascade agrees with the oracle and
    with pa_decode on the same batch."""
    w = W.make_workload("mixed_batch", num_seqs=24,
                        context=("list", [16, 100, 511, 512, 513, 900, 3000, 40, 8192, 77, 600, 1,
                                          2000, 520, 64, 1500, 700, 33, 5000, 528, 256, 1024, 4097, 2]))
    b = W.cascade_batch(w)
    d = DeviceCascade(b)
    ref = d.reference()
    for part in (0, 512):
        note(f"cascade mixed_batch reduced partition={part}")
        got = host_bits(d.cascade(partition_tokens=part))
        compare(got, ref, *BF16_TOL)
        plain = host_bits(pa.pa_decode(d.q, d.k_cache, d.v_cache, d.block_tables, d.context_lens, b.scale,
                                       partition_tokens=part))
        compare(plain, ref, *BF16_TOL)


@pytest.mark.parametrize("name", ["mixed_batch", "system_prompt"])
def test_cascade_full_size_sampled(lib, name):
    """Full size, in the launch configuration the benchmark times: the mixed
    batch (256 sequences, 128 sharing a 512-token prefix) and the system
    prompt batch (128 sequences sharing 4096 tokens); sampled (sequence, KV
    head) units against the oracle, every element against pa_decode."""
    w = W.make_workload(name)
    b = W.cascade_batch(w)
    d = DeviceCascade(b)
    note(f"cascade full-size {name}")
    got = host_bits(d.cascade())
    plain = host_bits(pa.pa_decode(d.q, d.k_cache, d.v_cache, d.block_tables, d.context_lens, b.scale))
    Hkv, g = w.spec.num_kv_heads, w.spec.group
    n_shared = int(b.group_start[1])
    ctx = b.context_lens
    rng = np.random.default_rng(21)
    pick = [0, n_shared - 1, min(n_shared, len(ctx) - 1), int(np.argmax(ctx)), int(np.argmin(ctx[:n_shared])),
            int(np.argmax(ctx[:n_shared]))]
    seqs = np.unique(np.concatenate([pick, rng.choice(len(ctx), 10, replace=False)]))
    units = np.concatenate([seqs * Hkv + rng.integers(0, Hkv, len(seqs)), seqs[:4] * Hkv + Hkv - 1])
    units = np.unique(units)
    ref = d.reference(units=units)
    sel = np.stack([got[u // Hkv, (u % Hkv) * g:(u % Hkv + 1) * g] for u in units])
    compare(sel, ref, *BF16_TOL)
    diff = np.abs(W.bf16_bits_to_f32(got).astype(np.float64) - W.bf16_bits_to_f32(plain))
    assert np.isfinite(diff).all() and diff.max() <= 1e-2 and diff.mean() <= 1e-3


def test_cascade_no_groups_is_a_plain_decode(lib):
    w = W.make_workload("tiny")
    d = DeviceWorkload(w)
    e = torch.zeros((0,), dtype=torch.int32, device="cuda")
    note("cascade without groups")
    got = pa.pa_decode_cascade(d.q, d.k_cache, d.v_cache, d.block_tables, d.context_lens,
                               torch.zeros((0, 1), dtype=torch.int32, device="cuda"), e,
                               torch.zeros((1,), dtype=torch.int32, device="cuda"), w.scale, max_group_size=0)
    compare(host_bits(got), oracle.decode_workload(w), *BF16_TOL)


def test_cascade_argument_errors_and_checks(lib):
    b = W.make_prefix_groups(num_q_heads=8, num_kv_heads=2, head_dim=64, block_size=16,
                             groups=[(32, [40, 50]), (16, [20])], lead=[3], seed=15)
    d = DeviceCascade(b)
    note("cascade argument errors")
    S, Hq, D = b.q.shape
    ws = torch.empty(1 << 22, dtype=torch.uint8, device="cuda")
    out = torch.empty_like(d.q)
    tensors = [d.q, d.k_cache, d.v_cache, d.block_tables, d.context_lens, d.prefix_tables, d.prefix_lens,
               d.group_start]
    o = pa._opts(partition_tokens=-1)

    def call(descs=None, ws_ptr=ws.data_ptr(), ws_bytes=1 << 22):
        ds = [pa.desc(t) for t in tensors] if descs is None else descs
        return lib.pa_decode_cascade(*map(pa._ref, ds), b.scale, pa._ref(pa.desc(out)), b.max_group_size, 1.0, 1.0,
                                     ws_ptr, ws_bytes, pa.ctypes.byref(o), None)

    for i in (6, 7):  # with prefix tables, the other two group arrays are required
        ds = [pa.desc(t) for t in tensors]
        ds[i].data = None
        assert call(ds) == pa.PA_ERR_NULL
        ds[i].data = tensors[i].data_ptr() + 2
        assert call(ds) == pa.PA_ERR_ALIGN
    ds = [pa.desc(t) for t in tensors]
    ds[5].data = tensors[5].data_ptr() + 2
    assert call(ds) == pa.PA_ERR_ALIGN
    assert call(ws_bytes=256) == pa.PA_ERR_WORKSPACE
    assert call(ws_ptr=None) == pa.PA_ERR_WORKSPACE
    assert call(ws_ptr=ws.data_ptr() + 16) == pa.PA_ERR_ALIGN
    torch.cuda.synchronize()
    # the opt-in checks of the group arrays
    t = lambda a: torch.from_numpy(np.asarray(a, np.int32)).cuda()
    N, pt = b.num_blocks, d.prefix_tables
    assert pa.pa_check_cascade_inputs(pt, d.prefix_lens, d.group_start, 2, S, d.k_cache) == pa.PA_OK
    bad_table = b.prefix_tables.copy()
    bad_table[1, 0] = N
    cases = {
        "partial block": (pt, t([32, 8]), d.group_start, 2),
        "past the table row": (pt, t([48, 16]), d.group_start, 2),
        "falling offsets": (pt, d.prefix_lens, t([1, 3, 2]), 2),
        "past the batch": (pt, d.prefix_lens, t([1, 3, S + 1]), 3),
        "group too large": (pt, d.prefix_lens, d.group_start, 1),
        "entry past the pool": (t(bad_table), d.prefix_lens, d.group_start, 2),
    }
    for what, (a, l, s, mg) in cases.items():
        note(f"cascade check: {what}")
        assert pa.pa_check_cascade_inputs(a, l, s, mg, S, d.k_cache) == pa.PA_ERR_PRECONDITION, what
