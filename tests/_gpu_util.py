"""Helpers for the GPU tests: move a generated workload to the device and
compare a bf16 device output with the float64 oracle."""
import sys

import numpy as np
import torch

import paged_kv_decode_mapping_amd as pa


def note(msg: str) -> None:
    """Name the case before a GPU step (flushed, so it survives a lost box)."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def dev_u8(codes: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(codes)).cuda()


def host_bits(t: torch.Tensor) -> np.ndarray:
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# Reduced copies of the named workloads: a few sequences, several tiles and
# partitions, ragged tails.
REDUCED = {
    "tiny": dict(),
    "llama7b_mha": dict(num_seqs=3, context=("list", [512, 1000, 2048])),
    "llama70b_gqa": dict(num_seqs=2, context=("list", [4096, 1234])),
    "long_splitk": dict(num_seqs=2, context=("list", [5000, 2049])),
    "mixed_batch": dict(num_seqs=10, context=("list", [16, 100, 511, 512, 513, 900, 3000, 40, 8192, 77])),
}


def head_major(t: torch.Tensor) -> torch.Tensor:
    """The same logical pool [N, bs, Hkv, D] stored head-major: a new
    [N, Hkv, bs, D] allocation holding the data, returned as the permuted
    view with shape [N, bs, Hkv, D] (strides [Hkv*bs*D, D, bs*D, 1])."""
    N, bs, Hkv, D = t.shape
    hm = torch.empty((N, Hkv, bs, D), dtype=t.dtype, device=t.device)
    hm.copy_(t.permute(0, 2, 1, 3))
    return hm.permute(0, 2, 1, 3)


def cache_bits(t: torch.Tensor) -> np.ndarray:
    """A device cache's logical [N, bs, Hkv, D] contents as host bits (uint16
    for bf16, uint8 codes for fp8), whatever its layout."""
    c = t.contiguous().cpu()
    return c.numpy() if c.dtype == torch.uint8 else c.view(torch.int16).numpy().view(np.uint16)


class DeviceWorkload:
    def __init__(self, w, k_cache=None, v_cache=None, layout="page"):
        self.w = w
        self.q = dev_bf16(w.q)
        kc = w.k_cache if k_cache is None else k_cache
        vc = w.v_cache if v_cache is None else v_cache
        self.fp8 = kc.dtype == np.uint8
        self.k_cache = dev_u8(kc) if self.fp8 else dev_bf16(kc)
        self.v_cache = dev_u8(vc) if self.fp8 else dev_bf16(vc)
        if layout == "head_major":
            self.k_cache, self.v_cache = head_major(self.k_cache), head_major(self.v_cache)
        else:
            assert layout == "page", layout
        self.block_tables = torch.from_numpy(w.block_tables).cuda()
        self.context_lens = torch.from_numpy(w.context_lens).cuda()
        self.new_k = dev_bf16(w.new_k)
        self.new_v = dev_bf16(w.new_v)
        self.slot_mapping = torch.from_numpy(w.slot_mapping).cuda()

    def decode(self, **kw):
        return pa.pa_decode(self.q, self.k_cache, self.v_cache, self.block_tables, self.context_lens,
                            self.w.scale, **kw)


def compare(out_bits: np.ndarray, ref: np.ndarray, max_tol: float, mean_tol: float):
    got = bf16_to_f64(out_bits)
    assert got.shape == ref.shape
    assert np.all(np.isfinite(got)), "non-finite output"
    err = np.abs(got - ref)
    mx, mean = float(err.max()), float(err.mean())
    assert mx <= max_tol and mean <= mean_tol, f"max {mx:.3g} (tol {max_tol}) mean {mean:.3g} (tol {mean_tol})"
    return mx, mean
