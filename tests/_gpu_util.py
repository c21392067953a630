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


class DeviceWorkload:
    def __init__(self, w, k_cache=None, v_cache=None):
        self.w = w
        self.q = dev_bf16(w.q)
        kc = w.k_cache if k_cache is None else k_cache
        vc = w.v_cache if v_cache is None else v_cache
        self.fp8 = kc.dtype == np.uint8
        self.k_cache = dev_u8(kc) if self.fp8 else dev_bf16(kc)
        self.v_cache = dev_u8(vc) if self.fp8 else dev_bf16(vc)
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
