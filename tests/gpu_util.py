"""Helpers for GPU parity tests: move seeded bf16 bits to the device and
results back, and name each case on stdout before it runs."""

import sys

import numpy as np


def announce(*what):
    print("[case]", *what, flush=True)
    sys.stdout.flush()


def to_dev_bf16(bits: np.ndarray):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).view(torch.bfloat16)
    return t.cuda()


def bf16_dev_to_f64(t) -> np.ndarray:
    import torch
    u = t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return (u.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def s_t_bits(q) -> int:
    import torch
    return int(q.rec[:1].cpu().numpy().view(np.uint32)[0])


def quantized_host(q):
    """(codes, scales, s_t bits) of a device NVFP4 as numpy."""
    return q.codes.cpu().numpy(), q.scales.cpu().numpy(), s_t_bits(q)


def upload_nvfp4(oq, device="cuda"):
    """Oracle NVFP4 tensor -> device buffers (for GEMM-only tests)."""
    import torch
    import fp4_block_scaled_elem_amd as mq
    R, K = oq.shape
    q = mq.NVFP4.empty(R, K, device=device)
    q.codes.copy_(torch.from_numpy(oq.codes))
    q.scales.copy_(torch.from_numpy(oq.scales))
    q.set_s_t(float(oq.s_t))
    return q
