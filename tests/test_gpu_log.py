"""MQ_LOG=1: every launch prints its kernel, grid and shape to stderr.

The flag is read once per process, so each case runs a short child process
(one after the other, never in parallel).
"""

import os
import subprocess
import sys

import pytest

from tests.gpu_util import announce

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

SCRIPT = """
import sys
sys.path.insert(0, {root!r})
import torch
import fp4_block_scaled_elem_amd as mq
x = torch.randn(40, 512, device="cuda").to(torch.bfloat16)
w = (torch.randn(300, 512, device="cuda") * 0.02).to(torch.bfloat16)
y = mq.prefill_linear(x, mq.quantize(w))
z = mq.decode_linear(x[:3].contiguous(), w)
torch.cuda.synchronize()
print("done", flush=True)
""".format(root=ROOT)


def _run(env_extra):
    env = dict(os.environ)
    env.pop("MQ_LOG", None)
    env.update(env_extra)
    r = subprocess.run([sys.executable, "-c", SCRIPT], env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and "done" in r.stdout, r.stderr[-2000:]
    return [line for line in r.stderr.splitlines() if line.startswith("mq: ")]


def test_log_lists_every_launch():
    announce("MQ_LOG=1")
    lines = _run({"MQ_LOG": "1"})
    kernels = [line.split()[1] for line in lines]
    # weight quantization (300 x 512: amax pass + encode), activation
    # quantization (40 x 512, at most 2^17 elements: the encode kernel takes
    # the maximum itself, one launch), the GEMM (40 rows: the small-problem
    # kernel: on so few tiles one 16-row W tile and one 16-row A tile per
    # workgroup, 19 x 3 of them), the GEMV
    assert kernels.count("amax_kernel") == 1 and kernels.count("quantize_kernel") == 2, lines
    quant = [line for line in lines if " quantize_kernel " in line]
    assert "elements=153600 mode=0" in quant[0] and "elements=20480 mode=2" in quant[1], quant
    assert kernels.count("gemm_small_kernel") == 1 and kernels.count("gemv_bf16_kernel") == 1, lines
    gemm = next(line for line in lines if " gemm_small_kernel " in line)
    assert "M=40 K=512" in gemm and "tiles=3x19" in gemm and "grid=57 " in gemm and "lds=" in gemm


def test_log_is_silent_by_default():
    announce("MQ_LOG unset")
    assert _run({}) == []
