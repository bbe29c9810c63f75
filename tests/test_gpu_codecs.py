"""Exhaustive GPU checks of the conversions every NVFP4 kernel is built on.

The quantizer and the fused GEMM prologue take each element code from
gfx950's fp32 -> fp4 conversion (``encode8``) and each group-scale byte from
its fp32 -> fp8 conversion (``e4m3_from_f32``); the GEMM and the NVFP4 GEMV
take each operand from ``sigma_pair`` + ``dequant8``.  The parity tests
sample these; here they are run over their whole domains, through
test-support entry points of libmq.so that call exactly those device
functions, and compared with the oracle's definitions of the formats
(``oracle.e2m1_encode_magnitude``, ``oracle.e4m3_encode``,
``oracle.e2m1_decode`` x ``oracle.e4m3_decode``).

A conversion of the binary32 pattern p is a step function of p: the GPU
reports every p whose result differs from that of p - 1.  Within the sign
half that is swept the oracle's result is a non-decreasing function of |y|
(nearest value of a sorted table, ties to even), and |y| grows with the
pattern, so when the oracle agrees with a step's value at the step's first
and last pattern it agrees on every pattern between them: agreement at
the 2 x (number of steps) end points is agreement on all 2^32 inputs.

Finally the quantizer entry point itself is swept: under a given tensor
scale (normal, tiny and subnormal), for every E4M3 group-scale byte that
scale can produce, a group max mapping to it and every finite bf16
magnitude at or below that max, with both signs -- codes and scale bytes
against ``oracle.quantize_nvfp4`` byte for byte.
"""

import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_util import announce, to_dev_bf16

pytestmark = pytest.mark.gpu


def _mq():
    import fp4_block_scaled_elem_amd as mq
    return mq


def _steps(which, lo, hi, cap=4096):
    """Sorted (pattern, value) steps of conversion `which` over [lo, hi]."""
    import torch
    mq = _mq()
    out = torch.zeros(1 + 2 * cap, dtype=torch.int32, device="cuda")
    mq.mq_check_codec_steps(which, lo, hi, out)
    torch.cuda.synchronize()
    h = out.cpu().numpy().view(np.uint32)
    n = int(h[0])
    assert 0 < n <= cap, f"{n} steps (capacity {cap})"
    st = h[1:1 + 2 * n].reshape(n, 2).astype(np.int64)
    st = st[np.argsort(st[:, 0])]
    assert st[0, 0] == lo, "the first pattern must open a step"
    assert len(np.unique(st[:, 0])) == n
    return st


def _as_f32(p):
    return np.asarray(p, dtype=np.int64).astype(np.uint32).view(np.float32)


def _end_points(st, hi):
    first = st[:, 0]
    last = np.concatenate([st[1:, 0] - 1, [hi]])
    return first, last


def _check_steps(st, hi, expect):
    """expect(patterns) -> values; compared at both ends of every step."""
    first, last = _end_points(st, hi)
    got = st[:, 1]
    for where, p in (("first", first), ("last", last)):
        want = expect(p).astype(np.int64)
        bad = np.nonzero(want != got)[0]
        assert bad.size == 0, (f"{bad.size} steps differ at their {where} pattern, e.g. "
                               f"p=0x{int(p[bad[0]]):08X} gpu={int(got[bad[0]])} oracle={int(want[bad[0]])}")
    # consecutive steps carry different values (else they would be one step)
    assert np.all(got[1:] != got[:-1])


def _e2m1_code(p):
    y = _as_f32(p)
    mag = oracle.e2m1_encode_magnitude(np.abs(y)).astype(np.int64)
    return (np.signbit(y).astype(np.int64) << 3) | mag


@pytest.mark.parametrize("half", ["positive", "negative"])
def test_element_code_every_binary32(half):
    # every non-NaN binary32 y of one sign (zero and infinity included)
    announce("codec exhaustive e2m1", half)
    lo, hi = (0x00000000, 0x7F800000) if half == "positive" else (0x80000000, 0xFF800000)
    st = _steps(0, lo, hi)
    print(f"  {len(st)} steps:", [(hex(int(p)), int(v)) for p, v in st], flush=True)
    _check_steps(st, hi, _e2m1_code)
    # eight magnitudes, each once, in order
    assert list(st[:, 1] & 7) == list(range(8))


def test_group_scale_byte_every_binary32():
    # every non-negative binary32 rho: finite, +inf and the NaN patterns
    # (the kernels clamp with minNum, so NaN maps to 448 -> 0x7E)
    announce("codec exhaustive e4m3")
    lo, hi = 0x00000000, 0x7FFFFFFF
    st = _steps(1, lo, hi)
    print(f"  {len(st)} steps, last {[(hex(int(p)), int(v)) for p, v in st[-3:]]}", flush=True)
    finite = st[:, 0] <= 0x7F7FFFFF
    assert finite.all(), "a step inside the inf/NaN patterns"
    # finite and +inf end points against the oracle; the last step runs on
    # through +inf and every NaN pattern, so it must be the saturated 0x7E
    first, last = _end_points(st, 0x7F800000)
    for where, p in (("first", first), ("last", last)):
        want = oracle.e4m3_encode(_as_f32(p)).astype(np.int64)
        bad = np.nonzero(want != st[:, 1])[0]
        assert bad.size == 0, (f"{bad.size} steps differ at their {where} pattern, e.g. "
                               f"p=0x{int(p[bad[0]]):08X} gpu=0x{int(st[bad[0], 1]):02X} oracle=0x{int(want[bad[0]]):02X}")
    assert st[-1, 1] == 0x7E
    # all 127 finite E4M3 bytes appear, in order
    assert list(st[:, 1]) == list(range(0x7F))


def test_dequantized_operand_every_scale_and_code():
    # binary16 operand g * sigma of every E4M3 scale byte (in each of the
    # four byte positions of a scale dword) and every 4-bit code, bit for bit
    announce("codec dequant table")
    import torch
    mq = _mq()
    out = torch.zeros((128, 4, 16), dtype=torch.int16, device="cuda")
    mq.mq_check_dequant_table(out)
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint16)[:0x7F]                    # scale bytes 0x00..0x7E
    g = oracle.e2m1_decode(np.arange(16))                              # float64, -0 for code 8
    sigma = oracle.e4m3_decode(np.arange(0x7F)).astype(np.float64)
    want = (sigma[:, None] * g[None, :]).astype(np.float16)           # exact: <= 6 significant bits
    assert np.all(np.abs(sigma[:, None] * g[None, :]) == np.abs(want.astype(np.float64)))
    want_bits = want.view(np.uint16)
    for k in range(4):
        bad = np.argwhere(got[:, k, :] != want_bits)
        assert bad.size == 0, f"byte position {k}: {len(bad)} operands differ, first (S, code) = {tuple(bad[0])}"


def _scale_sweep_inputs(s_t):
    """Rows of 16-element groups: for each E4M3 byte S reachable under s_t,
    the largest group max a_S mapping to S (S grows with a, so the group
    reciprocal and every element code depend on S alone), then every finite
    bf16 magnitude m <= a_S
    (15 per group, the max in a rotating position, signs alternating by
    group).  Reachability and a_S come from the oracle alone."""
    mags = np.arange(0, 0x7F80, dtype=np.uint16)                       # 0 .. largest finite bf16
    # each magnitude alone in a group of zeros: its group's scale byte
    probe = np.zeros((len(mags), 16), np.uint16)
    probe[:, 0] = mags
    S = oracle.quantize_nvfp4(probe.reshape(-1, 16), s_t=s_t).scales[:, 0]
    groups = []
    reached = []
    for s in np.unique(S):
        a = mags[len(S) - 1 - np.argmax(S[::-1] == s)]                 # largest magnitude giving s
        reached.append(int(s))
        sweep = mags[mags <= a]
        pad = (-len(sweep)) % 15
        sweep = np.concatenate([sweep, np.zeros(pad, np.uint16)]).reshape(-1, 15)
        for i, row in enumerate(sweep):
            g = np.insert(row, i % 16, a)
            if i % 2:
                g = g | np.uint16(0x8000)
            groups.append(g)
    x = np.stack(groups).astype(np.uint16)
    pad = (-len(x)) % 64
    x = np.concatenate([x, np.zeros((pad, 16), np.uint16)])
    return x.reshape(-1, 64 * 16), reached


@pytest.mark.parametrize("s_t", [np.float32(1.0 / 448.0), np.float32(2.0 ** -100), np.float32(2.0 ** -140)],
                         ids=["normal", "tiny", "subnormal"])
def test_quantizer_every_scale_byte_and_magnitude(s_t):
    announce("quantizer sweep, given s_t", float(s_t))
    import torch
    mq = _mq()
    x, reached = _scale_sweep_inputs(s_t)
    print(f"  {len(reached)} reachable scale bytes, {x.size} elements", flush=True)
    R, K = x.shape
    q = mq.NVFP4.empty(R, K)
    q.set_s_t(float(s_t))
    mq.mq_quantize_nvfp4(to_dev_bf16(x), q, mq.MQ_SCALE_GIVEN)
    torch.cuda.synchronize()
    oq = oracle.quantize_nvfp4(x, s_t=s_t)
    assert set(np.unique(oq.scales)) == set(reached)
    assert np.array_equal(q.scales.cpu().numpy(), oq.scales), "scale bytes differ"
    assert np.array_equal(q.codes.cpu().numpy(), oq.codes), "codes differ"
