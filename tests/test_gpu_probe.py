"""The matrix-core rate probe (mcg_mfma_probe) runs the GEMM kernels' instructions
on fragments loaded once.  These tests pin what it computes, so that its rate is
the rate of real instructions.  With every operand element equal to 1, one
instruction adds k to every accumulator element, where k is its dense k ("CDNA3
dense MFMA builtins", Instruction throughput: 16 for the 16-bit 32x32 instruction,
32 for int8, 64 for fp8) or, for the 2:4 instructions, its kept values (half the
dense k; "RDNA4 sparse WMMA builtins", Structured sparsity).  Each of a thread's
8 accumulators of 16 registers receives instr_per_wave / 8 instructions, so the
thread's sum is 8 * 16 * k * instr_per_wave / 8."""
import pytest
import torch

from gpu_util import need_gpu, say

pytestmark = pytest.mark.gpu

# byte pattern of 1.0 in each element format
ONE = {"bf16": (0x80, 0x3F), "f16": (0x00, 0x3C), "i8": (0x01,), "e4m3": (0x38,), "e5m2": (0x3C,)}
# k of one multiplied instruction per output element: dense k, or the kept values of the 2:4 instruction
K_DENSE = {"bf16": 16, "f16": 16, "i8": 32, "e4m3": 64, "e5m2": 64}
K_KEPT = {"bf16": 16, "f16": 16, "i8": 32, "e4m3": 32, "e5m2": 32}


def ones(fmt, nbytes=65536):
    pat = torch.tensor(ONE[fmt], dtype=torch.uint8)
    return pat.repeat(nbytes // len(ONE[fmt])).cuda()


@pytest.mark.parametrize("pair,sparse", [(("bf16", "bf16"), 0), (("f16", "f16"), 0), (("i8", "i8"), 0),
                                         (("e4m3", "e4m3"), 0), (("e4m3", "e5m2"), 0), (("e5m2", "e4m3"), 0),
                                         (("bf16", "bf16"), 1), (("f16", "f16"), 1), (("i8", "i8"), 1),
                                         (("e4m3", "e4m3"), 1), (("e5m2", "e4m3"), 1)])
def test_probe_runs_real_instructions(pair, sparse):
    mcg = need_gpu()
    fa, fb = pair
    say(f"probe {fa} x {fb} sparse={sparse}")
    instr, nwg = 64, 3
    a, b = ones(fa), ones(fb)
    # index codes 0x4 per group of four: kept values at positions 0 and 1
    idx = torch.full((16384,), 0x44444444, dtype=torch.int32, device="cuda")
    sink = torch.full((nwg * 512,), float("nan"), device="cuda")
    clocks = torch.zeros(2 * nwg, dtype=torch.int64, device="cuda")
    mcg.mfma_probe(fa, fb, sparse, a, b, idx, instr, nwg, sink, clocks)
    torch.cuda.synchronize()
    k = K_KEPT[fa] if sparse else K_DENSE[fa]
    # each of the 8 accumulators gets instr / 8 instructions; 16 registers each
    expect = 8 * 16 * k * (instr // 8)
    assert torch.all(sink == expect), (sink.min().item(), sink.max().item(), expect)
    c = clocks.view(nwg, 2).cpu()
    assert torch.all(c > 0)
    ghz = (c[:, 0].double() / c[:, 1].double() * 0.1)
    assert torch.all((ghz > 0.3) & (ghz < 3.5)), ghz


def test_probe_zero_operands_reach_the_published_rate():
    # with all-zero operands the clock stays near its peak, so the probe's rate
    # approaches the published dense bf16 peak (2.5 PFLOP/s on 256 CUs at 2.4 GHz)
    mcg = need_gpu()
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    z = torch.zeros(65536, dtype=torch.uint8, device="cuda")
    sink = torch.empty(ncu * 512, device="cuda")
    clocks = torch.zeros(2 * ncu, dtype=torch.int64, device="cuda")
    instr = 16384
    mcg.mfma_probe("bf16", "bf16", 0, z, z, None, instr, ncu, sink, clocks)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    mcg.mfma_probe("bf16", "bf16", 0, z, z, None, instr, ncu, sink, clocks)
    ev1.record()
    torch.cuda.synchronize()
    t = ev0.elapsed_time(ev1) * 1e-3
    rate = ncu * 8 * instr * 2 * 32 * 32 * 16 / t
    c = clocks.view(ncu, 2).cpu().double()
    ghz = (c[:, 0] / c[:, 1] * 0.1).mean().item()
    say(f"zero-operand bf16 probe: {rate / 1e12:.0f} TFLOP/s at {ghz:.2f} GHz")
    assert torch.all(sink == 0)
    assert rate > 0.8 * 2.5e15 * ncu / 256
