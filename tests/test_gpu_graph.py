"""The path under HIP graph capture (torch.cuda.CUDAGraph over the C ABI).

Every entry point enqueues kernels only (no allocation, no memset, no host
synchronisation), so a caller can capture it. The graph is replayed several
times with eager work and synchronisations in between, and every replay must
reproduce the eager outputs bit for bit.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import block_scaled_fp4_absmax_amd as fp4
from block_scaled_fp4_absmax_amd import inputs
from parity_util import note, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fp4.lib()


def test_graph_replays_match_eager():
    note("case: HIP graph of rotate+quantize (MXFP4) and dequantize with inverse rotation "
         "(prepared calls), NVFP4 RaZeR with computed s_t, and the GEMM (tiles and split-K); "
         "4 replays")
    x = to_dev(inputs.gen_c4(rows=512, cols=4096))
    w = to_dev(inputs.gen_c5(0, rows=256, cols=4096))
    perm = fp4.build_permutation(fp4.channel_energy(x)).cuda()
    # static outputs
    c = torch.empty((512, 2048), dtype=torch.uint8, device="cuda")
    s = torch.empty((512, 128), dtype=torch.uint8, device="cuda")
    d = torch.empty((512, 4096), dtype=torch.bfloat16, device="cuda")
    cn = torch.empty((256, 2048), dtype=torch.uint8, device="cuda")
    sn = torch.empty((256, 256), dtype=torch.uint8, device="cuda")
    tn = torch.empty(1, dtype=torch.float32, device="cuda")
    cw = torch.empty((256, 2048), dtype=torch.uint8, device="cuda")
    sw = torch.empty((256, 128), dtype=torch.uint8, device="cuda")
    out = torch.empty((512, 256), dtype=torch.float32, device="cuda")
    out16 = torch.empty((16, 256), dtype=torch.bfloat16, device="cuda")  # split-K GEMM
    # prepared calls follow the stream current at each run, the capture stream included
    p_rot = fp4.rotate_quantize(x, perm, 32, codes=c, scales=s, prepare=True)
    p_deq = fp4.dequantize(c, s, fp4.MXFP4, perm=perm, hadamard=32, out=d, prepare=True)

    def work():
        p_rot.run()
        p_deq.run()
        fp4.quantize(w, fp4.NVFP4, fp4.RAZER, tensor_scale=tn, scale_given=False, codes=cn,
                     scales=sn)
        fp4.rotate_quantize(w, None, 32, codes=cw, scales=sw)
        fp4.gemm(c, s, cw, sw, out=out)
        fp4.gemm(c[:16], s[:16], cw, sw, out=out16)

    work()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (c, s, d, cn, sn, tn, cw, sw, out, out16)]
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        work()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        work()
    for rep in range(4):
        for t in (c, s, d, cn, sn, tn, cw, sw, out, out16):
            t.zero_()  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip((c, s, d, cn, sn, tn, cw, sw, out, out16), ref):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"replay {rep}"
