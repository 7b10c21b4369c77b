"""The library's calls captured in one HIP graph, as the bench times them.

Every compute entry point (compress, decompress, the sparse GEMM with either
operand compressed through the decode and tile kernels, the dense GEMM, both
hybrids, both fused quantizers and the plain ones) is captured once; the graph
is replayed three times, with the outputs overwritten, other eager launches
and a synchronisation between replays, and every replay must reproduce the
eager results bit for bit.  The kernels are deterministic (each output is
written by one workgroup, cross-wave sums run in a fixed order, no atomics),
so equality is exact."""
import pytest
import torch

import semi_structured_sparse_sp24_amd as sp
from semi_structured_sparse_sp24_amd import inputs
from tests._util import say

pytestmark = pytest.mark.gpu

BF = torch.bfloat16


def _dev(t, dtype):
    return t.to(dtype).cuda()


def _q(t, dt):
    bits, sc = (inputs.quantize_e4m3_rows if dt == inputs.E4M3 else inputs.quantize_i8_rows)(t)
    tdt = torch.float8_e4m3fn if dt == inputs.E4M3 else torch.int8
    return torch.from_numpy(bits).view(tdt).cuda(), torch.from_numpy(sc).cuda()


def _build():
    """(calls, outputs): each call issues one library launch into preallocated outputs."""
    calls, outs = [], {}

    def out(name, t):
        outs[name] = t
        return t

    # bf16 weight path: compress, decompress, decode and tile GEMMs (a ragged tail), dense GEMM
    N, K = 1296, 1024
    W = _dev(inputs.normal((N, K), 0.02, 1), BF)
    v, m = out("v", torch.empty((N, K // 2), dtype=BF, device="cuda")), \
        out("m", torch.empty((N, K // 32), dtype=torch.int32, device="cuda"))
    calls.append(lambda: sp.prune_compress(W, values=v, meta=m))
    Wp = out("Wp", torch.empty((N, K), dtype=BF, device="cuda"))
    calls.append(lambda: sp.decompress(v, m, K, out=Wp))
    for M in (4, 16, 600, 2048):
        X = _dev(inputs.normal((M, K), 1.0, 10 + M), BF)
        Y = out(f"Y{M}", torch.empty((M, N), dtype=BF, device="cuda"))
        Yd = out(f"Yd{M}", torch.empty((M, N), dtype=BF, device="cuda"))
        calls.append(lambda X=X, Y=Y, M=M: sp.sp24_gemm(sp.SPARSE_W, v, m, X, M, N, K, out=Y))
        calls.append(lambda X=X, Yd=Yd: sp.dense_gemm(X, Wp, out=Yd))
    # online bf16: the activation compressed on every call
    M = 512
    Xo = _dev(inputs.normal((M, K), 1.0, 3), BF)
    xv = out("xv", torch.empty((M, K // 2), dtype=BF, device="cuda"))
    xm = out("xm", torch.empty((M, K // 32), dtype=torch.int32, device="cuda"))
    Yo = out("Yo", torch.empty((M, N), dtype=BF, device="cuda"))
    calls.append(lambda: sp.prune_compress(Xo, values=xv, meta=xm))
    calls.append(lambda: sp.sp24_gemm(sp.SPARSE_X, xv, xm, W, M, N, K, out=Yo))
    # row-split and K-split hybrids
    NS, ND = 1024, 272
    Yh = out("Yh", torch.empty((M, NS + ND), dtype=BF, device="cuda"))
    Wd = W[NS:].contiguous()
    vs, ms = v[:NS], m[:NS]
    calls.append(lambda: sp.hybrid_gemm(vs, ms, Wd, Xo, NS, ND, out=Yh))
    KS = 768
    Wk = _dev(inputs.normal((N, K), 0.02, 4), BF)
    vk = out("vk", torch.empty((N, KS // 2), dtype=BF, device="cuda"))
    mk = out("mk", torch.empty((N, KS // 32), dtype=torch.int32, device="cuda"))
    Wks = Wk[:, :KS].contiguous()
    Wkd = Wk[:, KS:].contiguous()
    Yk = out("Yk", torch.empty((M, N), dtype=BF, device="cuda"))
    calls.append(lambda: sp.prune_compress(Wks, values=vk, meta=mk))
    calls.append(lambda: sp.ksplit_gemm(vk, mk, Wkd, Xo, N, KS, out=Yk))
    # fused online quantizers into the scaled fp8 / int8 activation-compressed GEMMs, and the dense sides
    Xa = inputs.outliers(inputs.normal((M, K), 1.0, 5), 0.01, 20.0, 6)
    Xb = _dev(Xa, BF)
    for dt, fused, plain, tdt in ((inputs.E4M3, sp.quantize_prune_compress, sp.quantize_e4m3, torch.float8_e4m3fn),
                                  (inputs.I8, sp.quantize_i8_prune_compress, sp.quantize_i8, torch.int8)):
        Wq, sw = _q(inputs.normal((N, K), 0.02, 7), dt)
        qv = out(f"qv{dt}", torch.empty((M, K // 2), dtype=tdt, device="cuda"))
        qm = out(f"qm{dt}", torch.empty((M, K // 32), dtype=torch.int32, device="cuda"))
        qs = out(f"qs{dt}", torch.empty(M, dtype=torch.float32, device="cuda"))
        qq = out(f"qq{dt}", torch.empty((M, K), dtype=tdt, device="cuda"))
        qqs = out(f"qqs{dt}", torch.empty(M, dtype=torch.float32, device="cuda"))
        Ys = out(f"Ys{dt}", torch.empty((M, N), dtype=BF, device="cuda"))
        Yq = out(f"Yq{dt}", torch.empty((M, N), dtype=BF, device="cuda"))
        calls.append(lambda fused=fused, qv=qv, qm=qm, qs=qs: fused(Xb, values=qv, meta=qm, scales=qs))
        calls.append(lambda qv=qv, qm=qm, qs=qs, Wq=Wq, sw=sw, Ys=Ys:
                     sp.sp24_gemm(sp.SPARSE_X, qv, qm, Wq, M, N, K, scale_x=qs, scale_w=sw, out=Ys))
        calls.append(lambda plain=plain, qq=qq, qqs=qqs: plain(Xb, out=qq, scales=qqs))
        calls.append(lambda qq=qq, qqs=qqs, Wq=Wq, sw=sw, Yq=Yq: sp.dense_gemm(qq, Wq, scale_x=qqs, scale_w=sw, out=Yq))
    return calls, outs


def _bytes(t):
    return t.view(torch.uint8) if t.element_size() == 1 else t.view(torch.int16 if t.element_size() == 2 else torch.int32)


def test_graph_replays_match_eager():
    say("graph capture of every entry point")
    calls, outs = _build()
    for c in calls:
        c()
    torch.cuda.synchronize()
    ref = {k: _bytes(t).clone() for k, t in outs.items()}
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for c in calls:
                c()
    torch.cuda.synchronize()
    for rep in range(3):
        # overwrite every output so that a replay that skipped a launch would show
        for t in outs.values():
            _bytes(t).fill_(0x5a if t.element_size() == 1 else 0x3a5a)
        # eager launches of the same kernels between replays, on other buffers
        a = torch.randn((64, 1024), device="cuda").to(BF)
        sp.prune_compress(a)
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            g.replay()
        torch.cuda.synchronize()
        for k, t in outs.items():
            assert torch.equal(_bytes(t), ref[k]), f"replay {rep}: output {k} differs from the eager run"
        say("  replay", rep, "matches")
