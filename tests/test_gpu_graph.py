"""The IndexCache loop captured as one HIP graph (the decode step of a serving loop): every
replay must equal an eager call on the same inputs, with eager work and synchronisation
between the replays and the inputs changed in place before some of them.  The library
launches kernels only (no memsets, copies, allocations or synchronisation), so the whole
loop is capturable; the workspace and outputs are passed in."""
import numpy as np
import pytest
import torch

import dsa_indexer_indexcache_amd as dsa
import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


def announce(msg):
    print("[case] " + msg, flush=True)


@pytest.mark.parametrize("qk_dtype", ["bf16", "fp8"])
def test_decode_step_graph_replays_equal_eager(qk_dtype):
    announce("graph replay decode FSSSFSSS %s" % qk_dtype)
    lens = [5000, 7300, 2100, 9000]
    roles, k = "FSSSFSSS", 512
    layers = [synth.make_layer(len(lens), int(np.sum(lens)), 64, 128, 32, wid=14, layer=l, qk_dtype=qk_dtype,
                               device=DEV) for l in range(len(roles))]
    ld = [dsa.layer_dict(x) for x in layers]
    seqs = dsa.Seqs.decode(lens)
    outs = [torch.empty((len(lens), 32, 512), dtype=torch.float32, device=DEV) for _ in roles]
    icache = torch.empty((len(lens), k), dtype=torch.int32, device=DEV)
    first = dsa.indexcache_forward(roles, ld, k, seqs, outs=outs, index_cache=icache)
    ws = first.ws
    torch.cuda.synchronize()

    def eager():
        o = [torch.empty_like(x) for x in outs]
        ic = torch.empty_like(icache)
        dsa.indexcache_forward(roles, ld, k, seqs, outs=o, index_cache=ic)
        torch.cuda.synchronize()
        return o, ic

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        dsa.indexcache_forward(roles, ld, k, seqs, outs=outs, index_cache=icache, ws=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        dsa.indexcache_forward(roles, ld, k, seqs, outs=outs, index_cache=icache, ws=ws)
    torch.cuda.synchronize()

    gen = torch.Generator(device=DEV)
    for rep in range(4):
        if rep >= 2:   # new inputs in place: the replay must see them
            gen.manual_seed(100 + rep)
            layers[0].q.copy_(torch.randn(layers[0].q.shape, generator=gen, device=DEV).to(torch.bfloat16))
            layers[4].w.copy_((torch.randn(layers[4].w.shape, generator=gen, device=DEV) / 8).to(torch.bfloat16))
        outs[3].fill_(float("nan"))
        icache.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        want, want_ic = eager()
        assert torch.equal(icache, want_ic), "replay %d: index cache differs" % rep
        for l in range(len(roles)):
            assert torch.equal(outs[l], want[l]), "replay %d: layer %d output differs" % (rep, l)
    print("4 replays equal to eager", flush=True)
