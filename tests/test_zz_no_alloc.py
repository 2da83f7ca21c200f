"""hy_moe_forward_noalloc (scratch in the library's static per-device buffer) against
hy_moe_forward_ex with a caller workspace, through the C ABI: the same kernels run
on the same inputs, so outputs and routing must be bitwise identical. Calls run back
to back on one device with shrinking and growing batches (each call must rewrite
whatever it reads of the buffer), on both expert paths, on Sherry weights (with a bf16
or a Sherry shared expert) and on the W8A8 format; the first case is also checked
against the fp64 oracle."""
import pytest

import hy_inputs as hi
import oracle
from parity import bf16_tensor_to_np, check_out, check_routing, routing_to_np

torch = pytest.importorskip("torch")
hm = pytest.importorskip("sparse_moe_transformer_route_amd")

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
KEYS = ("topk_idx", "topk_w", "counts", "offsets", "perm_src", "margin")


def say(msg):
    print(msg, flush=True)


def compare(inp, k, path, label, a8=False):
    fmt = (hm.WEIGHTS_SHERRY_TERNARY if "qgate" in inp else hm.WEIGHTS_FP8_W8A8 if a8 else
           hm.WEIGHTS_FP8_E4M3 if "fgate" in inp else hm.WEIGHTS_BF16)
    T, d = inp["x"].shape
    E = inp["router"].shape[0]
    I = (inp["sgate"] if "qgate" in inp else inp["fsgate"] if "fgate" in inp else inp["gate"]).shape[1]
    say(f"[case] {label}: T={T} d={d} E={E} k={k} I={I} path={path} w8a8={a8}")
    ws = hm.alloc_workspace(T, d, E, k, I, fmt, device=DEV)
    ref = hm.forward_layer(inp, k, want_routing=True, path=path, workspace=ws, fp8_activations=a8)
    got = hm.forward_layer(inp, k, want_routing=True, path=path, noalloc=True, fp8_activations=a8)
    torch.cuda.synchronize()
    assert torch.equal(got["out"].view(torch.int16), ref["out"].view(torch.int16)), label
    for key in KEYS:
        assert torch.equal(got[key].view(torch.int32), ref[key].view(torch.int32)), (label, key)
    return got


def test_noalloc_matches_workspace_entry_point():
    big = hi.LayerConfig("na", T=96, d=1024, E=32, k=4, I=512, seed=11)
    inp = hi.dev_layer(big, device=DEV)
    got = compare(inp, big.k, hm.PATH_AUTO, "streaming path, first call")
    # the first call against the oracle as well
    L = hi.host_layer(big)
    lg = oracle.logits(L["x"], L["router"], L["bias"])
    g = routing_to_np(got)
    sets, _, _ = check_routing(g["topk_idx"], lg, big.k)
    ref = oracle.forward(L["x"], L["router"], L["bias"], L["gate"], L["up"], L["down"], L["shared"]["gate"],
                         L["shared"]["up"], L["shared"]["down"], big.k, sets_in=sets)
    worst, _ = check_out(bf16_tensor_to_np(got["out"]), ref["out"])
    say(f"       oracle max_rel_err={worst:.3e}")
    # a smaller batch right after: the buffer holds the larger call's contents
    small = dict(inp)
    small["x"] = inp["x"][:37].contiguous()
    compare(small, big.k, hm.PATH_AUTO, "streaming path, smaller second call")
    # grouped path, larger again, then smaller
    compare(inp, big.k, hm.PATH_GROUPED, "grouped path")
    compare(small, big.k, hm.PATH_GROUPED, "grouped path, smaller")


def test_noalloc_ternary_and_hy4_decode_shape():
    tern = hi.LayerConfig("nat", T=24, d=1024, E=16, k=4, I=512, ternary=True, seed=12)
    inp = hi.dev_layer(tern, device=DEV)
    compare(inp, tern.k, hm.PATH_AUTO, "Sherry weights")
    tsh = hi.LayerConfig("nats", T=24, d=1024, E=16, k=4, I=512, ternary=True, tshared=True, seed=15)
    compare(hi.dev_layer(tsh, device=DEV), tsh.k, hm.PATH_AUTO, "Sherry weights, Sherry shared expert")
    # the Hy4 decode batch at its largest admitted size and at T=32, on a few experts'
    # worth of shape (d, I as the Hy4 layer; fewer experts keep the weights small)
    cfg = hi.LayerConfig("nah", T=251, d=6144, E=16, k=8, I=2048, seed=13)
    inp = hi.dev_layer(cfg, device=DEV)
    compare(inp, cfg.k, hm.PATH_AUTO, "largest admitted batch at d=6144, I=2048")
    small = dict(inp)
    small["x"] = inp["x"][:32].contiguous()
    compare(small, cfg.k, hm.PATH_AUTO, "T=32 after it")


def test_noalloc_w8a8():
    # W8A8 runs the grouped path with the token rows' and hidden rows' MXFP8 codes and
    # scales in the buffer as well: a larger call, then a smaller one
    cfg = hi.LayerConfig("naw", T=300, d=512, E=8, k=2, I=512, fp8=True, a8=True, seed=14)
    inp = hi.dev_layer(cfg, device=DEV)
    compare(inp, cfg.k, hm.PATH_AUTO, "W8A8", a8=True)
    small = dict(inp)
    small["x"] = inp["x"][:70].contiguous()
    compare(small, cfg.k, hm.PATH_AUTO, "W8A8, smaller second call", a8=True)


def test_noalloc_rejects_batches_beyond_the_buffer():
    # the limits the header states at the Hy4 layer shape: T <= 251, and T <= 383 for W8A8
    assert hm.workspace_size(251, 6144, 256, 8, 2048) <= hm.NOALLOC_SCRATCH_BYTES
    assert hm.workspace_size(252, 6144, 256, 8, 2048) > hm.NOALLOC_SCRATCH_BYTES
    assert hm.workspace_size(383, 6144, 256, 8, 2048, hm.WEIGHTS_FP8_W8A8) <= hm.NOALLOC_SCRATCH_BYTES
    assert hm.workspace_size(384, 6144, 256, 8, 2048, hm.WEIGHTS_FP8_W8A8) > hm.NOALLOC_SCRATCH_BYTES
    # the check is on the host and needs no weights: the pointers (one small device
    # buffer) are never dereferenced when the call is rejected or the batch is empty
    a = hm.HyMoeArgs()
    buf = torch.empty(256, dtype=torch.uint8, device=DEV)
    p = buf.data_ptr()
    a.x = a.W_router = a.W_gate = a.W_up = a.W_down = a.Ws_gate = a.Ws_up = a.Ws_down = a.out = p
    a.T, a.d, a.E, a.k, a.I = 252, 6144, 256, 8, 2048
    assert hm.forward_noalloc(a) == hm.ERR_WORKSPACE
    a.T = 0
    assert hm.forward_noalloc(a) == hm.OK
