"""moe_forward_noalloc (the entry point for callers that cannot allocate)
against moe_forward, through the C ABI: bit for bit on two calls in a row,
the second with a smaller batch (the library's scratch array keeps the first
call's contents), across the layer's dtypes and tile paths; a batch whose
workspace exceeds the array is refused before anything is launched."""
import pytest
import torch

import mixture_experts_layer_10_amd as moe
from synth import make_inputs, workload

from gpu_helpers import say

pytestmark = pytest.mark.gpu


def _small(**kw):
    w = dict(T=96, hidden=512, n_experts=64, expert_begin=0, expert_end=64, top_k=6, n_group=8, topk_group=4,
             score_fn="sigmoid", renormalize=True, routed_scale=1.0, inter=256, shared_inter=256, dtype="bf16",
             capacity_factor=0.0, score_bias="normal0.1", router_bias="none")
    w.update(kw)
    return w


CASES = {
    # bf16 with a shared expert (overlapped in moe_forward: co-resident tiles)
    "small_bf16": (_small(T=200), 77),
    "small_bf16_capacity_share": (_small(T=300, expert_begin=8, expert_end=40, capacity_factor=1.0,
                                         router_bias="zipf1.1"), 33),
    "toy_fp32": (workload("toy_fp32", T=300), 100),
    "small_fp8": (_small(dtype="fp8", T=150, score_bias="zero"), 40),
    "small_mxfp4": (_small(dtype="mxfp4", T=150, score_bias="zero"), 1),
    # the DeepSeek-V3 EP8 share at the real hidden size
    "ep8_decode_bf16": (workload("ep8_decode_bf16", T=256), 64),
}


def _run(w, T, out_dtype):
    w = dict(w, T=T)
    dev = "cuda" if w["hidden"] >= 4096 else "cpu"
    inp = {k: (v.cuda() if v is not None else None) for k, v in make_inputs(w, device=dev).items()}
    cfg = moe.config_from_workload(w, out_dtype=out_dtype)
    W = moe.make_weights(cfg, inp["w13"], inp["w2"], inp["shared_w13"], inp["shared_w2"], inp.get("w13_scale"),
                         inp.get("w2_scale"), inp.get("shared_w13_scale"), inp.get("shared_w2_scale"))
    od = torch.float32 if out_dtype == "f32" else torch.bfloat16
    E, k, H = w["n_experts"], w["top_k"], w["hidden"]
    ref = dict(y=torch.empty(T, H, dtype=od, device="cuda"), l=torch.empty(T, E, device="cuda"),
               i=torch.empty(T, k, dtype=torch.int32, device="cuda"))
    got = {n: torch.full_like(t, 7) for n, t in ref.items()}
    moe.moe_forward(cfg, inp["x"], inp["w_router"], inp["router_bias"], inp["score_bias"], W, ref["y"],
                    moe.workspace(cfg, T), logits_out=ref["l"], topk_ids_out=ref["i"])
    moe.moe_forward_noalloc(cfg, inp["x"], inp["w_router"], inp["router_bias"], inp["score_bias"], W, got["y"],
                            logits_out=got["l"], topk_ids_out=got["i"])
    torch.cuda.synchronize()
    return ref, got


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
def test_noalloc_equals_forward_twice(name, out_dtype):
    w, T2 = CASES[name]
    for T in (w["T"], T2):
        say("noalloc case", name, out_dtype, "T", T)
        ref, got = _run(w, T, out_dtype)
        for n in ("y", "l", "i"):
            assert torch.equal(got[n], ref[n]), (name, T, n)
        assert moe.moe_dispatch_errors() == 0         # the static array's error word: routed ids are valid


def test_noalloc_refuses_a_batch_past_its_scratch():
    w = workload("ep8_decode_bf16", T=340)          # 64.2 MiB of workspace, the array holds 64
    inp = make_inputs(w, device="cuda")
    cfg = moe.config_from_workload(w, out_dtype="bf16")
    assert moe.workspace_bytes(cfg, 340) > moe.NOALLOC_SCRATCH_BYTES >= moe.workspace_bytes(cfg, 339)
    W = moe.make_weights(cfg, inp["w13"], inp["w2"], inp["shared_w13"], inp["shared_w2"])
    y = torch.full((340, w["hidden"]), 3.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(moe.MoEError) as e:
        moe.moe_forward_noalloc(cfg, inp["x"], inp["w_router"], None, inp["score_bias"], W, y)
    assert e.value.status == -3                       # MOE_ERR_WORKSPACE_TOO_SMALL
    torch.cuda.synchronize()
    assert torch.all(y == 3.0)                        # nothing was launched
