"""Shared helpers of the GPU parity tests: run the HIP path stage by stage
through the C ABI, and compare with the oracle on the same inputs."""
import math
import sys

import numpy as np
import torch

import mixture_experts_layer_10_amd as moe
from oracle import moe_oracle as O
from synth import make_inputs

# Layer-output tolerance, max |dy| / RMS(y): fp32 and bf16 as the carrier
# types' rounding allows; fp8 and mxfp4 both quantise x and h to e4m3 on both
# sides (the oracle models it), so only accumulation order and the rare
# e4m3 code of h that lands one step apart remain.
TOL = {"f32": 1e-5, "bf16": 2e-2, "fp8": 6e-2, "mxfp4": 6e-2}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def host(t):
    """torch tensor -> numpy (float values, or uint8 codes for float8)."""
    if t is None:
        return None
    t = t.detach().cpu()
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).numpy()
    if t.dtype in (torch.bfloat16, torch.float16):
        return t.float().numpy()
    return t.numpy()


class Run:
    """Inputs of workload `w` on the GPU and the outputs of each HIP stage."""

    def __init__(self, w, out_dtype="f32", gen_device="cpu", seed=0, packed=False):
        self.w = w
        self.cfg = moe.config_from_workload(w, out_dtype=out_dtype)
        self.ocfg = O.Config.from_workload(w)
        inp = make_inputs(w, device=gen_device, seed=seed)
        self.inp = {k: (v.cuda() if v is not None else None) for k, v in inp.items()}
        self.T = w["T"]
        self.ws = moe.workspace(self.cfg, self.T)
        i = self.inp
        self.W = moe.make_weights(self.cfg, i["w13"], i["w2"], i["shared_w13"], i["shared_w2"],
                                  i.get("w13_scale"), i.get("w2_scale"), i.get("shared_w13_scale"),
                                  i.get("shared_w2_scale"))
        if packed:
            # the 256 x 256 tiles then read the prepacked copy of the weights
            self.packed = moe.moe_prepack_weights(self.cfg, self.W)
            self.W = moe.make_weights(self.cfg, i["w13"], i["w2"], i["shared_w13"], i["shared_w2"],
                                      packed=self.packed)

    def stages(self):
        c, i, T = self.cfg, self.inp, self.T
        E, k, El, H = c.n_experts, c.top_k, c.n_local, c.hidden
        dev = "cuda"
        r = {}
        r["logits"] = torch.empty(T, E, dtype=torch.float32, device=dev)
        moe.moe_router_gemm(c, i["x"], i["w_router"], i["router_bias"], r["logits"], self.ws)
        r["ids"] = torch.empty(T, k, dtype=torch.int32, device=dev)
        r["w"] = torch.empty(T, k, dtype=torch.float32, device=dev)
        moe.moe_route(c, r["logits"], i["score_bias"], r["ids"], r["w"])
        r["raw_counts"] = torch.empty(El, dtype=torch.int32, device=dev)
        r["counts"] = torch.empty(El, dtype=torch.int32, device=dev)
        r["offsets"] = torch.empty(El + 1, dtype=torch.int32, device=dev)
        r["perm"] = torch.full((T * k,), -7, dtype=torch.int32, device=dev)
        r["inv"] = torch.empty(T * k, dtype=torch.int32, device=dev)
        moe.moe_dispatch(c, r["ids"], r["raw_counts"], r["counts"], r["offsets"], r["perm"], r["inv"], self.ws)
        rd = torch.float32 if c.dtype == moe.DTYPE_F32 else torch.bfloat16
        r["rows"] = torch.zeros(T * k, H, dtype=rd, device=dev)
        r["shared"] = torch.zeros(T, H, dtype=torch.float32, device=dev) if c.shared_inter else None
        moe.moe_expert_ffn(c, i["x"], r["perm"], r["offsets"], self.W, r["rows"], r["shared"], self.ws)
        od = torch.float32 if c.out_dtype == moe.DTYPE_F32 else torch.bfloat16
        r["y"] = torch.empty(T, H, dtype=od, device=dev)
        moe.moe_combine(c, r["rows"], r["inv"], r["w"], r["shared"], r["y"])
        torch.cuda.synchronize()
        return r

    def forward(self, y=None, logits_out=None, ids_out=None):
        c, i = self.cfg, self.inp
        od = torch.float32 if c.out_dtype == moe.DTYPE_F32 else torch.bfloat16
        if y is None:
            y = torch.empty(self.T, c.hidden, dtype=od, device="cuda")
        moe.moe_forward(c, i["x"], i["w_router"], i["router_bias"], i["score_bias"], self.W, y, self.ws,
                        logits_out=logits_out, topk_ids_out=ids_out)
        return y

    def oracle_forward(self, logits):
        """Oracle layer output given the GPU's logits (whole batch)."""
        i = self.inp
        scales = {k: host(i.get(k)) for k in ("w13_scale", "w2_scale", "shared_w13_scale", "shared_w2_scale")}
        return O.forward(self.ocfg, host(i["x"]), host(i["w_router"]), host(i["w13"]), host(i["w2"]),
                         router_bias=host(i["router_bias"]), score_bias=host(i["score_bias"]),
                         shared_w13=host(i["shared_w13"]), shared_w2=host(i["shared_w2"]),
                         logits=host(logits), scales=scales)


def check_rows(got, want, dtype):
    """Routed expert rows against the oracle's, max |d| / RMS(want) per row.

    Both sides round each row to its bf16 carrier; where the exact value sits
    at a rounding boundary the two roundings land one bf16 step apart (2**-7
    relative at most), which is allowed per element. For e4m3 layers h is
    requantised on both sides and a code can land one e4m3 step apart, moving
    that row by one step of one h element times a column of W_d: 99% of rows
    meet the tolerance, every row 4x it."""
    tol = TOL[dtype]
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    slack = 2.0 ** -7 * np.abs(want) if dtype != "f32" else 0.0
    rms = math.sqrt(float(np.mean(want * want)))
    row_err = np.max(np.maximum(np.abs(got - want) - slack, 0.0), axis=1) / rms
    say(f"    rows: max err {float(np.max(row_err)):.2e}, 99th percentile {float(np.quantile(row_err, 0.99)):.2e}")
    if dtype in ("fp8", "mxfp4"):
        assert float(np.quantile(row_err, 0.99)) < tol
        assert float(np.max(row_err)) < 4 * tol
    else:
        assert float(np.max(row_err)) < tol
