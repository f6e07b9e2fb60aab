"""Shared helpers of the GPU parity tests: build inputs from the seeded
generator, run the HIP layer through the C ABI, and run the oracle on the
same bits.  Imported only by tests (and the smoke entry point)."""
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

from oracle import moe_oracle as O
from workloads import (bf16_bits_to_f32, expert_stack, expert_weight, router_inputs,
                       storage_bits)


def log(*a):
    print(f"[{time.strftime('%H:%M:%S')}]", *a, flush=True)


def to_device(cfg, a32_or_bits):
    """Host array (uint16 bf16 bits or float32) -> device tensor."""
    a = np.ascontiguousarray(a32_or_bits)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to("cuda").view(torch.bfloat16)
    return torch.from_numpy(a.astype(np.float32, copy=False)).to("cuda")


class LayerInputs:
    """x, W_gate and expert stacks of one config, on host and device."""

    def __init__(self, cfg, keep_host=True):
        self.cfg = cfg
        t = time.time()
        self.x, self.wg = router_inputs(cfg)
        self.stacks = {}
        dev = {}
        kinds = ["w1", "w3", "w2"] + (["ws1", "ws3", "ws2"] if cfg.E_shared else [])
        for kind in kinds:
            st = expert_stack(cfg, kind, bits=True)
            dev[kind] = to_device(cfg, st)
            if keep_host:
                self.stacks[kind] = st
            else:
                del st
        self.dev = dev
        self.x_dev = to_device(cfg, storage_bits(cfg, self.x))
        self.wg_dev = to_device(cfg, storage_bits(cfg, self.wg))
        torch.cuda.synchronize()
        log(f"inputs for {cfg.name} (T={cfg.T}) ready in {time.time() - t:.1f}s")

    def host_expert(self, kind, e):
        """float32 values of one expert (from the kept bits or regenerated)."""
        if kind in self.stacks:
            a = self.stacks[kind][e]
            return bf16_bits_to_f32(a) if a.dtype == np.uint16 else a
        return expert_weight(self.cfg, kind, e)

    def _routed64(self, e):
        return tuple(self.host_expert(k, e).astype(np.float64) for k in ("w1", "w3", "w2"))

    def load_routed(self, e):
        """fp64 weights of routed expert e.  The oracle asks for experts in
        increasing order, so the next few are widened ahead in threads."""
        if not hasattr(self, "_pool"):
            self._pool = ThreadPoolExecutor(max_workers=8)
            self._fut = {}
        for nxt in range(e, min(self.cfg.E, e + 8)):
            if nxt not in self._fut:
                self._fut[nxt] = self._pool.submit(self._routed64, nxt)
        for old in [k for k in self._fut if k < e]:
            del self._fut[old]
        return self._fut.pop(e).result()

    def load_shared(self, s):
        return tuple(self.host_expert(k, s) for k in ("ws1", "ws3", "ws2"))


def run_gpu(inp, bufs=None):
    import top_routing_expert_softmax_amd as M
    cfg = inp.cfg
    d = inp.dev
    b = M.layer_forward(inp.x_dev, inp.wg_dev, d["w1"], d["w3"], d["w2"], cfg.k, cfg.CF,
                        d.get("ws1"), d.get("ws3"), d.get("ws2"), bufs=bufs)
    torch.cuda.synchronize()
    return b


def host(b):
    """Copy every output of a layer run to numpy."""
    out = {}
    for name in ("logits", "topk_idx", "topk_w", "counts", "offsets", "token_of_row",
                 "row_of_pair", "drop_mask", "f", "P", "scalars"):
        out[name] = getattr(b, name).cpu().numpy()
    out["y"] = b.y.float().cpu().numpy()
    out["R"] = int(out["offsets"][-1])
    return out


def oracle_routing(inp):
    cfg = inp.cfg
    r = O.route(inp.x, inp.wg, cfg.k)
    counts = O.expert_counts(r["idx"], cfg.E)
    cap = O.capacity(cfg.T, cfg.E, cfg.k, cfg.CF)
    disp = O.dispatch(r["idx"], cfg.E, cap)
    stats = O.aux_stats(r["logits"], counts, cfg.T, cfg.k, cap)
    return r, counts, cap, disp, stats


def oracle_y(inp, r, disp, tokens):
    cfg = inp.cfg
    shared = None
    if cfg.E_shared:
        shared = np.zeros((len(tokens), cfg.d_model))
        for s in range(cfg.E_shared):
            shared += O.swiglu_expert(inp.x[tokens], *inp.load_shared(s))
    return O.combine_grouped(inp.x, r["weights"], r["idx"], disp, inp.load_routed, cfg.E,
                             tokens=np.asarray(tokens), shared_out=shared)


# ------------------------------------------------------------- comparisons --

def check_routing(g, r, counts, disp):
    """Everything integer (and the exact logits) must match bit for bit."""
    assert np.array_equal(g["logits"].astype(np.float64), r["logits"]), "logits differ"
    assert np.array_equal(g["topk_idx"], r["idx"]), "top-k indices differ"
    assert np.max(np.abs(g["topk_w"] - r["weights"])) <= 2e-6, "top-k weights differ"
    assert np.array_equal(g["counts"], counts), "counts differ"
    assert np.array_equal(g["offsets"], disp["offsets"]), "offsets differ"
    assert np.array_equal(g["row_of_pair"], disp["row_of_pair"]), "row_of_pair differs"
    assert np.array_equal(g["drop_mask"], disp["drop"]), "drop mask differs"
    assert np.array_equal(g["token_of_row"], disp["token_of_row"]), "token_of_row differs"


def check_stats(g, stats, rel=1e-5):
    def close(a, b):
        return abs(a - b) <= rel * max(abs(b), 1e-30)
    assert np.allclose(g["f"], stats["f"], rtol=1e-6, atol=0), "f differs"
    assert np.allclose(g["P"], stats["P"], rtol=rel, atol=1e-7), "P differs"
    assert close(g["scalars"][0], stats["L_balance"]), (g["scalars"][0], stats["L_balance"])
    assert close(g["scalars"][1], stats["z_loss"]), (g["scalars"][1], stats["z_loss"])
    assert abs(g["scalars"][2] - stats["drop_rate"]) <= 1e-12, (g["scalars"][2], stats["drop_rate"])


def y_errors(y, ref):
    """max |err| / max |ref| and sum |err| / sum |ref|."""
    err = np.abs(y.astype(np.float64) - ref)
    return float(err.max() / max(np.abs(ref).max(), 1e-30)), \
        float(err.sum() / max(np.abs(ref).sum(), 1e-30))


def check_y(cfg, y, ref):
    mx, mean_rel = y_errors(y, ref)
    if cfg.dtype == "f32":
        assert mx <= 1e-4, f"fp32 max error {mx:.3e} > 1e-4 of max|ref|"
    else:
        assert mx <= 2e-2, f"bf16 max error {mx:.3e} > 2e-2 of max|ref|"
        assert mean_rel <= 5e-3, f"bf16 mean relative error {mean_rel:.3e} > 5e-3"
    return mx, mean_rel
