"""Seeded generators for x, W_gate and the expert weight stacks.

Every tensor is drawn from numpy's PCG64 with a seed derived from
(config seed, tensor code, expert index), so one expert can be regenerated on
its own.  bf16 configs round each value once, round-to-nearest-even, and both
sides receive those exact bits.

Storage layouts (what the C-ABI takes):
  x       [T, d]      row-major
  w_gate  [d, E]      row-major (the pages' W_gate in R^{d x E})
  w1, w3  [E, F, d]   row f of expert e holds column f of that expert's W1/W3
  w2      [E, d, F]   row i of expert e holds column i of that expert's W2
  ws1, ws3, ws2       the same for the E_shared shared experts
i.e. each stored row is one output feature's weights along the contracted
dimension (the [out, in] layout of a linear layer).
"""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from .configs import MoEConfig

_TENSOR_CODE = {"x": 1, "w_gate": 2, "zipf": 3,
                "w1": 11, "w3": 13, "w2": 12, "ws1": 21, "ws3": 23, "ws2": 22}


def _rng(cfg: MoEConfig, tensor: str, index: int = 0) -> np.random.Generator:
    ss = np.random.SeedSequence(entropy=cfg.seed,
                                spawn_key=(_TENSOR_CODE[tensor], index))
    return np.random.Generator(np.random.PCG64(ss))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest even."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    b = a.view(np.uint32)
    r = (b >> np.uint32(16)) & np.uint32(1)
    b = (b + np.uint32(0x7FFF) + r) >> np.uint32(16)
    return b.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32)
            << np.uint32(16)).view(np.float32)


def _round_to_dtype(cfg: MoEConfig, a32: np.ndarray) -> np.ndarray:
    if cfg.dtype == "bf16":
        return bf16_bits_to_f32(f32_to_bf16_bits(a32))
    return a32


def storage_bits(cfg: MoEConfig, a32: np.ndarray) -> np.ndarray:
    """What goes to the device: uint16 bf16 bits or the float32 array."""
    if cfg.dtype == "bf16":
        return f32_to_bf16_bits(a32)
    return np.ascontiguousarray(a32, dtype=np.float32)


def _x_ints(cfg: MoEConfig) -> np.ndarray:
    g = _rng(cfg, "x")
    shape = (cfg.T, cfg.d_model)
    if cfg.x_kind == "uniform16":
        m = g.integers(-8, 9, size=shape, dtype=np.int64)
    elif cfg.x_kind == "gauss16":
        m = np.clip(np.rint(16.0 * g.standard_normal(shape)), -128, 128).astype(np.int64)
    else:
        raise ValueError(cfg.x_kind)
    if cfg.zipf_s > 0:
        m[:, 0] = 16          # the constant-one input feature
    return m


def zipf_offsets(cfg: MoEConfig) -> np.ndarray:
    """Per-expert logit offsets -tau*s*ln(rank), rank a seeded permutation of
    1..E, rounded to multiples of 2**-6 (exact in bf16 while |o| < 4)."""
    ranks = _rng(cfg, "zipf").permutation(cfg.E) + 1
    o = np.rint(64.0 * (-cfg.zipf_tau * cfg.zipf_s * np.log(ranks))) / 64.0
    if np.max(np.abs(o)) >= 4.0:
        raise ValueError("Zipf offsets leave the bf16-exact range; lower zipf_tau")
    return o


def _wg_ints(cfg: MoEConfig) -> np.ndarray:
    g = _rng(cfg, "w_gate")
    shape = (cfg.d_model, cfg.E)
    if cfg.wg_kind == "uniform":
        n = g.integers(-8, 9, size=shape, dtype=np.int64)
    elif cfg.wg_kind == "gauss":
        n = np.clip(np.rint(cfg.wg_sd * g.standard_normal(shape)), -255, 255).astype(np.int64)
    else:
        raise ValueError(cfg.wg_kind)
    if cfg.zipf_s > 0:
        # row 0 meets the constant feature; offsets o = n0 * 2**-wg_shift
        n[0, :] = np.rint(zipf_offsets(cfg) * 2.0 ** cfg.wg_shift).astype(np.int64)
    return n


def router_inputs(cfg: MoEConfig, check_grid: bool = True):
    """x [T,d] and W_gate [d,E] as float32 arrays holding exact grid values.

    With check_grid the integer bound sum_i |m_ti n_ie| < 2**24 is asserted
    for every (t, e), so fp32 accumulation of x.W_gate in any order is exact.
    """
    m = _x_ints(cfg)
    n = _wg_ints(cfg)
    if check_grid:
        # float64 BLAS is exact here: every partial sum is an integer < 2**53
        bound = np.abs(m).astype(np.float64) @ np.abs(n).astype(np.float64)
        worst = float(bound.max())
        if worst >= 2.0 ** 24:
            raise AssertionError(f"router grid bound violated: {worst} >= 2**24")
    x = (m.astype(np.float64) * 2.0 ** -4).astype(np.float32)
    wg = (n.astype(np.float64) * 2.0 ** -cfg.wg_shift).astype(np.float32)
    # every value is exact in the layer dtype by construction
    assert np.array_equal(_round_to_dtype(cfg, x), x)
    assert np.array_equal(_round_to_dtype(cfg, wg), wg)
    return x, wg


def _expert_shape(cfg: MoEConfig, kind: str):
    if kind in ("w1", "w3", "ws1", "ws3"):
        return (cfg.d_ff, cfg.d_model)
    if kind in ("w2", "ws2"):
        return (cfg.d_model, cfg.d_ff)
    raise ValueError(kind)


def expert_weight(cfg: MoEConfig, kind: str, e: int, bits: bool = False) -> np.ndarray:
    """One expert's weight in storage layout: float32 values (rounded to the
    layer dtype) or, with bits=True, the device storage (uint16 for bf16)."""
    g = _rng(cfg, kind, e)
    a = g.standard_normal(_expert_shape(cfg, kind), dtype=np.float32)
    a *= np.float32(cfg.w_sd)
    if bits:
        return storage_bits(cfg, a)
    return _round_to_dtype(cfg, a)


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def expert_stack(cfg: MoEConfig, kind: str, bits: bool = True, out=None) -> np.ndarray:
    """All experts of one kind stacked: [E or E_shared, rows, cols].

    kind in w1/w3/w2 (routed) or ws1/ws3/ws2 (shared).  Generated with a
    thread pool, one expert per task (numpy's generators release the GIL)."""
    n_exp = cfg.E_shared if kind.startswith("ws") else cfg.E
    shape = (n_exp,) + _expert_shape(cfg, kind)
    if bits and cfg.dtype == "bf16":
        dt = np.uint16
    else:
        dt = np.float32
    if out is None:
        out = np.empty(shape, dtype=dt)

    def work(e):
        out[e] = expert_weight(cfg, kind, e, bits=bits)

    if n_exp:
        with ThreadPoolExecutor(max_workers=_threads()) as ex:
            list(ex.map(work, range(n_exp)))
    return out
