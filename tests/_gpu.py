"""Helpers shared by the GPU tests: move generator output to the device and
back, and compare against the float64 oracle at the stated tolerance."""
from __future__ import annotations

import functools

import numpy as np
import torch

import synth
import paged_kv_cache_reshape_amd as pa

# Tolerances.  Every element: |y - y*| <= atol + rtol * |y*| (bfloat16 inputs
# with float32 accumulation: atol 2e-3, rtol 1e-2; float32 inputs: 1e-5 both).
# On top of it the stated maxima where the output's own rounding leaves room
# for them: bfloat16 round-to-nearest-even costs at most half an ulp, 2^-10
# below |y| = 0.5 and at most 2^-8 |y| anywhere, so max abs <= 2e-3 is asserted
# over |y*| < 0.5 and max rel <= 1e-2 over |y*| >= 0.2 (float32: max abs <=
# 1e-5 over |y*| < 0.5, max rel <= 1e-5 over |y*| >= 0.2 is not asserted --
# near 0.2 it asks for 2e-6 absolute, below what float32 sums of thousands of
# terms guarantee -- the elementwise bound stands there).
TOL = {"bf16": (2e-3, 1e-2), "f32": (1e-5, 1e-5)}


def dev_tensor(arr: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    if dtype == "bf16" and arr.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(
            torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(arr)).to(device)


def host_storage(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> numpy array in the generator's storage convention."""
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def host_f64(t: torch.Tensor) -> np.ndarray:
    return t.to(torch.float64).cpu().numpy()


@functools.lru_cache(maxsize=3)
def cached_inputs(name: str, poison: bool = False, seed: int | None = None):
    return synth.make_inputs(synth.WORKLOADS[name], seed=seed, poison=poison)


def upload(inp: dict, device="cuda") -> dict:
    dt = inp["workload"].dtype
    return dict(
        q=dev_tensor(inp["q"], dt, device),
        key=dev_tensor(inp["key"], dt, device),
        value=dev_tensor(inp["value"], dt, device),
        k_cache=dev_tensor(inp["k_cache"], dt, device),
        v_cache=dev_tensor(inp["v_cache"], dt, device),
        block_tables=torch.from_numpy(inp["block_tables"]).to(device),
        context_lens=torch.from_numpy(inp["context_lens"]).to(device),
        slot_mapping=torch.from_numpy(inp["slot_mapping"]).to(device),
        scale=float(inp["scale"]),
    )


LITERAL = {"bf16": (2e-3, 1e-2), "f32": (1e-5, None)}


def assert_close(got: np.ndarray, ref: np.ndarray, dtype: str, what: str = ""):
    """Elementwise bound, then the literal maxima where they apply; returns
    (max abs error, max rel error over |y*| >= 0.2)."""
    atol, rtol = TOL[dtype]
    assert got.shape == ref.shape
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - ref)
    bad = err > atol + rtol * np.abs(ref)
    big = np.abs(ref) >= 0.2
    small = np.abs(ref) < 0.5
    max_rel = float((err[big] / np.abs(ref[big])).max()) if big.any() else 0.0
    max_abs_small = float(err[small].max()) if small.any() else 0.0
    assert not bad.any(), (f"{what}: {int(bad.sum())} of {bad.size} outside "
                           f"{atol} + {rtol}|y|; max abs {err.max():.3g}, "
                           f"max rel {max_rel:.3g}")
    lit_abs, lit_rel = LITERAL[dtype]
    assert max_abs_small <= lit_abs, (f"{what}: max abs error {max_abs_small:.3g} over "
                                      f"|y*| < 0.5 exceeds {lit_abs}")
    if lit_rel is not None:
        assert max_rel <= lit_rel, (f"{what}: max rel error {max_rel:.3g} over |y*| >= 0.2 "
                                    f"exceeds {lit_rel}")
    return float(err.max()), max_rel


def setopt(monkeypatch, name: str, value) -> None:
    """Set a PAGEDATTN_* override for this test and make the library see it
    (conftest re-reads the restored environment after the test)."""
    monkeypatch.setenv(name, str(value))
    pa.reload_options()
