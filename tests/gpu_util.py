"""Helpers for the GPU parity tests: device upload of the shared seeded inputs
and the comparison rules (tolerances are written in the tests that use them)."""

import numpy as np
import torch

from workloads import bf16_bits_to_f32

O_TOL_BF16 = 1e-2     # max-abs on O for the bf16 paths
O_TOL_QUANT = 3e-2    # max-abs on O for the quantised path
ML_RTOL = 1e-3        # softmax max / sum relative tolerance


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def f64(bits: np.ndarray) -> np.ndarray:
    return bf16_bits_to_f32(bits).astype(np.float64)


def to_np(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy().astype(np.float64)
    return t.cpu().numpy()


def check_o(o_gpu: np.ndarray, o_ref: np.ndarray, tol: float, what: str = "O"):
    assert o_gpu.shape == o_ref.shape, (o_gpu.shape, o_ref.shape)
    assert np.all(np.isfinite(o_gpu)), f"{what}: non-finite values"
    err = np.abs(o_gpu - o_ref).max() if o_ref.size else 0.0
    assert err <= tol, f"{what}: max abs error {err:.3e} > {tol}"
    return err


def check_o_channel_scaled(o_gpu: np.ndarray, o_ref: np.ndarray, v: np.ndarray, tol: float, what: str = "O"):
    """Max-abs check in units of each V channel's magnitude.

    The quantised tolerance is stated for N(0,1)-scale inputs; a V channel with
    scale c gives outputs (and errors) c times larger in that channel, so the
    error of channel d is divided by max(1, rms_d), rms_d being the RMS of V
    over the tokens of that (batch, kv-head, channel). o: [B, Nq, S, D];
    v: [B, Nkv, Skv, D] (float values)."""
    B, Nq = o_ref.shape[:2]
    g = Nq // v.shape[1]
    rms = np.sqrt((np.asarray(v, np.float64) ** 2).mean(axis=2))            # [B, Nkv, D]
    denom = np.maximum(1.0, np.repeat(rms, g, axis=1))[:, :, None, :]        # [B, Nq, 1, D]
    assert np.all(np.isfinite(o_gpu)), f"{what}: non-finite values"
    raw = np.abs(o_gpu - o_ref)
    err = (raw / denom).max() if o_ref.size else 0.0
    print(f"[gpu-test] {what}: channel-scaled max err {err:.3e} (raw max-abs {raw.max() if raw.size else 0:.3e})",
          flush=True)
    assert err <= tol, f"{what}: channel-scaled max error {err:.3e} > {tol}"
    return err


def check_ml(m_gpu, l_gpu, m_ref, l_ref, rtol: float = ML_RTOL, what: str = ""):
    """Rows with no kept key must give m = -inf and l = 0 exactly; elsewhere
    |dm| <= rtol * max(1, |m|) and |dl| <= rtol * l."""
    m_gpu, l_gpu, m_ref, l_ref = (np.asarray(x, dtype=np.float64) for x in (m_gpu, l_gpu, m_ref, l_ref))
    dead = np.isneginf(m_ref)
    assert np.array_equal(np.isneginf(m_gpu), dead), f"{what}: -inf pattern of softmax_max differs"
    assert np.all(l_gpu[dead] == 0), f"{what}: softmax_sum of empty rows must be 0"
    live = ~dead
    dm = np.abs(m_gpu[live] - m_ref[live]) / np.maximum(1.0, np.abs(m_ref[live]))
    dl = np.abs(l_gpu[live] - l_ref[live]) / l_ref[live]
    assert dm.size == 0 or dm.max() <= rtol, f"{what}: softmax_max rel err {dm.max():.3e}"
    assert dl.size == 0 or dl.max() <= rtol, f"{what}: softmax_sum rel err {dl.max():.3e}"


def banner(msg: str):
    print(f"[gpu-test] {msg}", flush=True)
