"""Annealed BCJR-QAT on a synthetic least-squares toy: the method's training loop in miniature, on the GPU path.

The latent weights are trained through the soft codeword at temperature T while T anneals from T0 to a near-zero
T_end, and the hard Viterbi code of the latent weights is the result (gist.science Technical Summary, "Annealing";
T0 = 0.3 per "Schedule Correction (Skip-High-T)").  The forward is soft_quantize's soft codeword kernel, the backward
its exact gradient kernel.

Toy: W [64, 32] is 64 sequences of n = 32 weights on the L = 8 trellis; inputs X [256, 32] have column scales from 3
down to 0.05 and the target is Y = X W^T.  PTQ takes the Viterbi code of W, which minimises the weight error.  The
task weights the columns unequally, so training the latent weights on ||X w_soft^T - Y||^2 can find codes with a
lower task loss.  Plain SGD (lr 0.1) for 300 steps, T from 0.3 to 1e-4.  The last steps, near T_end, are sensitive
to rounding (the fp64 oracle run of one toy ends at 2.19, the float32 GPU run at 2.28, against PTQ's 2.31), so the
comparison with PTQ is made over twelve toys.
"""
import time

import numpy as np
import pytest
import torch

import differentiable_bcjr_amd as dba
import workloads

pytestmark = pytest.mark.gpu

L, K, N, R, M = 8, 2, 32, 64, 256
LR, STEPS = 0.1, 300


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    return torch.device("cuda:0")


def _toy(seed=7):
    rng = np.random.Generator(np.random.PCG64(seed))
    c = rng.standard_normal(1 << L)
    c = (c / c.std()).astype(np.float32)
    W = rng.standard_normal((R, N)).astype(np.float32)
    X = rng.standard_normal((M, N)) * np.geomspace(3.0, 0.05, N)
    return c, W, X, X @ W.T.astype(np.float64)


def _gpu_qat(dev, c, W, X, Y, temps):
    ct = torch.from_numpy(c).to(dev)
    Xt = torch.from_numpy(X.astype(np.float32)).to(dev)
    Yt = torch.from_numpy(Y.astype(np.float32)).to(dev)
    lat = torch.from_numpy(W.copy()).to(dev).requires_grad_(True)
    for T in temps:
        ws = dba.soft_quantize(lat, ct, L, K, T)
        loss = ((Xt @ ws.t() - Yt) ** 2).mean()
        (g,) = torch.autograd.grad(loss, lat)
        with torch.no_grad():
            lat -= LR * g
    return lat.detach()


def _task_loss(X, Y, Wq):
    return float(np.mean((X @ np.asarray(Wq, np.float64).T - Y) ** 2))


def test_qat_trajectory_matches_oracle_loop(oracle_mod, dev):
    """The first 20 annealed SGD steps: latent weights from the GPU path and from the same loop on the fp64 oracle."""
    c, W, X, Y = _toy()
    temps = dba.temperature_schedule(STEPS)[:20]
    got = _gpu_qat(dev, c, W, X, Y, temps).cpu().numpy()
    lat = W.astype(np.float64)
    for T in temps:
        ws, _ = oracle_mod.soft(lat.astype(np.float32), c, L, K, T)
        gws = (2.0 / (M * R)) * ((X @ ws.T - Y).T @ X)
        gw, _ = oracle_mod.grad(lat.astype(np.float32), c, gws.astype(np.float32), L, K, T)
        lat = lat - LR * gw
    moved = np.abs(lat - W).max()
    err = np.abs(got - lat).max()
    print(f"QAT toy, 20 steps: latent weights moved by up to {moved:.3e}; GPU vs oracle loop {err:.2e}", flush=True)
    assert moved > 1e-3 and err <= 1e-3 * moved


def _ratio(dev, seed, T0):
    """Task loss of the annealed-QAT hard code over that of the PTQ hard code, for one toy."""
    c, W, X, Y = _toy(seed)
    ct = torch.from_numpy(c).to(dev)
    _, w_ptq, _ = dba.viterbi_hard_code(torch.from_numpy(W).to(dev), ct, L, K)
    lat = _gpu_qat(dev, c, W, X, Y, dba.temperature_schedule(STEPS, T0=T0))
    _, w_qat, _ = dba.viterbi_hard_code(lat, ct, L, K)
    return _task_loss(X, Y, w_qat.cpu().numpy()) / _task_loss(X, Y, w_ptq.cpu().numpy())


def test_annealed_qat_beats_ptq(dev):
    """Twelve toys: the hard code after annealed QAT from T0 = 0.3 has a lower task loss than PTQ's.  Measured on this
    build: every toy below PTQ, mean ratio 0.948.  Starting hot (T0 = 1.0) is reported beside it: mean 0.961, with
    some toys ending above PTQ, the overshoot that the skip-high-T schedule avoids."""
    seeds = range(1, 13)
    cold = np.array([_ratio(dev, s, 0.3) for s in seeds])
    hot = np.array([_ratio(dev, s, 1.0) for s in seeds])
    print(f"QAT/PTQ task loss, T0 = 0.3: {np.round(cold, 3).tolist()} (mean {cold.mean():.4f}); "
          f"T0 = 1.0: {np.round(hot, 3).tolist()} (mean {hot.mean():.4f}, {(hot > 1).sum()} above PTQ)", flush=True)
    assert cold.mean() < 0.97 and (cold < 1.0).sum() >= 10


def test_annealed_qat_crystallises(dev):
    """At T_end the soft codeword of the trained latent weights is the Viterbi code (T -> 0 limit, abstract)."""
    c, W, X, Y = _toy()
    ct = torch.from_numpy(c).to(dev)
    temps = dba.temperature_schedule(STEPS)
    t0 = time.perf_counter()
    lat = _gpu_qat(dev, c, W, X, Y, temps)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    _, w_qat, _ = dba.viterbi_hard_code(lat, ct, L, K)
    ws_end = dba.soft_codeword(lat, ct, L, K, temps[-1])
    l_qat = _task_loss(X, Y, w_qat.cpu().numpy())
    l_soft = _task_loss(X, Y, ws_end.cpu().numpy())
    agree = float((ws_end - w_qat).abs().lt(1e-3).float().mean())
    print(f"QAT toy: hard code {l_qat:.4f}, soft codeword at T_end {l_soft:.4f}, {agree:.3f} of weights crystallised; "
          f"{STEPS} steps in {dt:.2f} s", flush=True)
    assert agree >= 0.99 and abs(l_soft - l_qat) <= 1e-3 * l_qat


def test_qat_step_time_at_layer_size(dev):
    """One QAT step on the 1024x1024 matrix (4096 sequences of 256 weights, L = 16, T = 0.1): soft codeword forward,
    exact gradient backward; with a trainable codebook the backward is the codebook-gradient kernel instead."""
    wl = workloads.WORKLOADS[2]
    ct = torch.from_numpy(wl.codebook()).to(dev)
    lat = torch.from_numpy(wl.weights()).to(dev).requires_grad_(True)
    up = torch.from_numpy(wl.upstream_grad()).to(dev)
    for train_codebook in (False, True):
        ct.requires_grad_(train_codebook)
        times = []
        for _ in range(3):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            ws = dba.soft_quantize(lat, ct, wl.L, wl.k, 0.1)
            (ws * up).sum().backward()
            torch.cuda.synchronize()
            times.append(time.perf_counter() - t0)
            lat.grad = None
            ct.grad = None
        print(f"QAT step at 1024x1024, L = 16 ({'codebook trained' if train_codebook else 'weights only'}): "
              f"{min(times) * 1e3:.1f} ms", flush=True)
        assert all(np.isfinite(times))
