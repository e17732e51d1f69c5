"""Float64 torch-autograd reference of the K-interval attention forward.

Used only as a pin for the oracle: the forward is written from the definitions
in "Pretraining Transformers with Quantized Softmax in Attention" (§3 Objects
and calibration, Reconstruction; App. A edge cases; App. B Weight-STE /
Prob-STE / FWM; App. C.2 (iii) strict forward), and its backward comes from
torch's automatic differentiation, a derivation route independent of the
oracle's closed forms.  torch's amax/amin split an extremum's gradient evenly
among tied entries, which is the tie convention the pages state.

Readings shared with the oracle (each a reading of a silent point, not a
formula copied from it): the clamp on t passes the gradient at its bounds;
degenerate MinMax rows use the constant width 1; Nearest rounds t = 1/2 up.

Gradient modes: "detached" detaches both row extrema; "max_only" / "min_only"
detach only the other extremum (the single-channel ablation of App. I); "p1"
is the detached gradient with a hook on the scores that projects each row's
gradient onto the zero-sum subspace over its visible keys (App. B "Detach").

FWM tail policies (App. C.3, App. D.4): "zero" drops keys below the window;
"floor" clamps z at -tau, so such a key weighs e^{-tau} and torch's clamp gives
it no gradient; "resolved" continues the grid b_q = -tau + q h to every integer
q below the window, with the grid value computed as exp(b_q) for any q.

Exponential baselines (App. B "Softmax", App. D.5 "Definitions"), written with
torch's own casts so that the backward is torch's native one: softmax (e^z);
BF16-exp (z cast to bfloat16, exp evaluated in bfloat16, cast back: autograd
then carries the gradient through the bfloat16 tensors in bfloat16); FP8-rounded
exp (e^z cast to float8_e4m3fn and back, plus e^z - sg(e^z), so the forward is
the rounded value and the derivative that of e^z).  The row maximum stays on the
gradient path (detached only in the detached, min_only and P1 modes).

Bin mean (§5, App. I; App. I.3 for the hybrid): the Nearest bins are taken from
the detached scores; each in-window key weighs the mean of e^z over its bin (a
scatter-add of torch.exp); the hybrid returns sg(P^N) + (P^C - sg(P^C)), so its
forward is the strict Nearest one and its gradient the bin mean's.
"""
import torch

DEGENERATE_EPS = 1e-12


def _st_clamp01(x):
    # value clamp(x, 0, 1); gradient of the identity (the bound is reached only by rounding)
    return x + (x.clamp(0.0, 1.0) - x).detach()


EXP_RECON = ("softmax", "exp_bf16", "exp_fp8")


def _exp_probs(s, mask, recon, grad):
    dt = s.dtype
    M = torch.where(mask, s, torch.tensor(-float("inf"), dtype=dt)).amax(dim=1, keepdim=True)
    if grad in ("detached", "p1", "min_only"):
        M = M.detach()
    z = torch.where(mask, s - M, torch.zeros_like(s))
    if recon == "softmax":
        w = torch.exp(z)
    elif recon == "exp_bf16":
        w = torch.exp(z.to(torch.bfloat16)).to(dt)
    else:
        we = torch.exp(z)
        w = we.detach().to(torch.float8_e4m3fn).to(dt) + (we - we.detach())
    w = torch.where(mask, w, torch.zeros_like(w))
    return w / w.sum(dim=1, keepdim=True)


def row_probs(s, mask, calib, recon, ste, grad, K, tau=8.0, tail_policy="zero"):
    """s: [R, n] float64, mask: [R, n] bool (visible keys).  Returns P [R, n]."""
    if recon in EXP_RECON:
        return _exp_probs(s, mask, recon, grad)
    dt = s.dtype
    pos_inf = torch.tensor(float("inf"), dtype=dt)
    M = torch.where(mask, s, -pos_inf).amax(dim=1, keepdim=True)
    m = torch.where(mask, s, pos_inf).amin(dim=1, keepdim=True)
    if grad in ("detached", "p1"):
        M, m = M.detach(), m.detach()
    elif grad == "max_only":
        m = m.detach()
    elif grad == "min_only":
        M = M.detach()
    rr = torch.arange(K + 1, dtype=dt)
    R = s.shape[0]
    if calib == "minmax":
        span = M - m
        deg = ~(span > DEGENERATE_EPS)
        h = torch.where(deg, torch.ones_like(span), span / K)
        b = (1.0 - rr / K) * (m - M)                        # [R, K+1]
        u = (s - m) / h
        tail = torch.zeros_like(mask)
    else:
        h = tau / K
        b = (-tau + rr * h).expand(R, K + 1)
        z = s - M
        if tail_policy == "resolved":
            tail = torch.zeros_like(mask)
            u = (torch.clamp(z, max=0.0) + tau) / h
        else:
            tail = (z < -tau).detach() if tail_policy == "zero" else torch.zeros_like(mask)
            u = (torch.clamp(z, -tau, 0.0) + tau) / h
    u_safe = torch.where(mask, u, torch.zeros_like(u))
    lo = None if (calib == "fwm" and tail_policy == "resolved") else 0
    r = torch.clamp(torch.floor(u_safe.detach()), lo, K - 1).long()
    t = _st_clamp01(u_safe - r.to(dt))
    ell = r + (t.detach() >= 0.5).long()
    if calib == "fwm":
        Er, Er1, EN = (torch.exp(-tau + q.to(dt) * h) for q in (r, r + 1, ell))
    else:
        E = torch.exp(b)
        Er, Er1, EN = (torch.gather(E, 1, q) for q in (r, r + 1, ell))
    wL = (1.0 - t) * Er + t * Er1
    wN = EN
    keep = mask & ~tail
    zero = torch.zeros_like(wL)
    wL = torch.where(keep, wL, zero)
    wN = torch.where(keep, wN, zero)
    if recon in ("binmean", "nearest_binmean"):
        # bins fixed (detached decisions); values e^{s - M} depend on the scores alone
        Mv = torch.where(mask, s, -pos_inf).amax(dim=1, keepdim=True).detach()
        ez = torch.where(keep, torch.exp(torch.where(keep, s - Mv, zero)), zero)
        bins = torch.where(keep, ell, torch.full_like(ell, K + 1))
        S = torch.zeros(R, K + 2, dtype=dt).scatter_add(1, bins, ez)
        cnt = torch.zeros(R, K + 2, dtype=dt).scatter_add(1, bins, keep.to(dt))
        wC = torch.where(keep, S.gather(1, bins) / cnt.gather(1, bins).clamp_min(1.0), zero)
        PC = wC / wC.sum(dim=1, keepdim=True)
        if recon == "binmean":
            return PC
        PN = (wN / wN.sum(dim=1, keepdim=True)).detach()
        return PN + (PC - PC.detach())
    if recon == "lerp":
        return wL / wL.sum(dim=1, keepdim=True)
    if ste == "weight":
        w = wL + (wN - wL).detach()
        return w / w.sum(dim=1, keepdim=True)
    PN = (wN / wN.sum(dim=1, keepdim=True)).detach()
    PL = wL / wL.sum(dim=1, keepdim=True)
    return PL + (PN - PL).detach()


def row_grad(s, g, calib, recon, ste, grad, K, tau=8.0, tail_policy="zero"):
    """Single row: returns (P, dS) as float64 tensors."""
    s = torch.as_tensor(s, dtype=torch.float64).reshape(1, -1).clone().requires_grad_(True)
    g = torch.as_tensor(g, dtype=torch.float64).reshape(1, -1)
    mask = torch.ones_like(s, dtype=torch.bool)
    P = row_probs(s, mask, calib, recon, ste, grad, K, tau, tail_policy)
    (P * g).sum().backward()
    dS = s.grad[0]
    if grad == "p1":
        dS = dS - dS.mean()
    return P.detach()[0], dS


def head_grad(Q, K_, V, dO, calib, recon, ste, grad, K, tau=8.0, causal=True, scale=None, tail_policy="zero"):
    """One head, materialized T x T in float64: returns O, dQ, dK, dV."""
    Q = torch.as_tensor(Q, dtype=torch.float64).clone().requires_grad_(True)
    Kt = torch.as_tensor(K_, dtype=torch.float64).clone().requires_grad_(True)
    V = torch.as_tensor(V, dtype=torch.float64).clone().requires_grad_(True)
    dO = torch.as_tensor(dO, dtype=torch.float64)
    T, D = Q.shape
    c = (1.0 / D ** 0.5) if scale is None else scale
    S = c * (Q @ Kt.T)
    mask = torch.ones(T, T, dtype=torch.bool)
    if causal:
        mask = torch.tril(mask)
    if grad == "p1":
        cnt = mask.sum(dim=1, keepdim=True).to(S.dtype)
        S.register_hook(lambda gS: torch.where(mask, gS - torch.where(mask, gS, 0.0).sum(1, keepdim=True) / cnt, gS))
    P = row_probs(S, mask, calib, recon, ste, grad, K, tau, tail_policy)
    O = P @ V
    (O * dO).sum().backward()
    return O.detach(), Q.grad, Kt.grad, V.grad
