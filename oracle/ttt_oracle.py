"""Plain CPU oracle for the TTT-Linear fast-weight scan.

TEST INFRASTRUCTURE ONLY.  This module is the slow, obviously correct
reference that the GPU path is checked against.  Only the test suite, the
smoke check and the CPU-baseline leg of the benchmark may import it; the
product path never calls it, and it imports nothing from the GPU package.

Arithmetic is float64 NumPy (a ``dtype`` argument exists only so that the
conditioning of a workload can be probed by re-running in float32).  The
code is vectorised over the independent (batch, head) axis only; the time
axis is an explicit Python loop in the order the pages state the method.

Sources (web pages, cited by title and section):

* "Edifice.Recurrent.TTT" (hexdocs), sections "Paper-Faithful
  Implementation", "Equations (TTT-Linear)" and "Architecture": the
  per-token recurrence, the 1/d scaling of the inner learning rate, the
  learnable inner LayerNorm, the sigmoid output gate applied to the output
  of the *updated* inner weight, and the straight-through inner gradient
  ``grad_W = error_t k_t^T``.
* "Error Correction in Trained TTT Layers" (aiqbench), abstract: the inner
  gradient of the LayerNorm squared-error objective with the LayerNorm
  Jacobian retained ("exact" mode).
* "PonderTTT", section "Technical Architecture" (dual-form updates) and
  "cortex_rust ... layers/ttt.rs", ``forward_chunkwise`` (every token of a
  chunk takes its gradient at the chunk-start weight, last chunk may be
  short): the mini-batch / dual mode.
* "cortex_rust ... layers/ttt.rs", ``TTT_NORM_EPS``: epsilon 1e-6.

Readings taken where the pages are silent (each is listed in the design
notes): epsilon sits inside the square root, the LayerNorm variance is the
biased (1/d) one, gamma/beta are per head, eta is one scalar per
(batch, head, token), the gate is elementwise, the output uses the updated
weight, the loss is 0.5*||.||^2, the dual-mode causal sum is inclusive, and
a final short chunk uses the same rule.

Parity status of each public function is stated in its docstring; the
forward functions are pinned by ``tests/test_oracle.py``, the backward
(``ttt_linear_backward`` and its helpers) by ``tests/test_oracle_backward.py``
and the two-layer inner model (``mlp_inner_grads``, ``ttt_mlp_forward``) by
``tests/test_oracle_mlp.py``.
"""
from __future__ import annotations

import numpy as np

#: LayerNorm epsilon.  The cortex_rust page fixes 1e-6 as its normalisation
#: epsilon (``TTT_NORM_EPS``); it is used here inside the square root.
EPS = 1e-6

#: Inner-gradient choices.
LN_ST = "st"        # gradient of 0.5||pred - v||^2 w.r.t. pred, times k^T
LN_EXACT = "exact"  # LayerNorm Jacobian applied (Error Correction ... abstract)
LN_NONE = "none"    # inner LayerNorm removed (diagnostic: delta rule)


def sigmoid(x: np.ndarray) -> np.ndarray:
    """Logistic function, written so that +-inf map to exactly 1 and 0."""
    x = np.asarray(x)
    out = np.empty_like(x)
    pos = x >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-x[pos]))
    ex = np.exp(x[~pos])
    out[~pos] = ex / (1.0 + ex)
    return out


def silu(x: np.ndarray) -> np.ndarray:
    """SiLU, x * sigmoid(x): the activation the `:mlp` variant of
    "Edifice.Recurrent.TTT" (Options, `:variant`) applies to keys and queries
    before the inner model.  Pinned against torch's silu."""
    return np.asarray(x) * sigmoid(x)


def silu_grad(x: np.ndarray) -> np.ndarray:
    """d silu / dx = sigmoid(x) (1 + x (1 - sigmoid(x))).  Pinned by autograd."""
    s = sigmoid(x)
    return s * (1.0 + np.asarray(x) * (1.0 - s))


def layer_norm(z: np.ndarray, gamma: np.ndarray, beta: np.ndarray, eps: float = EPS):
    """Learnable LayerNorm over the last axis.

    "Edifice.Recurrent.TTT", "Paper-Faithful Implementation" item 3 and
    "Equations (TTT-Linear)": ``pred_t = LayerNorm(W_{t-1} k_t)``.
    Returns ``(pred, xhat, s)`` with ``s = sqrt(var + eps)`` (biased variance).
    Pinned against ``torch.nn.functional.layer_norm``.
    """
    d = z.shape[-1]
    mu = z.sum(axis=-1, keepdims=True) / d
    c = z - mu
    var = (c * c).sum(axis=-1, keepdims=True) / d
    s = np.sqrt(var + eps)
    xhat = c / s
    return gamma * xhat + beta, xhat, s


def ln_jacobian(xhat: np.ndarray, s: np.ndarray, gamma: np.ndarray) -> np.ndarray:
    """Explicit Jacobian d pred / d z of the learnable LayerNorm.

    J[..., i, m] = gamma_i / s * (delta_im - 1/d - xhat_i xhat_m / d).
    Used by the exact inner gradient ("Error Correction in Trained TTT
    Layers", abstract: the inner gradient of the LayerNorm squared-error
    objective).  Pinned by finite differences and by autograd through
    ``torch.nn.functional.layer_norm``.
    """
    d = xhat.shape[-1]
    eye = np.eye(d, dtype=xhat.dtype)
    core = eye - 1.0 / d - xhat[..., :, None] * xhat[..., None, :] / d
    return (gamma[..., :, None] / s[..., None]) * core


def inner_grad_vector(z, v, gamma, beta, ln: str, eps: float = EPS):
    """The vector delta such that the inner update is ``W -= eta * delta k^T``.

    * ``st``: delta = LN(z) - v  ("Equations (TTT-Linear)": grad_W = error k^T)
    * ``exact``: delta = J^T (LN(z) - v), the gradient of
      0.5*||LN(z) - v||^2 with respect to z ("Error Correction ..." abstract)
    * ``none``: delta = z - v (LayerNorm removed; the delta rule of the
      "Key Innovations" equivalence with linear attention)
    """
    if ln == LN_NONE:
        return z - v
    pred, xhat, s = layer_norm(z, gamma, beta, eps)
    err = pred - v
    if ln == LN_ST:
        return err
    if ln == LN_EXACT:
        jac = ln_jacobian(xhat, s, gamma)
        return np.matmul(np.swapaxes(jac, -1, -2), err[..., None])[..., 0]
    raise ValueError(f"unknown ln mode {ln!r}")


def ttt_linear_forward(q, k, v, eta_logit, gate_logit, W0, gamma=None, beta=None,
                       *, ln: str = LN_ST, dual: bool = False, chunk: int = 16,
                       eps: float = EPS, dtype=np.float64, update_mask=None,
                       silu_qk: bool = False, return_ln_stats: bool = False):
    """The TTT-Linear scan, token by token.

    Shapes (row-major): q, k, v, gate_logit [B,H,T,d]; eta_logit [B,H,T];
    W0 [B,H,d,d] with z = W k meaning z_i = sum_j W[i,j] k_j; gamma, beta
    [H,d] (ignored when ``ln == "none"``).  Returns ``(out [B,H,T,d],
    W_final [B,H,d,d])`` in ``dtype``.

    For each token t ("Equations (TTT-Linear)" and "Architecture" of
    "Edifice.Recurrent.TTT"):

      eta_t   = sigmoid(eta_logit_t) / d           (1/d: "Paper-Faithful" item 2)
      z_t     = P k_t, with P = W (per-token) or P = W_c, the weight at the
                start of t's chunk (dual mode: "PonderTTT" dual-form updates,
                "cortex_rust" forward_chunkwise)
      delta_t = inner_grad_vector(z_t, v_t)        (LN then error; see above)
      W       = W - eta_t * delta_t k_t^T
      o_t     = (W q_t) * sigmoid(gate_logit_t)    (updated W, sigmoid gate)

    ``silu_qk``: the `:mlp` variant of "Edifice.Recurrent.TTT" (Options,
    `:variant`): SiLU is applied to k_t and q_t before the inner model, so
    z_t = W silu(k_t) and o_t = (W_t silu(q_t)) * sigmoid(g_t); silu(k_t) also
    takes k_t's place in the update.

    ``update_mask`` (dual mode only): [B,H,ceil(T/chunk)], one SKIP (0) /
    UPDATE (nonzero) decision per chunk ("PonderTTT", "Core Idea" and
    "Technical Architecture": learned SKIP/UPDATE decisions per input
    chunk).  A skipped chunk applies no update: its tokens take eta_t = 0, so
    W passes the chunk unchanged and the chunk's outputs read W_c q_t.

    ``return_ln_stats``: also return ``{"mean": [B,H,T], "std": [B,H,T],
    "delta": [B,H,T,d]}``: the mean and the (biased) standard deviation over
    the d features of every z_t that enters the LayerNorm (a diagnostic of how
    far off-centre the LayerNorm's inputs are; zeros without LayerNorm), and
    every inner-gradient vector delta_t.

    Parity: pinned (eta -> 0 closed form, delta-rule unrolled product,
    autograd inner-gradient steps, finite differences, dual-form special
    cases, overwrite and cancellation identities, resume, independence; the
    mask against eta_logit = -inf on its skipped chunks).
    """
    f = lambda a: None if a is None else np.asarray(a, dtype=dtype)
    q, k, v, eta_logit, gate_logit, W0 = map(f, (q, k, v, eta_logit, gate_logit, W0))
    if silu_qk:
        q, k = silu(q), silu(k)
    B, H, T, d = q.shape
    if ln != LN_NONE:
        gamma = f(gamma)[None, :, :]   # [1,H,d], broadcast over batch
        beta = f(beta)[None, :, :]
    if dual and chunk < 1:
        raise ValueError("chunk must be >= 1 in dual mode")
    keep = None
    if update_mask is not None:
        if not dual:
            raise ValueError("update_mask needs dual mode")
        keep = np.asarray(update_mask) != 0
        if keep.shape != (B, H, -(-T // chunk)):
            raise ValueError(f"update_mask must be [B,H,ceil(T/chunk)], got {keep.shape}")

    W = W0.copy()
    out = np.zeros((B, H, T, d), dtype=dtype)
    z_mean = np.zeros((B, H, T), dtype=dtype)
    z_std = np.zeros((B, H, T), dtype=dtype)
    deltas = np.zeros((B, H, T, d), dtype=dtype) if return_ln_stats else None
    eta_all = sigmoid(eta_logit) / dtype(d)
    gate_all = sigmoid(gate_logit)
    Wc = W
    for t in range(T):
        if dual and t % chunk == 0:
            Wc = W.copy()
        P = Wc if dual else W
        kt = k[:, :, t, :]
        z = np.matmul(P, kt[..., None])[..., 0]
        if return_ln_stats and ln != LN_NONE:
            z_mean[:, :, t] = z.mean(axis=-1)
            z_std[:, :, t] = np.sqrt(((z - z_mean[:, :, t][..., None]) ** 2).mean(axis=-1))
        delta = inner_grad_vector(z, v[:, :, t, :], gamma, beta, ln, eps)
        if return_ln_stats:
            deltas[:, :, t, :] = delta
        eta = eta_all[:, :, t][..., None, None]
        if keep is not None:
            eta = np.where(keep[:, :, t // chunk][..., None, None], eta, dtype(0))
        W = W - eta * (delta[..., :, None] * kt[..., None, :])
        out[:, :, t, :] = np.matmul(W, q[:, :, t, :][..., None])[..., 0] * gate_all[:, :, t, :]
    if return_ln_stats:
        return out, W, dict(mean=z_mean, std=z_std, delta=deltas)
    return out, W


def ln_jacobian_derivative(xhat: np.ndarray, s: np.ndarray, gamma: np.ndarray) -> np.ndarray:
    """Derivative of the LayerNorm Jacobian: D[..., i, m, p] = d J[i, m] / d z_p.

    With N[i, m] = (delta_im - 1/d - xhat_i xhat_m / d) / s (so J = gamma_i N),
    d s / d z_p = xhat_p / d and d xhat_i / d z_p = N[i, p]:

      D[i, m, p] = gamma_i * ( -(xhat_p / (d s)) N[i, m]
                               - (N[i, p] xhat_m + xhat_i N[m, p]) / (d s) )

    The backward of the exact inner gradient needs it (delta = J^T e with both
    J and e functions of z).  Pinned by finite differences of ``ln_jacobian``.
    """
    d = xhat.shape[-1]
    eye = np.eye(d, dtype=xhat.dtype)
    N = (eye - 1.0 / d - xhat[..., :, None] * xhat[..., None, :] / d) / s[..., None]
    ds = s[..., None, None] * d
    term1 = -(xhat[..., None, None, :] / ds) * N[..., :, :, None]
    term2 = -(N[..., :, None, :] * xhat[..., None, :, None]
              + xhat[..., :, None, None] * N[..., None, :, :]) / ds
    return gamma[..., :, None, None] * (term1 + term2)


def inner_grad_vector_vjp(dd, z, v, gamma, beta, ln: str, eps: float = EPS):
    """Vector-Jacobian product of ``inner_grad_vector``.

    Given dd = dL/d delta, returns ``(dz, dv, dgamma, dbeta)`` (dgamma and dbeta
    per (batch, head) row, before summing over batch and tokens; None without
    LayerNorm), from the explicit Jacobians of each step:

    * ``none``:  delta = z - v
    * ``st``:    delta = gamma xhat + beta - v, d delta / d z = J
    * ``exact``: delta = J^T e with e = gamma xhat + beta - v;
                 d delta_m / d z_p = sum_i D[i, m, p] e_i + (J^T J)[m, p],
                 d delta_m / d gamma_i = N[i, m] (e_i + gamma_i xhat_i),
                 d delta / d beta = J^T, d delta / d v = -J^T.
    """
    if ln == LN_NONE:
        return dd, -dd, None, None
    pred, xhat, s = layer_norm(z, gamma, beta, eps)
    jac = ln_jacobian(xhat, s, gamma)                      # [.., i, m]
    mv = lambda M, x: np.matmul(M, x[..., None])[..., 0]
    if ln == LN_ST:
        dz = mv(np.swapaxes(jac, -1, -2), dd)              # J^T dd
        return dz, -dd, dd * xhat, dd
    if ln == LN_EXACT:
        e = pred - v
        dJ = ln_jacobian_derivative(xhat, s, gamma)         # [.., i, m, p]
        d_delta_dz = (np.einsum("...imp,...i->...mp", dJ, e)
                      + np.matmul(np.swapaxes(jac, -1, -2), jac))
        dz = mv(np.swapaxes(d_delta_dz, -1, -2), dd)       # sum_m dd_m d delta_m / d z_p
        de = mv(jac, dd)                                    # J dd
        d = z.shape[-1]
        N = (np.eye(d, dtype=z.dtype) - 1.0 / d
             - xhat[..., :, None] * xhat[..., None, :] / d) / s[..., None]
        dgamma = mv(N, dd) * (e + gamma * xhat)
        return dz, -de, dgamma, de
    raise ValueError(f"unknown ln mode {ln!r}")


def ttt_linear_backward(q, k, v, eta_logit, gate_logit, W0, gamma, beta, dout, dW_final=None,
                        *, ln: str = LN_ST, dual: bool = False, chunk: int = 16,
                        eps: float = EPS, dtype=np.float64, silu_qk: bool = False):
    """Gradients of the scan: reverse-mode through ``ttt_linear_forward``.

    For a loss L with dL/d out = ``dout`` [B,H,T,d] and dL/d W_final =
    ``dW_final`` [B,H,d,d] (None: zero), returns a dict with dq, dk, dv,
    dgate_logit [B,H,T,d], deta_logit [B,H,T], dW0 [B,H,d,d] and dgamma,
    dbeta [H,d] (summed over batch and tokens; None without LayerNorm).

    The forward is replayed once, keeping every W_t; the tokens are then
    walked backwards undoing the forward's steps in reverse order:

      o_t = y_t * sigmoid(g_t), y_t = W_t q_t
        -> d y_t = dout_t * sigmoid(g_t),
           d g_t = dout_t * y_t * sigmoid'(g_t),
           dW_t += d y_t q_t^T,   dq_t = W_t^T d y_t
      W_t = W_{t-1} - eta_t delta_t k_t^T
        -> d eta_t = -delta_t^T dW_t k_t,  d delta_t = -eta_t dW_t k_t,
           dk_t += -eta_t dW_t^T delta_t,  dW_{t-1} += dW_t,
           d eta_logit_t = d eta_t sigmoid'(eta_logit_t) / d
      delta_t = inner_grad_vector(z_t, v_t)  -> inner_grad_vector_vjp
      z_t = P k_t (P = W_{t-1}, or the chunk-start W_c in the dual form)
        -> dP += dz_t k_t^T,  dk_t += P^T dz_t

    In the dual form dP accumulates over the chunk and joins dW at the
    chunk's first token.  With ``silu_qk`` the walk runs on silu(q), silu(k)
    and the last step multiplies dq, dk by silu'(q), silu'(k).  Parity: pinned
    by central finite differences of the forward and by autograd
    (``tests/test_oracle_backward.py``, ``tests/test_oracle_silu.py``).
    """
    f = lambda a: None if a is None else np.asarray(a, dtype=dtype)
    q, k, v, eta_logit, gate_logit, W0, dout = map(f, (q, k, v, eta_logit, gate_logit, W0, dout))
    q_in, k_in = q, k
    if silu_qk:
        q, k = silu(q), silu(k)
    B, H, T, d = q.shape
    has_ln = ln != LN_NONE
    if has_ln:
        gam = f(gamma)[None, :, :]
        bet = f(beta)[None, :, :]
    else:
        gam = bet = None
    mv = lambda M, x: np.matmul(M, x[..., None])[..., 0]
    outer = lambda a, b: a[..., :, None] * b[..., None, :]

    # replay the forward, keeping W after every token
    eta_all = sigmoid(eta_logit) / dtype(d)
    gate_all = sigmoid(gate_logit)
    Ws = np.empty((T + 1, B, H, d, d), dtype=dtype)
    Ws[0] = W0
    start = np.zeros(T, dtype=np.int64)          # index into Ws of the gradient point
    for t in range(T):
        start[t] = (t - t % chunk) if dual else t
        P = Ws[start[t]]
        z = mv(P, k[:, :, t, :])
        delta = inner_grad_vector(z, v[:, :, t, :], gam, bet, ln, eps)
        Ws[t + 1] = Ws[t] - eta_all[:, :, t][..., None, None] * outer(delta, k[:, :, t, :])

    g = {n: np.zeros_like(q) for n in ("dq", "dk", "dv", "dgate_logit")}
    g["deta_logit"] = np.zeros_like(eta_logit)
    dgamma = np.zeros((B, H, d), dtype=dtype) if has_ln else None
    dbeta = np.zeros((B, H, d), dtype=dtype) if has_ln else None
    dW = np.zeros((B, H, d, d), dtype=dtype) if dW_final is None else f(dW_final).copy()
    dP = np.zeros_like(dW)                        # dual form: gradient at the chunk-start W
    for t in range(T - 1, -1, -1):
        kt, qt, vt = k[:, :, t, :], q[:, :, t, :], v[:, :, t, :]
        eta = eta_all[:, :, t]
        sg = gate_all[:, :, t, :]
        Wt = Ws[t + 1]
        P = Ws[start[t]]
        z = mv(P, kt)
        delta = inner_grad_vector(z, vt, gam, bet, ln, eps)
        # output
        y = mv(Wt, qt)
        dy = dout[:, :, t, :] * sg
        g["dgate_logit"][:, :, t, :] = dout[:, :, t, :] * y * sg * (1.0 - sg)
        dW = dW + outer(dy, qt)
        g["dq"][:, :, t, :] = mv(np.swapaxes(Wt, -1, -2), dy)
        # update
        dWk = mv(dW, kt)
        deta = -(delta * dWk).sum(axis=-1)
        ddelta = -eta[..., None] * dWk
        dk = -eta[..., None] * mv(np.swapaxes(dW, -1, -2), delta)
        sl = sigmoid(eta_logit[:, :, t])
        g["deta_logit"][:, :, t] = deta * sl * (1.0 - sl) / dtype(d)
        # inner gradient
        dz, dv, dga, dbe = inner_grad_vector_vjp(ddelta, z, vt, gam, bet, ln, eps)
        g["dv"][:, :, t, :] = dv
        if has_ln:
            dgamma += dga
            dbeta += dbe
        # z = P k
        dk = dk + mv(np.swapaxes(P, -1, -2), dz)
        g["dk"][:, :, t, :] = dk
        if dual:
            dP = dP + outer(dz, kt)
            if start[t] == t:                      # first token of its chunk
                dW = dW + dP
                dP = np.zeros_like(dP)
        else:
            dW = dW + outer(dz, kt)
    if silu_qk:
        g["dq"] = g["dq"] * silu_grad(q_in)
        g["dk"] = g["dk"] * silu_grad(k_in)
    g["dW0"] = dW
    g["dgamma"] = dgamma.sum(axis=0) if has_ln else None
    g["dbeta"] = dbeta.sum(axis=0) if has_ln else None
    return g


def mlp_inner_grads(W1, W2, k, v, gamma, beta, ln: str, eps: float = EPS):
    """Gradients of the two-layer inner model's loss for one token.

    The inner model is f(x) = W2 silu(W1 x): a reading of "Edifice.Recurrent.TTT",
    Options, `:variant`, which says the `:mlp` variant turns the hidden state
    into a two-layer MLP with SiLU, and of "Error Correction in Trained TTT
    Layers", abstract, which trains TTT-MLP under the same LayerNorm
    squared-error objective as TTT-Linear.  With
    h = W1 k, a = silu(h), z = W2 a and delta_z the gradient of the loss with
    respect to z (``inner_grad_vector``: straight-through, exact or without
    LayerNorm), the chain rule gives

        dL/dW2 = delta_z a^T
        dL/dW1 = ((W2^T delta_z) * silu'(h)) k^T

    with W1, W2 the weights before the update.  Returns ``(dW1, dW2)``.
    Pinned by torch autograd of the loss and by central finite differences
    (tests/test_oracle_mlp.py).
    """
    mv = lambda M, x: np.matmul(M, x[..., None])[..., 0]
    outer = lambda a, b: a[..., :, None] * b[..., None, :]
    h = mv(W1, k)
    a = silu(h)
    z = mv(W2, a)
    dz = inner_grad_vector(z, v, gamma, beta, ln, eps)
    da = mv(np.swapaxes(W2, -1, -2), dz)
    dh = da * silu_grad(h)
    return outer(dh, k), outer(dz, a)


def ttt_mlp_forward(q, k, v, eta_logit, gate_logit, W1_0, W2_0, gamma=None, beta=None,
                    *, ln: str = LN_ST, dual: bool = False, chunk: int = 16,
                    eps: float = EPS, dtype=np.float64):
    """The scan with a two-layer inner model f(x) = W2 silu(W1 x), token by token.

    Shapes: q, k, v, gate_logit [B,H,T,d]; eta_logit [B,H,T]; W1_0, W2_0
    [B,H,d,d] (hidden width d); gamma, beta [H,d].  Returns ``(out, W1_final,
    W2_final)``.  For each token t (the TTT-Linear steps of "Edifice.Recurrent.TTT",
    "Equations (TTT-Linear)", with the inner model replaced):

      eta_t = sigmoid(eta_logit_t) / d
      (dW1, dW2) = mlp_inner_grads(P1, P2, k_t, v_t)   P = W (per-token) or the
                                                        chunk-start W (dual form)
      W1 = W1 - eta_t dW1,  W2 = W2 - eta_t dW2
      o_t = (W2 silu(W1 q_t)) * sigmoid(gate_logit_t)   (updated weights)

    Parity: pinned by tests/test_oracle_mlp.py (autograd of every inner step,
    an independent torch scan, the eta -> 0 closed form, a hand-worked d = 1
    case, dual with chunk 1 against per-token).
    """
    f = lambda a: None if a is None else np.asarray(a, dtype=dtype)
    q, k, v, eta_logit, gate_logit, W1, W2 = map(f, (q, k, v, eta_logit, gate_logit, W1_0,
                                                     W2_0))
    B, H, T, d = q.shape
    if ln != LN_NONE:
        gamma = f(gamma)[None, :, :]
        beta = f(beta)[None, :, :]
    if dual and chunk < 1:
        raise ValueError("chunk must be >= 1 in dual mode")
    W1 = W1.copy()
    W2 = W2.copy()
    out = np.zeros((B, H, T, d), dtype=dtype)
    eta_all = sigmoid(eta_logit) / dtype(d)
    gate_all = sigmoid(gate_logit)
    mv = lambda M, x: np.matmul(M, x[..., None])[..., 0]
    P1, P2 = W1, W2
    for t in range(T):
        if dual and t % chunk == 0:
            P1, P2 = W1.copy(), W2.copy()
        if not dual:
            P1, P2 = W1, W2
        dW1, dW2 = mlp_inner_grads(P1, P2, k[:, :, t, :], v[:, :, t, :], gamma, beta, ln, eps)
        eta = eta_all[:, :, t][..., None, None]
        W1 = W1 - eta * dW1
        W2 = W2 - eta * dW2
        out[:, :, t, :] = mv(W2, silu(mv(W1, q[:, :, t, :]))) * gate_all[:, :, t, :]
    return out, W1, W2


def input_projections(x, w_proj, b_proj=None):
    """The layer's input projections, the step before the scan.

    "Edifice.Recurrent.TTT", "Equations (TTT-Linear)" (the projection lines:
    q_t = W_q x_t, k_t = W_k x_t, v_t = W_v x_t, and the learning-rate gate
    from W_eta x_t) and "Architecture" (the TTT layer projects its input to
    Q, K, V, eta and gate).  One matrix product per head; the gate and the
    eta logit come out before any sigmoid (the scan applies it).

    x: [B, T, hidden].  w_proj: [H, 4d+1, hidden], the rows of one head
    stacked as W_q (d rows), W_k (d), W_v (d), W_gate (d), W_eta (1) (a layout
    choice; the pages give no order).  b_proj: [H, 4d+1] or None; the pages
    write the projections without a bias, so None is their reading and a
    bias is an option.  Returns q, k, v, eta_logit, gate_logit in the scan's
    layouts ([B, H, T, d], eta_logit [B, H, T]), float64.

    Parity: pinned by tests/test_oracle_projection.py (a brute-force loop on
    tiny inputs, one-hot weight rows that pick out coordinates of x, the
    bias alone, linearity).
    """
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w_proj, dtype=np.float64)
    H, R, hidden = w.shape
    d = (R - 1) // 4
    if R != 4 * d + 1 or x.shape[-1] != hidden:
        raise ValueError("w_proj must be [H, 4d+1, hidden] with x [B, T, hidden]")
    y = np.einsum("btk,hrk->bhtr", x, w)
    if b_proj is not None:
        y = y + np.asarray(b_proj, dtype=np.float64)[None, :, None, :]
    q, k, v, gate = (np.ascontiguousarray(y[..., i * d:(i + 1) * d]) for i in range(4))
    eta = np.ascontiguousarray(y[..., 4 * d])
    return q, k, v, eta, gate


def rel_max_err(got, ref) -> float:
    """Relative max error of one output tensor: max|got - ref| / max|ref|
    (max|got - ref| when ref is all zero).  The two tensors must have the same
    shape.  Pinned by tests/test_oracle_checker.py (hand-worked values, the
    zero and empty cases, non-finite results)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if got.shape != ref.shape:
        raise ValueError(f"shape mismatch: {got.shape} vs {ref.shape}")
    den = np.max(np.abs(ref)) if ref.size else 0.0
    num = np.max(np.abs(got - ref)) if ref.size else 0.0
    if den == 0.0:
        return float(num)
    return float(num / den)
