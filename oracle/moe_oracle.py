"""CPU oracle of the routed Mixture-of-Experts expert layer.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run anything in this
directory.  The product path (the HIP library and its Python binding) never
calls it, shares no code with it and must fail loudly without its own native
library.

What it computes is the plain, dense definition of a dropless top-k routed
MoE layer, one expert at a time, in float64 numpy with explicit bit-level
bf16 / E4M3 / E8M0 conversions.  It does no tiling, fusion or scheduling.

Sources (titles of the web pages the method comes from):

* "LigerCute - native CUTLASS + NVSHMEM kernels" (Liger-Kernel
  liger_cute_kernels README), sections "Overview" (symmetric buffers sized
  from the total routed-token capacity: nothing is dropped), "Forward pass"
  (routed tokens are sorted, the expert MLP runs, a final local combine
  applies the router weights) and "Backward pass" (activation recomputation,
  input and expert-weight gradients, routed dX reduced back to tokens).
* "LightMoE" README (lightmoe 0.1.0 metadata), sections "Standalone GEMM /
  Grouped GEMM" (contiguous expert-major rows, int32 ``m_indptr`` of length
  E+1, experts with zero rows are valid), "MoE inference" (stage order:
  dispatch, input quantisation, gate/up projection, gated activation,
  requantisation, down projection, routing-weight application, deterministic
  combine; ``top_k_ids`` int32 with distinct experts per token,
  ``top_k_weights`` fp32) and "MoE training" (dispatch returns gather
  indices, ``m_indptr``, routing weights and inverse slots; deterministic
  dispatch, combine, input-, weight- and router-gradient kernels).
* "cutedsl-megamoe" skill page (FlashInfer), section on the reference
  helpers: MXFP8 data is quantised per block of 32 with E8M0 scales.
* The OCP Microscaling Formats (MX) v1.0 specification, section 6.3
  (conversion of a block of 32 values: shared exponent = floor(log2(amax))
  minus the element format's largest exponent, elements quantised with
  saturation) and section 5.3 / 5.4 (E8M0 scale, FP8 E4M3 element with bias 7,
  no infinities, a single NaN mantissa pattern, largest normal 448).

Readings where the pages leave a step open (each is also listed with the
design notes of the repository):

* Top-k is taken on the fp32 logits (softmax is monotone), descending, ties to
  the lowest expert index; weights are the softmax restricted to the k chosen
  logits, which equals softmax over all E renormalised over the k.
* SwiGLU: h = silu(G) * U with silu(x) = x * sigmoid(x); W_gate feeds silu.
  The other gated activations (bounded SwiGLU, SwiGLU-OAI, GeGLU, ReGLU) are
  read from their public definitions (see ``activation``).
* Rounding points: h, the expert outputs O and the layer output Y are rounded
  to bf16 (round-to-nearest-even); accumulation is exact (float64 here).
* Combine adds the k weighted expert rows of a token in slot order
  (descending logit), in high precision, then rounds once.
* Backward: bf16 roundings are straight-through (identity) in the
  derivative.  The only rounded intermediate is h (recomputed exactly as in
  the forward); every other intermediate -- the gradient of the expert output
  rows dO = w * dY, P = dY W_down^T, and the gradients dg, du of the gate and up
  pre-activations -- is exact; dX and dW_* are rounded to bf16 once, after
  exact accumulation; the router-weight gradient is <h_r, dY_t W_down^T> (not
  rounded).
* Accumulation is exact up to float64 rounding (the definition, computed as
  closely as float64 allows), where an fp32 implementation accumulates in fp32;
  the difference is far inside the comparison tolerance.
"""
from __future__ import annotations

import numpy as np

# ----------------------------------------------------------------------------
# bf16 (1 sign, 8 exponent, 7 mantissa bits)
# ----------------------------------------------------------------------------

BF16_MAX = float.fromhex("0x1.fep127")


def bf16_decode(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64 (exact widening)."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return u.view(np.float32).astype(np.float64)


def bf16_round(x) -> np.ndarray:
    """Round float64 values to the nearest bf16 value (ties to even), as float64.

    bf16 keeps 8 significant bits: a normal value m*2**e (0.5 <= |m| < 1) is
    rounded to a multiple of 2**(e-8); below 2**-126 the spacing is fixed at
    2**-133 (subnormals).  Values past the largest finite bf16 plus half an
    ulp become infinite.
    """
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    q = np.maximum(e - 8, -133)
    y = np.ldexp(np.rint(np.ldexp(x, -q)), q)
    y = np.where(np.abs(y) > BF16_MAX, np.copysign(np.inf, x), y)
    return np.where(np.isnan(x), np.nan, y)


def bf16_encode(x) -> np.ndarray:
    """float64 -> bf16 bit patterns (round to nearest even)."""
    y = bf16_round(x).astype(np.float32)          # exact: y is a bf16 value
    return (y.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


# ----------------------------------------------------------------------------
# FP8 E4M3 ("FN": bias 7, no infinities, NaN = S.1111.111) and E8M0 scales
# OCP MX v1.0, sections 5.3-5.4
# ----------------------------------------------------------------------------

E4M3_MAX = 448.0
E4M3_EMAX = 8          # exponent of the largest normal (448 = 1.75 * 2**8)


def e4m3_decode(codes) -> np.ndarray:
    """E4M3FN byte codes -> float64 (NaN for 0x7F / 0xFF)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    ex = (c >> 3) & 0xF
    man = c & 0x7
    val = np.where(ex == 0, np.ldexp(man.astype(np.float64), -9),
                   np.ldexp(1.0 + man / 8.0, ex - 7))
    val = np.where((ex == 15) & (man == 7), np.nan, val)
    return sign * val


def e4m3_round(x) -> np.ndarray:
    """Round float64 to the nearest E4M3FN value, ties to even, saturating at +-448."""
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    q = np.maximum(e - 4, -9)                   # 4 significant bits; subnormal spacing 2**-9
    y = np.ldexp(np.rint(np.ldexp(x, -q)), q)
    return np.clip(y, -E4M3_MAX, E4M3_MAX)


def e4m3_encode(x) -> np.ndarray:
    """float64 (finite) -> E4M3FN byte codes, saturating round to nearest even."""
    y = e4m3_round(x)
    a = np.abs(y)
    sign = np.where(np.signbit(y), 0x80, 0)
    _, e = np.frexp(np.where(a > 0, a, 1.0))
    unb = e - 1                                      # floor(log2 a) for a > 0
    normal = a >= 2.0 ** -6
    ex_field = np.where(normal, unb + 7, 0)
    man = np.where(normal, np.rint(np.ldexp(a, -unb) * 8.0 - 8.0), np.rint(np.ldexp(a, 9)))
    code = sign | (ex_field.astype(np.int64) << 3) | man.astype(np.int64)
    return np.where(a == 0, sign, code).astype(np.uint8)


def e8m0_decode(s) -> np.ndarray:
    """E8M0 scale bytes -> float64 powers of two (255 is NaN)."""
    s = np.asarray(s, dtype=np.uint8).astype(np.int64)
    return np.where(s == 255, np.nan, np.ldexp(1.0, s - 127))


def mx_quantize(v, block: int = 32):
    """MXFP8 (E4M3 elements, E8M0 scale) quantisation along the last axis.

    OCP MX v1.0 section 6.3: for each block of 32 consecutive values, the
    shared exponent is floor(log2(max |v|)) - 8 (8 = largest E4M3 exponent),
    clamped to the E8M0 range [-127, 127]; each element is v / 2**shared
    rounded to E4M3 with saturation.  A block whose values are all zero gets
    scale byte 0 and zero elements.
    Returns (codes uint8 [..., K], scale bytes uint8 [..., K/32]).
    """
    v = np.asarray(v, dtype=np.float64)
    K = v.shape[-1]
    if K % block:
        raise ValueError("last axis must be a multiple of the block size")
    vb = v.reshape(v.shape[:-1] + (K // block, block))
    amax = np.max(np.abs(vb), axis=-1)
    _, e = np.frexp(np.where(amax > 0, amax, 1.0))
    shared = np.clip((e - 1) - E4M3_EMAX, -127, 127)
    scale_bytes = np.where(amax > 0, shared + 127, 0).astype(np.uint8)
    codes = e4m3_encode(np.ldexp(vb, -shared[..., None]))
    codes = np.where((amax > 0)[..., None], codes, 0).astype(np.uint8)
    return codes.reshape(v.shape), scale_bytes


def mx_dequantize(codes, scales, block: int = 32) -> np.ndarray:
    codes = np.asarray(codes)
    K = codes.shape[-1]
    vals = e4m3_decode(codes).reshape(codes.shape[:-1] + (K // block, block))
    return (vals * e8m0_decode(scales)[..., None]).reshape(codes.shape)


def mx_fake_quant(v) -> np.ndarray:
    """The value an MXFP8 tensor represents after quantising ``v``."""
    return mx_dequantize(*mx_quantize(v))


# ----------------------------------------------------------------------------
# Routing: softmax -> top-k -> renormalise
# ----------------------------------------------------------------------------


def route(logits, k: int):
    """Top-k routing of fp32 logits [T, E].

    Experts are ranked by logit, descending, ties to the lowest expert index
    (comparison of the fp32 logits themselves; -0.0 equals +0.0).  The k
    weights are the softmax over all E logits renormalised over the k chosen
    ones, i.e. exp(l_j - l_max) / sum over the chosen of exp(l - l_max).
    Returns (topk_idx int32 [T, k], topk_w float64 [T, k]).
    """
    lg = np.asarray(logits, dtype=np.float32)
    T, E = lg.shape
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    key = lg.astype(np.float64) + 0.0               # -0.0 -> +0.0
    order = np.argsort(-key, axis=1, kind="stable")  # stable: equal logits keep index order
    idx = order[:, :k].astype(np.int32)
    sel = np.take_along_axis(key, order[:, :k], axis=1)
    ex = np.exp(sel - sel[:, :1])
    w = ex / ex.sum(axis=1, keepdims=True)
    return idx, w


def route_backward(logits, k: int, d_topk_w):
    """Gradient with respect to the router logits [T, E] of a loss whose gradient
    with respect to the top-k weights of ``route(logits, k)`` is d_topk_w [T, k]
    (LightMoE "MoE training": router gradients; the routing weights are made
    differentiable with respect to the router output).

    The chosen set is piecewise constant in the logits (its derivative is zero
    almost everywhere), and on it the weights are the softmax of the chosen
    logits, whose Jacobian is diag(w) - w w^T.  So for the chosen expert
    e = topk_idx[t, j]:  d_logits[t, e] = w_j (d_j - sum_i w_i d_i);  every other
    logit gets 0.  float64.
    """
    idx, w = route(logits, k)
    dw = np.asarray(d_topk_w, dtype=np.float64)
    g = w * (dw - (w * dw).sum(axis=1, keepdims=True))
    out = np.zeros(np.shape(logits), dtype=np.float64)
    np.put_along_axis(out, idx.astype(np.int64), g, axis=1)
    return out


# ----------------------------------------------------------------------------
# Dispatch: expert-major order of the T*k assignments
# ----------------------------------------------------------------------------


def dispatch(topk_idx, E: int):
    """Expert-major dispatch of the T*k assignments.

    Assignment (t, j) has flat slot s = t*k + j.  Rows are ordered by expert,
    and inside an expert by slot (so by token).  Returns int32 arrays
    expert_offsets [E+1] (exclusive prefix sum of per-expert counts),
    row_token [T*k], row_slot [T*k] and slot_row [T*k] (inverse of row_slot).
    """
    sel = np.asarray(topk_idx, dtype=np.int64)
    T, k = sel.shape
    flat = sel.reshape(-1)
    counts = np.bincount(flat, minlength=E)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    row_slot = np.argsort(flat, kind="stable").astype(np.int32)
    row_token = (row_slot // k).astype(np.int32)
    slot_row = np.empty(T * k, dtype=np.int32)
    slot_row[row_slot] = np.arange(T * k, dtype=np.int32)
    return offsets, row_token, row_slot, slot_row


# ----------------------------------------------------------------------------
# Expert MLP (gate/up projection, SwiGLU, down projection) and combine
# ----------------------------------------------------------------------------


def silu(x):
    x = np.asarray(x, dtype=np.float64)
    return x / (1.0 + np.exp(-x))


def _as_f64(w) -> np.ndarray:
    """Weights may be given as bf16 bits (uint16) or as real values."""
    w = np.asarray(w)
    return bf16_decode(w) if w.dtype == np.uint16 else w.astype(np.float64)


def _expert_getter(W):
    """W: array [E, K, N] (bits or values) or a callable e -> [K, N]; None (the gate of an
    ungated expert) gives None for every expert."""
    if W is None:
        return lambda e: None
    if callable(W):
        return lambda e: _as_f64(W(e))
    return lambda e: _as_f64(W[e])


# ----------------------------------------------------------------------------
# Gated activations h = f(G, U) (LightMoE "Highlights": SwiGLU-OAI, bounded
# SwiGLU, GeGLU and ReGLU epilogues; "MoE inference": an activation clamp of 10
# for one model family).  The pages name the variants but print no formulas;
# these are the public definitions of the model families that use them:
#   swiglu        silu(G) U
#   swiglu_clamp  silu(min(G, c)) clamp(U, -c, c)                 (bounded SwiGLU)
#   swiglu_oai    g sigmoid(1.702 g) (u + 1), g = min(G, c), u = clamp(U, -c, c)
#   geglu         gelu(G) U, gelu(x) = x Phi(x) with the normal CDF Phi (erf form)
#   reglu         max(G, 0) U
# and one ungated activation (LightMoE "MoE inference": its experts load only an up and a
# down weight), whose h depends on U alone:
#   relu2         max(U, 0)^2
# ----------------------------------------------------------------------------
ACTIVATIONS = ("swiglu", "swiglu_clamp", "swiglu_oai", "geglu", "reglu", "relu2")
UNGATED = ("relu2",)


def is_gated(act: str) -> bool:
    """Whether the expert has a gate projection (every activation but ReLU^2)."""
    return act not in UNGATED
OAI_ALPHA = 1.702


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def _clamps(G, U, act, limit):
    if act in ("swiglu_clamp", "swiglu_oai"):
        if not (limit and limit > 0):
            raise ValueError(f"{act} needs a positive limit")
        return np.minimum(G, limit), np.clip(U, -limit, limit)
    return G, U


def activation(G, U, act: str = "swiglu", limit=None):
    """h = f(G, U) elementwise, float64 (G is ignored, and may be None, for ReLU^2)."""
    U = np.asarray(U, dtype=np.float64)
    if act == "relu2":
        return np.maximum(U, 0.0) ** 2
    G = np.asarray(G, dtype=np.float64)
    g, u = _clamps(G, U, act, limit)
    if act in ("swiglu", "swiglu_clamp"):
        return silu(g) * u
    if act == "swiglu_oai":
        return g * _sigmoid(OAI_ALPHA * g) * (u + 1.0)
    if act == "geglu":
        from scipy.special import ndtr
        return G * ndtr(G) * U
    if act == "reglu":
        return np.maximum(G, 0.0) * U
    raise ValueError(act)


def activation_grads(G, U, act: str = "swiglu", limit=None):
    """(df/dG, df/dU) elementwise, float64 (a clamp passes the gradient where its
    argument lies inside the bounds, the bounds included).  ReLU^2 has no gate: its
    df/dG is None."""
    U = np.asarray(U, dtype=np.float64)
    if act == "relu2":
        return None, 2.0 * np.maximum(U, 0.0)
    G = np.asarray(G, dtype=np.float64)
    g, u = _clamps(G, U, act, limit)
    if act in ("swiglu_clamp", "swiglu_oai"):
        pg = (G <= limit).astype(np.float64)
        pu = ((U >= -limit) & (U <= limit)).astype(np.float64)
    else:
        pg = pu = 1.0
    if act in ("swiglu", "swiglu_clamp"):
        return u * dsilu(g) * pg, silu(g) * pu
    if act == "swiglu_oai":
        s = _sigmoid(OAI_ALPHA * g)
        return (s + OAI_ALPHA * g * s * (1.0 - s)) * (u + 1.0) * pg, g * s * pu
    if act == "geglu":
        from scipy.special import ndtr
        phi = np.exp(-0.5 * G * G) / np.sqrt(2.0 * np.pi)
        return (ndtr(G) + G * phi) * U, G * ndtr(G)
    if act == "reglu":
        return (G > 0).astype(np.float64) * U, np.maximum(G, 0.0)
    raise ValueError(act)


def expert_forward_rows(x_rows, wg, wu, wd, mxfp8: bool = False, exact: bool = False,
                        act: str = "swiglu", limit=None):
    """One expert's MLP on rows x_rows [n, H] (float64 values).

    G = x Wg, U = x Wu, h = bf16(f(G, U)), O = bf16(h Wd), f = ``activation(.., act, limit)``
    (SwiGLU by default; ReLU^2 has no gate: wg is not used and G is None).  With
    ``mxfp8`` the GEMM operands x, W and h are the values their MXFP8 (32-long
    blocks along the contraction axis) representation holds.  ``exact``
    skips every rounding (used to check derivatives).
    Returns (G, U, h, O) as float64.
    """
    gated = is_gated(act)
    if mxfp8:
        x_rows = mx_fake_quant(x_rows)
        wg = mx_fake_quant(wg.T).T if gated else None
        wu = mx_fake_quant(wu.T).T
        wd = mx_fake_quant(wd.T).T
    G = x_rows @ wg if gated else None
    U = x_rows @ wu
    h = activation(G, U, act, limit)
    if not exact:
        h = bf16_round(h)
    hq = mx_fake_quant(h) if mxfp8 else h
    O = hq @ wd
    if not exact:
        O = bf16_round(O)
    return G, U, h, O


def expert_mlp(X, row_token, offsets, W_gate, W_up, W_down, mxfp8: bool = False,
               experts=None, exact: bool = False, act: str = "swiglu", limit=None):
    """Expert-major expert MLP over all routed rows.

    X: [T, H] (bf16 bits or values); row_token / offsets from ``dispatch``;
    W_gate, W_up: [E, H, I]; W_down: [E, I, H] (or callables e -> matrix; W_gate None for
    ReLU^2).  Returns (h [A, I], O [A, H]) as float64 (bf16 values).  Rows of experts
    not in ``experts`` (when given) are left NaN.
    """
    Xv = _as_f64(X)
    offsets = np.asarray(offsets, dtype=np.int64)
    E = offsets.shape[0] - 1
    A = int(offsets[-1])
    gg, gu, gd = _expert_getter(W_gate), _expert_getter(W_up), _expert_getter(W_down)
    I = gu(0).shape[1] if E else 0
    H = Xv.shape[1]
    h = np.full((A, I), np.nan)
    O = np.full((A, H), np.nan)
    todo = range(E) if experts is None else experts
    for e in todo:
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        rows = Xv[np.asarray(row_token[lo:hi], dtype=np.int64)]
        _, _, he, Oe = expert_forward_rows(rows, gg(e), gu(e), gd(e), mxfp8=mxfp8, exact=exact, act=act,
                                           limit=limit)
        h[lo:hi] = he
        O[lo:hi] = Oe
    return h, O


def grouped_gemm(A, B, m_indptr, mxfp8: bool = False, exact: bool = False):
    """LightMoE "Grouped GEMM": contiguous expert-major rows A [M, K], weights B [E, N, K]
    (bits or values, or a callable e -> [N, K]) and ``m_indptr`` [E + 1] (int32 offsets,
    zero-row experts valid).  C[r] = bf16(A[r] . B[e]^T) for m_indptr[e] <= r < m_indptr[e+1],
    with one rounding of the exact sum.  With ``mxfp8`` both operands are the values their
    MXFP8 representation (blocks of 32 along K) holds.  Rows outside every expert stay 0.
    Returns C [M, N] as float64."""
    Av = _as_f64(A)
    gb = _expert_getter(B)
    off = np.asarray(m_indptr, dtype=np.int64)
    E = off.shape[0] - 1
    M = Av.shape[0]
    N = gb(0).shape[0] if E else 0
    C = np.zeros((M, N))
    for e in range(E):
        lo, hi = int(off[e]), int(off[e + 1])
        if hi == lo:
            continue
        a, b = Av[lo:hi], gb(e)
        if mxfp8:
            a, b = mx_fake_quant(a), mx_fake_quant(b)
        C[lo:hi] = a @ b.T
    return C if exact else bf16_round(C)


def combine(O, slot_row, topk_w, exact: bool = False):
    """Y[t] = bf16( sum over j ascending of w[t, j] * O[slot_row[t*k + j]] )."""
    w = np.asarray(topk_w, dtype=np.float64)
    T, k = w.shape
    rows = np.asarray(slot_row, dtype=np.int64).reshape(T, k)
    acc = np.zeros((T, O.shape[1]))
    for j in range(k):
        acc = acc + w[:, j:j + 1] * O[rows[:, j]]
    return acc if exact else bf16_round(acc)


def layer_forward_tokens(X, topk_idx, topk_w, W_gate, W_up, W_down, tokens,
                         mxfp8: bool = False, exact: bool = False, act: str = "swiglu", limit=None):
    """The layer output Y for the listed tokens only, straight from the
    per-token definition (no dispatch): Y[t] = bf16(sum_j w[t,j] * MLP_e(x_t))."""
    Xv = _as_f64(X)
    gg, gu, gd = _expert_getter(W_gate), _expert_getter(W_up), _expert_getter(W_down)
    idx = np.asarray(topk_idx)
    w = np.asarray(topk_w, dtype=np.float64)
    tokens = np.asarray(tokens, dtype=np.int64)
    out = np.zeros((len(tokens), Xv.shape[1]))
    by_expert = {}
    for n, t in enumerate(tokens):
        for j in range(idx.shape[1]):
            by_expert.setdefault(int(idx[t, j]), []).append((n, int(t), j))
    contrib = {}
    for e, items in by_expert.items():
        rows = Xv[[t for _, t, _ in items]]
        _, _, _, Oe = expert_forward_rows(rows, gg(e), gu(e), gd(e), mxfp8=mxfp8, exact=exact, act=act,
                                          limit=limit)
        for (n, t, j), o in zip(items, Oe):
            contrib[(n, j)] = w[t, j] * o
    for n in range(len(tokens)):
        acc = np.zeros(Xv.shape[1])
        for j in range(idx.shape[1]):
            acc = acc + contrib[(n, j)]
        out[n] = acc
    return out if exact else bf16_round(out)


# ----------------------------------------------------------------------------
# Backward
# ----------------------------------------------------------------------------


def dsilu(x):
    """d/dx of x*sigmoid(x) = sigmoid(x) * (1 + x * (1 - sigmoid(x)))."""
    x = np.asarray(x, dtype=np.float64)
    s = 1.0 / (1.0 + np.exp(-x))
    return s * (1.0 + x * (1.0 - s))


def expert_backward_rows(x_rows, dy_rows, w_rows, wg, wu, wd, exact: bool = False, act: str = "swiglu",
                         limit=None):
    """Backward of one expert for its rows.

    x_rows, dy_rows: [n, H] token inputs and output gradients of the rows;
    w_rows: [n] routing weights.  G, U, h are recomputed as in the forward.
    P = dY W_down^T; dwt = <h, P>; dh = w P; dg = dh * df/dG, du = dh * df/dU
    (SwiGLU: du = dh * silu(G), dg = dh * U * silu'(G)); dO = w dY (exact); dXr = dg Wg^T + du Wu^T;
    dWg = x^T dg, dWu = x^T du, dWd = h^T dO (not yet rounded).  ReLU^2 has no gate:
    du = dh * 2 max(U, 0), dXr = du Wu^T, and dg, dWg are None.
    Returns dict of float64 arrays.
    """
    gated = is_gated(act)
    G = x_rows @ wg if gated else None
    U = x_rows @ wu
    h = activation(G, U, act, limit)
    if not exact:
        h = bf16_round(h)
    P = dy_rows @ wd.T
    dwt = np.sum(h * P, axis=1)
    dh = w_rows[:, None] * P
    fg, fu = activation_grads(G, U, act, limit)
    du = dh * fu
    dg = dh * fg if gated else None
    dO = w_rows[:, None] * dy_rows
    dXr = dg @ wg.T + du @ wu.T if gated else du @ wu.T
    return {"dwt": dwt, "dXr": dXr, "dWg": x_rows.T @ dg if gated else None, "dWu": x_rows.T @ du,
            "dWd": h.T @ dO, "dg": dg, "du": du, "h": h}


def backward(X, dY, topk_idx, topk_w, W_gate, W_up, W_down, experts=None, exact: bool = False, act: str = "swiglu",
             limit=None,
             want_dx: bool = True, E: int | None = None):
    """Gradients of the layer.

    Returns dict with dX [T, H], dW_gate / dW_up [E, H, I], dW_down [E, I, H]
    (bf16 values after exact accumulation; only for ``experts`` when given, the
    rest NaN; experts with no rows get exact zeros; dW_gate None for ReLU^2) and d_topk_w [T, k]
    (float64).  dX sums a token's k row contributions in slot order and is
    only complete when every expert is processed.  ``E`` is needed when the
    weights are given as callables.
    """
    rnd = (lambda a: a) if exact else bf16_round
    Xv, dYv = _as_f64(X), _as_f64(dY)
    idx = np.asarray(topk_idx, dtype=np.int64)
    w = np.asarray(topk_w, dtype=np.float64)
    T, k = idx.shape
    H = Xv.shape[1]
    gg, gu, gd = _expert_getter(W_gate), _expert_getter(W_up), _expert_getter(W_down)
    if E is None:
        E = W_up.shape[0]
    I = gu(int(idx[0, 0])).shape[1]
    gated = is_gated(act)
    todo = range(E) if experts is None else sorted(set(experts))
    dW = {n: {} for n in ("dWg", "dWu", "dWd")}
    dxr = np.zeros((T, k, H)) if want_dx else None
    dwt = np.full((T, k), np.nan)
    for e in todo:
        tt, jj = np.nonzero(idx == e)            # (t, j) in slot order
        if len(tt) == 0:
            dW["dWg"][e] = np.zeros((H, I)) if gated else None
            dW["dWu"][e] = np.zeros((H, I))
            dW["dWd"][e] = np.zeros((I, H))
            continue
        r = expert_backward_rows(Xv[tt], dYv[tt], w[tt, jj], gg(e), gu(e), gd(e), exact=exact, act=act, limit=limit)
        dW["dWg"][e] = rnd(r["dWg"]) if gated else None
        dW["dWu"][e] = rnd(r["dWu"])
        dW["dWd"][e] = rnd(r["dWd"])
        dwt[tt, jj] = r["dwt"]
        if want_dx:
            dxr[tt, jj] = r["dXr"]
    out = {"d_topk_w": dwt, "dW": dW}
    if want_dx:
        acc = np.zeros((T, H))
        for j in range(k):
            acc = acc + dxr[:, j]
        out["dX"] = rnd(acc)
    return out


def backward_tokens(X, dY, topk_idx, topk_w, W_gate, W_up, W_down, tokens, exact: bool = False,
                    act: str = "swiglu", limit=None):
    """dX and d_topk_w of the listed tokens only, straight from the per-row
    definition (same formulas as ``backward``).  Returns (dX [n, H], dwt [n, k])."""
    rnd = (lambda a: a) if exact else bf16_round
    Xv, dYv = _as_f64(X), _as_f64(dY)
    gg, gu, gd = _expert_getter(W_gate), _expert_getter(W_up), _expert_getter(W_down)
    idx = np.asarray(topk_idx, dtype=np.int64)
    w = np.asarray(topk_w, dtype=np.float64)
    tokens = np.asarray(tokens, dtype=np.int64)
    k = idx.shape[1]
    dX = np.zeros((len(tokens), Xv.shape[1]))
    dwt = np.zeros((len(tokens), k))
    for n, t in enumerate(tokens):
        acc = np.zeros(Xv.shape[1])
        for j in range(k):
            e = int(idx[t, j])
            r = expert_backward_rows(Xv[t:t + 1], dYv[t:t + 1], w[t, j:j + 1], gg(e), gu(e), gd(e), exact=exact,
                                     act=act, limit=limit)
            acc = acc + r["dXr"][0]
            dwt[n, j] = r["dwt"][0]
        dX[n] = acc
    return rnd(dX), dwt


def mx_requant_delta(h_exact, rel_eps: float = 2.0 ** -14, abs_slack=None):
    """Rounding decisions of the MXFP8 requantisation of h that another correct
    implementation may take the other way.

    h is rounded to bf16 and then quantised to MXFP8 (both decisions on a value
    that an fp32 implementation only knows to within a few fp32 ulps).  This
    perturbs the exact h of every element by +-rel_eps * (|h| + max|h| of its
    block / 64) -- far more than fp32 accumulation error -- plus ``abs_slack``
    (per element, when given: a known bound on how far an implementation's h may
    lie from the exact one, such as ``mx_block_dot_deviation`` implies), and
    returns, per element, the largest change of its MXFP8 value, plus the
    nominal MXFP8 h.  A decision within that distance of a boundary (an element
    code or, through the block maximum, the block's E8M0 scale) can go either
    way; elsewhere the change is exactly 0.
    """
    h = np.asarray(h_exact, dtype=np.float64)
    K = h.shape[-1]
    blk = np.abs(h).reshape(h.shape[:-1] + (K // 32, 32)).max(axis=-1)
    slack = rel_eps * (np.abs(h) + np.repeat(blk, 32, axis=-1) / 64.0)
    if abs_slack is not None:
        slack = slack + np.abs(np.asarray(abs_slack, dtype=np.float64))
    base = mx_fake_quant(bf16_round(h))
    up = mx_fake_quant(bf16_round(h + slack))
    dn = mx_fake_quant(bf16_round(h - slack))
    return base, np.maximum(np.abs(up - base), np.abs(dn - base))


def bf16_round_delta(x_exact, rel_eps: float = 2.0 ** -14):
    """Rounding decisions of x to bf16 that another correct implementation may take
    the other way: x is known to an fp32 implementation only to within a few fp32
    ulps, so this perturbs it by +-rel_eps * |x| (far more than fp32 error) and
    returns, per element, the largest change of its bf16 value (0 away from a
    rounding midpoint, one bf16 step next to one)."""
    x = np.asarray(x_exact, dtype=np.float64)
    slack = rel_eps * np.abs(x)
    base = bf16_round(x)
    return np.maximum(np.abs(bf16_round(x + slack) - base), np.abs(bf16_round(x - slack) - base))


def h_ambiguity_rows(x_rows, wg, wu, act: str = "swiglu", limit=None):
    """Per element of h = bf16(f(x Wg, x Wu)) for one expert's rows: the change another
    valid bf16 rounding of h can make (``bf16_round_delta`` of the exact value)."""
    G = x_rows @ wg if is_gated(act) else None
    U = x_rows @ wu
    return bf16_round_delta(activation(G, U, act, limit))


def mx_down_ambiguity(G, U, wd, act: str = "swiglu", limit=None, dG=None, dU=None):
    """For O = MXFP8(h) W_down with h = bf16(f(G, U)): per element of O, the
    largest change another valid rounding of the requantised h can cause
    (|delta| @ |W_down as MXFP8|, delta from ``mx_requant_delta``).  dG, dU (per
    element of G, U, when given) bound how far an implementation's G and U may lie
    from the exact ones; h then moves by up to |df/dG| |dG| + |df/dU| |dU| (to first
    order, taken 1.25 times), which widens the range of valid decisions."""
    abs_slack = None
    if dG is not None or dU is not None:
        gG, gU = activation_grads(G, U, act, limit)
        abs_slack = np.zeros(np.shape(U))
        if dU is not None:
            abs_slack = abs_slack + np.abs(gU) * np.abs(dU)
        if dG is not None and gG is not None:
            abs_slack = abs_slack + np.abs(gG) * np.abs(dG)
        abs_slack = 1.25 * abs_slack
    _, delta = mx_requant_delta(activation(G, U, act, limit), abs_slack=abs_slack)
    return delta @ np.abs(mx_fake_quant(np.asarray(wd, dtype=np.float64).T).T)


def e4m3_exponent(codes) -> np.ndarray:
    """Exponent field of E4M3FN codes, unbiased: E - 7 for normal codes and -6 for
    subnormal ones and zero (the E = 0 codes, whose significand is m / 8)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    ex = (c >> 3) & 0xF
    return np.where(ex == 0, -6, ex - 7)


# The scaled FP8 matrix instruction of the MI355X (gfx950, E4M3 operands with one E8M0 scale
# per 32 contraction elements) does not add its products exactly.  In every group of 8
# consecutive contraction elements, each product is truncated toward zero to a multiple of
# 2**(E - 13), where E is the largest sum of the two operands' exponent fields
# (``e4m3_exponent``) over the group's products; the truncated products are then added exactly,
# scaled by the block's two scales and accumulated in fp32.  This is a property of the
# hardware, measured on the device: single instructions with crafted operands give the rule's
# value for every case, and on Gaussian E4M3 codes (K = 4096, sums near 2e5) the rule
# reproduces the instruction to fp32 rounding (rms 0.001) where the exact sum is off by rms 4.
# tests/test_gpu_grouped_gemm.py::test_mxfp8_block_sum_rule checks it through the library's
# own MXFP8 grouped GEMM.  It is not a step of the method.
MX_BLOCK_SUM_BITS = 13
MX_BLOCK_SUM_GROUP = 8


def mx_block_dot(x_rows, w) -> np.ndarray:
    """x_rows @ w with both operands MXFP8-quantised along the contraction axis, each group
    of 8 products summed by the rule above (float64 for everything else)."""
    return _mx_block_dot(x_rows, w, deviation=False)


def mx_block_dot_deviation(x_rows, w) -> np.ndarray:
    """Per element of x_rows @ w (MXFP8 operands as in ``mx_block_dot``): the signed
    difference between the block-sum rule's result and the exact product of the
    quantised operands (the error the hardware's summation itself makes)."""
    return _mx_block_dot(x_rows, w, deviation=True)


def _mx_block_dot(x_rows, w, deviation: bool) -> np.ndarray:
    x = np.asarray(x_rows, dtype=np.float64)
    wt = np.asarray(w, dtype=np.float64).T
    n, K = x.shape
    N = wt.shape[0]
    nb = K // 32
    cx, sx = mx_quantize(x)
    cw, sw = mx_quantize(wt)
    vx, vw = e4m3_decode(cx), e4m3_decode(cw)
    ex, ew = e4m3_exponent(cx), e4m3_exponent(cw)
    G = MX_BLOCK_SUM_GROUP
    out = np.zeros((n, N))
    for i in range(n):
        p = (vx[i][None, :] * vw).reshape(N, nb, 32 // G, G)
        e = (ex[i][None, :] + ew).reshape(N, nb, 32 // G, G).max(axis=3)
        grid = np.ldexp(1.0, e - MX_BLOCK_SUM_BITS)[..., None]
        pt = np.trunc(p / grid) * grid
        blocks = (pt - p if deviation else pt).sum(axis=(2, 3))
        scale = np.ldexp(1.0, (sx[i].astype(np.int64) - 127)[None, :] + (sw.astype(np.int64) - 127))
        out[i] = (blocks * scale).sum(axis=1)
    return out
