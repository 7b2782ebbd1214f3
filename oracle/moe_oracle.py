"""Oracle: a plain, slow CPU reference of the MoE layer forward, in fp64.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import or call this module.  It shares no code with the
HIP path: it imports nothing from the GPU package, and the GPU package imports
nothing from here.  Inputs come in storage format from the seeded generator
(bf16 as uint16 bit patterns, fp8 as uint8 e4m3 codes plus fp32 block scales)
and are widened to fp64 here.

Citation keys used below:

[DD]  "Xiaohongshu dots3 note Open Source Deep Dive: 280B MoE Multimodal Model"
      (happyrock.cloud, English): §3.1 Expert Routing Mechanism (the
      Dots3MoELayer code), §3.3 layer figure ("Gate (Linear 5120→256)",
      "Weighted sum", "Shared Expert (always) … add"), §8.2 Ascend adaptation
      figure (FUSED_MC2: dispatch → gmm1 → swiglu → gmm2 → combine).
[AA]  "dots3-note 架构深度解析：16B 激活参数的 280B MoE 如何实现高效推理"
      (mlqm.cn): «核心架构参数一览» table, «稀疏激活Top-8 路由» section (sigmoid
      scoring, noaux_tc, norm_topk_prob, moe_intermediate_size 1536, BF16/FP8).
[D1]  "Transformers 中的 dots.llm1（Dots1）模型" (blog.gitcode.com):
      «MoE 路由与专家相关字段» table (norm_topk_prob, routed_scaling_factor) and
      «并行策略字段» (gate_up_proj packed, down_proj, grouped_gemm; silu act).

Readings where the pages are silent or disagree (each is also listed in the
design notes of the repository):

* Scores are sigmoid of the router logits [AA «稀疏激活»]; the softmax in the
  [DD §3.1] snippet is overruled by the config-level statement.
* noaux_tc: a per-expert bias is added to the sigmoid score to choose the
  experts; the weights use the unbiased scores.
* Group-limited routing [D1 «MoE 路由与专家相关字段»: n_group experts groups,
  topk_group groups chosen by a group score, then the top-k inside them; the
  article maps the fields to DeepSeek-V3's router].  The group score is not
  defined on the pages; reading: the sum of the two largest selection keys
  (score + bias) of the group (the whole group if it has one expert), groups
  ordered by score descending, lower group index first.  n_group = 1 is the
  plain top-k.
* Decoder block around the layer [DD §3.3 figure: "Residual + RMSNorm", MoE
  FFN, "Residual + Output"; D1: RMSNorm computes the variance in fp32, then
  rsqrt, then multiplies the weight; rms_norm_eps 1e-6]:
  out = h + MoE(RMSNorm(h)), RMSNorm(h) = gamma * h / sqrt(mean(h^2) + eps),
  with the normalised activations stored in the activation type (they are the
  layer's input tensor).
* Top-k order: key descending, lower expert index first among equal keys.
* Expert FFN = SwiGLU without biases: h = SiLU(x Wg^T) * (x Wu^T), y = h Wd^T,
  gate rows first in the packed gate_up weight [D1 «并行策略字段»].
* Weights renormalised over the k chosen scores (norm_topk_prob), then scaled
  by routed_scaling_factor.
* Output = shared-expert sum + Σ_j w[t,j] · y[t,j] [DD §3.1, §3.3].
* FP8: per-token-per-128-channel activation scales amax/448 (fp32), OCP e4m3
  with round-to-nearest-even and saturation; weights carry one fp32 scale per
  128x128 block; the intermediate h is quantised the same way as x.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

FP8_BLOCK = 128
E4M3_MAX = 448.0


# --------------------------------------------------------------------------
# Storage formats
# --------------------------------------------------------------------------

def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> fp64.  A bf16 value is the top half of an fp32."""
    u32 = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u32.view(np.float32).astype(np.float64)


def _e4m3_value(code: int) -> float:
    """OCP FP8 E4M3 ("fn"): 1 sign, 4 exponent (bias 7), 3 mantissa bits.
    Exponent field 0 is subnormal; S.1111.111 is NaN; there is no infinity."""
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** (1 - 7)
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


E4M3_TABLE = np.array([_e4m3_value(c) for c in range(256)], dtype=np.float64)
# non-negative finite values, codes 0..126, strictly increasing
_E4M3_POS = E4M3_TABLE[:127].copy()


def decode_e4m3(codes: np.ndarray) -> np.ndarray:
    return E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


def encode_e4m3(v: np.ndarray) -> np.ndarray:
    """fp32 values -> e4m3 codes: nearest value, ties to the even code,
    magnitudes above 448 saturate to 448, sign kept (so -0 -> 0x80)."""
    v = np.asarray(v, dtype=np.float32)
    a = np.abs(v).astype(np.float64)
    hi = np.searchsorted(_E4M3_POS, a, side="left")          # first value >= a
    hi = np.minimum(hi, 126)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _E4M3_POS[lo]
    d_hi = _E4M3_POS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    mag = np.where(pick_hi, hi, lo)
    mag = np.where(a >= E4M3_MAX, 126, mag)
    code = mag.astype(np.uint8) | np.where(np.signbit(v), 0x80, 0).astype(np.uint8)
    return np.where(np.isnan(v), np.uint8(0x7F), code).astype(np.uint8)


def quantize_fp8_rows(v32: np.ndarray):
    """Per row, per 128 channels: scale = amax / 448 in fp32 (1 if amax = 0),
    code = e4m3(v / scale) with the division in fp32.
    Returns (codes uint8 [R, C], scales fp32 [R, C/128])."""
    v32 = np.asarray(v32, dtype=np.float32)
    R, C = v32.shape
    assert C % FP8_BLOCK == 0
    blocks = v32.reshape(R, C // FP8_BLOCK, FP8_BLOCK)
    amax = np.abs(blocks).max(axis=2)
    scale = np.where(amax == 0, np.float32(1.0),
                     amax / np.float32(E4M3_MAX)).astype(np.float32)
    q = blocks / scale[:, :, None]                      # fp32 / fp32 -> fp32
    assert q.dtype == np.float32
    return encode_e4m3(q).reshape(R, C), scale


def dequantize_fp8_rows(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    return decode_e4m3(codes) * np.repeat(scales.astype(np.float64), FP8_BLOCK, axis=1)


def dequantize_fp8_weight(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """[N, K] codes with [N/128, K/128] block scales -> fp64 [N, K]."""
    s = np.repeat(np.repeat(scales.astype(np.float64), FP8_BLOCK, 0), FP8_BLOCK, 1)
    return decode_e4m3(codes) * s


def widen(a: np.ndarray, kind: str) -> np.ndarray:
    """Storage array -> fp64 ('f32', 'bf16', or 'f64' for hand-made test
    inputs; fp8 needs its scales)."""
    if kind == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    if kind == "bf16":
        return decode_bf16(a)
    if kind == "f64":
        return np.asarray(a, dtype=np.float64)
    raise ValueError(kind)


# --------------------------------------------------------------------------
# Router: logits, sigmoid scores, biased top-k, renormalised weights
# --------------------------------------------------------------------------

def sigmoid(z: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-z))


@dataclass
class Routing:
    logits: np.ndarray     # [T, E]
    scores: np.ndarray     # [T, E]  s = sigmoid(logits)
    keys: np.ndarray       # [T, E]  c = s + bias (selection only)
    idx: np.ndarray        # [T, k]  int32, slot order = key desc, index asc
    w: np.ndarray          # [T, k]  routing weights
    gap_sel: np.ndarray    # [T]     c_(k-1) - c_(k)  (0-based sorted positions)
    gap_ord: np.ndarray    # [T]     min_j<k-1 c_(j) - c_(j+1)
    gap_grp: np.ndarray = None  # [T] group score gap at the topk_group boundary


def group_scores(c: np.ndarray, n_group: int) -> np.ndarray:
    """[T, n_group]: per group of E / n_group consecutive experts, the sum of
    its two largest selection keys (its only key if the group has one)."""
    T, E = c.shape
    G = E // n_group
    top = np.sort(c.reshape(T, n_group, G), axis=2)[:, :, ::-1]
    return top[:, :, :min(2, G)].sum(axis=2)


def route(x: np.ndarray, w_router: np.ndarray, bias: np.ndarray, k: int,
          norm_topk_prob: bool = True, routed_scaling_factor: float = 1.0,
          n_group: int = 1, topk_group: int = 1) -> Routing:
    """Gate = Linear(hidden -> E, no bias) [DD §3.1, §3.3 "Gate (Linear 5120→256)"];
    sigmoid scores and noaux_tc selection [AA «稀疏激活»]; optional group
    limit [D1 n_group / topk_group]; top-k then renormalisation over the k
    chosen scores [DD §3.1; AA norm_topk_prob]; routed_scaling_factor
    [D1 MoE fields]."""
    x = np.asarray(x, dtype=np.float64)
    w_router = np.asarray(w_router, dtype=np.float64)
    T = x.shape[0]
    E = w_router.shape[0]
    assert 1 <= k <= E
    assert n_group >= 1 and E % n_group == 0 and 1 <= topk_group <= n_group
    assert k <= topk_group * (E // n_group)
    logits = x @ w_router.T
    s = sigmoid(logits)
    c = s + np.asarray(bias, dtype=np.float64)[None, :]
    # group limit: keep the experts of the topk_group best groups
    gs = group_scores(c, n_group)
    g_order = np.argsort(-gs, axis=1, kind="stable")
    gss = np.take_along_axis(gs, g_order, axis=1)
    gap_grp = (gss[:, topk_group - 1] - gss[:, topk_group] if topk_group < n_group
               else np.full(T, np.inf))
    keep = np.zeros((T, n_group), bool)
    np.put_along_axis(keep, g_order[:, :topk_group], True, axis=1)
    allowed = np.repeat(keep, E // n_group, axis=1)
    cm = np.where(allowed, c, -np.inf)
    # stable sort of -c: descending key, equal keys keep ascending expert index
    order = np.argsort(-cm, axis=1, kind="stable")
    idx = order[:, :k].astype(np.int32)
    cs = np.take_along_axis(cm, order, axis=1)
    gap_sel = cs[:, k - 1] - cs[:, k] if k < E else np.full(T, np.inf)
    if k >= 2:
        gap_ord = np.min(cs[:, :k - 1] - cs[:, 1:k], axis=1)
    else:
        gap_ord = np.full(T, np.inf)
    w = selection_weights(s, idx, norm_topk_prob, routed_scaling_factor)
    return Routing(logits, s, c, idx, w, gap_sel, gap_ord, gap_grp)


def selection_weights(s: np.ndarray, idx: np.ndarray, norm_topk_prob: bool = True,
                      routed_scaling_factor: float = 1.0) -> np.ndarray:
    """Routing weights of a chosen set: the unbiased sigmoid scores of the k
    chosen experts, renormalised to sum to 1 (norm_topk_prob [AA «稀疏激活»;
    DD §3.1 division by the sum of the top-k weights]), times
    routed_scaling_factor [D1 MoE fields]."""
    chosen = np.take_along_axis(s, np.asarray(idx, dtype=np.int64), axis=1)
    if norm_topk_prob:
        w = chosen / chosen.sum(axis=1, keepdims=True)
    else:
        w = chosen.copy()
    return w * routed_scaling_factor


def with_selection(r: Routing, idx: np.ndarray, norm_topk_prob: bool = True,
                   routed_scaling_factor: float = 1.0) -> Routing:
    """The same router scores with another chosen set `idx` [T, k] (where a
    near-tie admits more than one correct top-k): weights recomputed by
    selection_weights; logits, scores, keys and gaps kept."""
    idx = np.asarray(idx, dtype=np.int32)
    return Routing(r.logits, r.scores, r.keys, idx,
                   selection_weights(r.scores, idx, norm_topk_prob, routed_scaling_factor),
                   r.gap_sel, r.gap_ord, r.gap_grp)


# --------------------------------------------------------------------------
# Dispatch: histogram, exclusive scan, stable permutation
# --------------------------------------------------------------------------

@dataclass
class Dispatch:
    counts: np.ndarray     # [E]     rows per expert
    offsets: np.ndarray    # [E+1]   exclusive scan of counts
    perm: np.ndarray       # [T*k]   sorted position -> flat index f = t*k + j
    inv: np.ndarray        # [T*k]   flat index -> sorted position


def dispatch(idx: np.ndarray, E: int) -> Dispatch:
    """Group the (token, slot) pairs by expert.  Within an expert the pairs keep
    ascending flat order f = t*k + j, which is the order in which the per-expert
    mask gathers tokens in the [DD §3.1] loop (x[mask] is token-ascending, and
    a token picks an expert at most once).  Written as its definition:
    pos(f) = offsets[e(f)] + #{f' < f : e(f') = e(f)}."""
    flat = np.asarray(idx, dtype=np.int64).ravel()
    counts = np.zeros(E, dtype=np.int64)
    for e in flat:
        counts[e] += 1
    offsets = np.zeros(E + 1, dtype=np.int64)
    for e in range(E):
        offsets[e + 1] = offsets[e] + counts[e]
    seen = np.zeros(E, dtype=np.int64)
    inv = np.empty(flat.size, dtype=np.int64)
    for f, e in enumerate(flat):
        inv[f] = offsets[e] + seen[e]
        seen[e] += 1
    perm = np.empty_like(inv)
    perm[inv] = np.arange(flat.size)
    return Dispatch(counts.astype(np.int32), offsets.astype(np.int32),
                    perm.astype(np.int32), inv.astype(np.int32))


# --------------------------------------------------------------------------
# Experts
# --------------------------------------------------------------------------

def swiglu_hidden(a: np.ndarray, wg: np.ndarray, wu: np.ndarray) -> np.ndarray:
    """h = SiLU(a Wg^T) * (a Wu^T), SiLU(z) = z * sigmoid(z)
    [D1 hidden_act silu, gate_up_proj packed; DD §8.2 "gmm1 → swiglu"]."""
    g = a @ wg.T
    u = a @ wu.T
    return g * sigmoid(g) * u


class Weights:
    """Per-expert fp64 views of the stored weights (decoded on demand)."""

    def __init__(self, cfg, inp: dict):
        self.cfg = cfg
        self.inp = inp

    def _dec(self, w, s):
        if self.cfg.expert == "fp8":
            return dequantize_fp8_weight(w, s)
        return widen(w, self.cfg.expert)

    def expert(self, g: int):
        """Expert g < E is routed expert g; g = E + s is shared expert s.
        Returns fp64 (Wg [I,H], Wu [I,H], Wd [H,I])."""
        cfg, inp = self.cfg, self.inp
        fp8 = cfg.expert == "fp8"
        if g < cfg.E:
            gu, dn, I = inp["w_gate_up"][g], inp["w_down"][g], cfg.I
            sgu = inp["s_gate_up"][g] if fp8 else None
            sdn = inp["s_down"][g] if fp8 else None
        else:
            s = g - cfg.E
            gu, dn, I = inp["w_sh_gate_up"][s], inp["w_sh_down"][s], cfg.Is
            sgu = inp["s_sh_gate_up"][s] if fp8 else None
            sdn = inp["s_sh_down"][s] if fp8 else None
        nb = I // FP8_BLOCK
        wg = self._dec(gu[:I], sgu[:nb] if fp8 else None)
        wu = self._dec(gu[I:], sgu[nb:] if fp8 else None)
        wd = self._dec(dn, sdn)
        return wg, wu, wd


def expert_forward(cfg, a: np.ndarray, wg, wu, wd) -> np.ndarray:
    """One SwiGLU expert on rows a (fp64, already dequantised for fp8).
    For fp8 the intermediate h is rounded to fp32 and quantised per row per
    128 channels before the down projection."""
    h = swiglu_hidden(a, wg, wu)
    if cfg.expert == "fp8":
        hq, hs = quantize_fp8_rows(h.astype(np.float32))
        h = dequantize_fp8_rows(hq, hs)
    return h @ wd.T


def layer_inputs(cfg, inp: dict, tokens=None):
    """x as the experts see it (fp64) and as the router sees it (fp64).
    fp8: experts see the per-token-per-128 quantised x; the router sees x."""
    x_st = inp["x"] if tokens is None else inp["x"][tokens]
    x_r = widen(x_st, cfg.act)
    if cfg.expert == "fp8":
        xq, xs = quantize_fp8_rows(x_r.astype(np.float32))
        x_e = dequantize_fp8_rows(xq, xs)
    else:
        x_e = x_r
    return x_r, x_e


def route_inputs(cfg, inp: dict, tokens=None) -> Routing:
    x_r, _ = layer_inputs(cfg, inp, tokens)
    return route(x_r, widen(inp["w_router"], cfg.act), inp["bias"], cfg.k,
                 cfg.norm_topk_prob, cfg.routed_scaling_factor, cfg.n_group, cfg.topk_group)


@dataclass
class LayerResult:
    out: np.ndarray        # [n, H] fp64
    routing: Routing
    y: np.ndarray          # [n, k, H] routed expert outputs per (token, slot)
    ysh: np.ndarray        # [S, n, H] shared expert outputs
    tokens: np.ndarray     # token ids covered


def layer_forward(cfg, inp: dict, tokens=None, idx=None) -> LayerResult:
    """out[t] = Σ_s shared_s(x_t) + Σ_j w[t,j] · expert_{idx[t,j]}(x_t)
    [DD §3.1 forward; §3.3 "Weighted sum" then "Shared Expert (always) … add"].
    The layer is per-token independent, so a subset of tokens gives exactly
    the rows of the full result.  idx (optional, [len(tokens), k]) replaces
    the router's choice, e.g. by another valid top-k of a near-tied token;
    its weights are then the renormalised scores of that set."""
    tokens = np.arange(cfg.T) if tokens is None else np.asarray(tokens)
    x_r, x_e = layer_inputs(cfg, inp, tokens)
    r = route(x_r, widen(inp["w_router"], cfg.act), inp["bias"], cfg.k,
              cfg.norm_topk_prob, cfg.routed_scaling_factor, cfg.n_group, cfg.topk_group)
    if idx is not None:
        r = with_selection(r, idx, cfg.norm_topk_prob, cfg.routed_scaling_factor)
    n, H, k = tokens.size, cfg.H, cfg.k
    W = Weights(cfg, inp)
    y = np.zeros((n, k, H))
    for e in np.unique(r.idx):
        rows, slots = np.nonzero(r.idx == e)
        y[rows, slots] = expert_forward(cfg, x_e[rows], *W.expert(int(e)))
    ysh = np.zeros((cfg.S, n, H))
    for s in range(cfg.S):
        ysh[s] = expert_forward(cfg, x_e, *W.expert(cfg.E + s))
    out = ysh.sum(axis=0) + np.einsum("tj,tjh->th", r.w, y)
    return LayerResult(out, r, y, ysh, tokens)


def dense_layer_forward(cfg, inp: dict) -> np.ndarray:
    """Brute force: run EVERY routed expert on EVERY token and weight it by the
    routing mask m[t,e] = w[t,j] if idx[t,j] = e, else 0.  No dispatch."""
    x_r, x_e = layer_inputs(cfg, inp)
    r = route(x_r, widen(inp["w_router"], cfg.act), inp["bias"], cfg.k,
              cfg.norm_topk_prob, cfg.routed_scaling_factor, cfg.n_group, cfg.topk_group)
    W = Weights(cfg, inp)
    m = np.zeros((cfg.T, cfg.E))
    for j in range(cfg.k):
        m[np.arange(cfg.T), r.idx[:, j]] += r.w[:, j]
    out = np.zeros((cfg.T, cfg.H))
    for e in range(cfg.E):
        out += m[:, e:e + 1] * expert_forward(cfg, x_e, *W.expert(e))
    for s in range(cfg.S):
        out += expert_forward(cfg, x_e, *W.expert(cfg.E + s))
    return out


def sorted_expert_rows(cfg, inp: dict, routing: Routing, disp: Dispatch):
    """The intermediates in expert-sorted order, for step-by-step checks:
    h_sorted [T*k, I] and y_sorted [T*k, H] (routed rows, fp64), plus the
    shared h [S, T, Is] and y [S, T, H].  Row p holds token perm[p] // k
    processed by expert e with offsets[e] <= p < offsets[e+1]."""
    _, x_e = layer_inputs(cfg, inp)
    W = Weights(cfg, inp)
    R = cfg.T * cfg.k
    h_sorted = np.zeros((R, cfg.I))
    y_sorted = np.zeros((R, cfg.H))
    for e in range(cfg.E):
        lo, hi = int(disp.offsets[e]), int(disp.offsets[e + 1])
        if hi == lo:
            continue
        a = x_e[disp.perm[lo:hi] // cfg.k]
        wg, wu, wd = W.expert(e)
        h = swiglu_hidden(a, wg, wu)
        if cfg.expert == "fp8":
            hq, hs = quantize_fp8_rows(h.astype(np.float32))
            hd = dequantize_fp8_rows(hq, hs)
        else:
            hd = h
        h_sorted[lo:hi] = h
        y_sorted[lo:hi] = hd @ wd.T
    h_sh = np.zeros((cfg.S, cfg.T, cfg.Is))
    y_sh = np.zeros((cfg.S, cfg.T, cfg.H))
    for s in range(cfg.S):
        wg, wu, wd = W.expert(cfg.E + s)
        h = swiglu_hidden(x_e, wg, wu)
        if cfg.expert == "fp8":
            hq, hs = quantize_fp8_rows(h.astype(np.float32))
            hd = dequantize_fp8_rows(hq, hs)
        else:
            hd = h
        h_sh[s] = h
        y_sh[s] = hd @ wd.T
    return h_sorted, y_sorted, h_sh, y_sh


def combine(y_sorted: np.ndarray, y_shared: np.ndarray, w: np.ndarray,
            inv: np.ndarray, k: int) -> np.ndarray:
    """out[t] = Σ_s y_shared[s, t] + Σ_j w[t, j] · y_sorted[inv[t*k + j]]
    [DD §3.1 weighted add of routed outputs plus shared; §3.3]."""
    T = w.shape[0]
    out = np.asarray(y_shared, dtype=np.float64).sum(axis=0)
    for j in range(k):
        out = out + w[:, j:j + 1] * np.asarray(y_sorted, np.float64)[inv[np.arange(T) * k + j]]
    return out


# --------------------------------------------------------------------------
# Decoder block around the layer: RMSNorm before, residual add after
# --------------------------------------------------------------------------

def rmsnorm(h: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    """gamma * h / sqrt(mean(h^2) + eps) per row [D1: variance, rsqrt, times
    the weight; DD §3.3 "Residual + RMSNorm"]."""
    h = np.asarray(h, dtype=np.float64)
    ms = np.mean(h * h, axis=-1, keepdims=True)
    return np.asarray(gamma, dtype=np.float64)[None, :] * (h / np.sqrt(ms + eps))


def encode_bf16(v: np.ndarray) -> np.ndarray:
    """fp64 -> bf16 bit patterns with round-to-nearest-even, decided on the
    fp64 value itself (no double rounding through fp32).  Finite inputs."""
    v = np.asarray(v, dtype=np.float64)
    bits = v.astype(np.float32).view(np.uint32)
    hi = (bits >> 16).astype(np.uint32)          # bf16 truncation of the fp32 value
    lo_val = (hi << 16).view(np.float32).astype(np.float64)          # |lo_val| <= |v|, or equal up to fp32 rounding
    hi_val = ((hi + 1) << 16).view(np.float32).astype(np.float64)    # next bf16 away from zero
    a, lo_a, hi_a = np.abs(v), np.abs(lo_val), np.abs(hi_val)
    mid = (lo_a + hi_a) / 2.0                    # exact in fp64
    up = (a > mid) | ((a == mid) & ((hi & 1) == 1))
    return np.where(up, hi + 1, hi).astype(np.uint16)


def block_inputs(cfg, inp: dict, gamma: np.ndarray, tokens=None):
    """(h, xn_storage): the residual input h (fp64) and the normalised layer
    input in storage format (the activation type)."""
    h_st = inp["x"] if tokens is None else inp["x"][tokens]
    h = widen(h_st, cfg.act)
    xn = rmsnorm(h, gamma, cfg.rms_norm_eps)
    if cfg.act == "bf16":
        xn_st = encode_bf16(xn)
    else:
        xn_st = xn.astype(np.float32)
    return h, xn_st


def block_forward(cfg, inp: dict, gamma: np.ndarray, tokens=None, idx=None):
    """out = h + MoE(RMSNorm(h)) [DD §3.3 figure: "Residual + RMSNorm", MoE
    FFN, "Residual + Output"].  Returns (out fp64 [n, H], LayerResult).
    idx: optional choice of experts, as for layer_forward."""
    tokens = np.arange(cfg.T) if tokens is None else np.asarray(tokens)
    h, xn_st = block_inputs(cfg, inp, gamma, tokens)
    # the layer on the normalised rows only (x replaced by the normalised subset)
    full = dict(inp)
    full["x"] = np.zeros_like(inp["x"])
    full["x"][tokens] = xn_st
    res = layer_forward(cfg, full, tokens, idx=idx)
    return h + res.out, res


def rms(a: np.ndarray) -> float:
    return float(math.sqrt(np.mean(np.square(np.asarray(a, dtype=np.float64)))))
