"""Plain float64 NumPy oracle for DeepSeek-V2 Multi-head Latent Attention (MLA).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.  Slow on purpose: no
blocking, no fusion, no reordering beyond what each definition states; library
matrix products serve as single steps.

Sources (page title, section / equation):
  * "A. Conclusion, Limitation, and Future" DeepSeek-V2 reading notes
    (irregular6612.github.io), §2.1.1 eq. 1-8 (standard MHA, per-head split,
    scaled-dot softmax attention) and §2.1.2 eq. 9-13 (low-rank joint KV
    compression, up-projections W^UK / W^UV, query compression).
  * DeepSeek-V2 MLA blog (adg.csdn.net), part 2 §2.2.1.1 (only c^KV is cached;
    W^UK / W^UV can be absorbed), §2.2.2 (RoPE as position rotation matrices
    with R_m^T R_n depending on n - m; RoPE is incompatible with the low-rank
    cache; decoupled multi-head q^R and one shared k^R; concatenation
    [q^C; q^R], [k^C; k^R]; k^R is cached already rotated; cache holds
    (d_c + d_R) elements per token, d_c = 4 d_h, d_R = d_h / 2).

Readings where the pages are silent or garbled:
  R1 softmax scale: 1/sqrt(d_h + d_R), the width of the concatenated q.k.
  R2 RoPE: rotate adjacent pairs (x[2k], x[2k+1]) by pos * base^(-2k/d_R),
     angles formed in float64.
  R3 k^R is stored after rotation at its own position; c^KV is never rotated.
  R4 cached token j sits at position j; a decode query sits at position L and
     sees all L cached keys; chunk row m of a q_len-row chunk sees keys
     j < L - (q_len - 1 - m) (its own position included).
  R5 eq. 7's printed sum index is read as a sum over keys j.
  R6 a query row with no visible key yields o = 0 and lse = -inf.
  R7 W^UK / W^UV are stored [n_h, d_h, d_c]: head i owns rows i*d_h..(i+1)*d_h
     of eq. 10/11's matrices (eq. 4-6 ordering).
  R8 the extra RMSNorm after the compressed latents (blog part 3 §3.1.1 names it and
     gives no formula) is the standard one, g * x / sqrt(mean(x^2) + eps) over
     the latent's width, with a learned gain g; it is applied to c^KV before it
     is cached and to c^Q before its up-projections.
  R9 the decoupled key comes straight from the hidden state, k^R = W^KR h, and
     the decoupled query from the compressed query, q^R = W^QR c^Q (blog
     §2.2.2); both are rotated at the token's position.  Down-projections are
     stored as written in eq. 9 / 12, [d_out, d_model]; W^UQ and W^QR as
     [n_h * d_h, d_c'] and [n_h * d_R, d_c'], head i owning rows i*d_h.. and
     i*d_R.. respectively.
  R10 a model that does not compress its queries (V2-Lite: blog, the V2-Lite
     paragraph) projects both query parts straight from the hidden state,
     q^C = W^QC h (eq. 1's W^Q, per-head rows) and q^R = W^QR h.
  R11 YaRN (blog part 3 §3.1.3: applied to the decoupled RoPE key, scale 40, the two
     ramp parameters 1 and 32, target context 160K) is read as YaRN's
     interpolation by parts on the RoPE pair frequencies: with the original
     context L0 = 4096 (the blog extends a 4K window; 40 x 4096 = 163,840 is
     the stated 160K), pair k's frequency theta_k = base^(-2k/d) completes
     r_k = L0 theta_k / (2 pi) turns over L0 positions; a ramp
     g_k = clip((r_k - alpha) / (beta - alpha), 0, 1) with alpha = 1,
     beta = 32 keeps fast pairs (g = 1) and divides slow pairs by the scale
     (g = 0): theta'_k = (1 - g_k) theta_k / s + g_k theta_k.  The same
     frequencies rotate q^R (a score depends on the key's and the query's
     rotation together).  The blog's attention-entropy factor is not printed
     (its formula is missing from the page): it multiplies every score, so it
     is part of the softmax scale the caller passes, and it is 1 here.
  R12 the quantised latent cache (blog part 3 §3.1.4: the served model's KV
     cache is quantised to about 6 bits per element on average, scheme not
     given) is read as OCP FP8 E4M3 per element (sign, 4 exponent bits with
     bias 7, 3 mantissa bits; subnormals; largest finite value 448; no
     infinities) with two float32 scales per cached token, one for the 512
     latent elements and one for the 64 rotated RoPE elements.  The values to
     quantise are the float32 row (c^KV as given, k^R rotated in float64 and
     rounded to float32).  Per part: amax = max |x|, s = amax / 448 in float32
     (s = 1 for an all-zero part), code = the E4M3 value nearest to the
     float32 quotient x / s, ties to even, clamped to +-448; the cached value
     stands for s * code.  Attention over the quantised cache is the same
     attention over those dequantised rows.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "rope_rotate", "rope_theta", "yarn_theta", "mla_attention_naive",
    "e4m3_value", "e4m3_round", "e4m3_code", "quantize_rows", "dequantize_rows",
    "kv_cache_rows_fp8", "kv_cache_rows", "absorb_query",
    "latent_attention", "split_ranges", "combine_splits", "out_projection",
    "visible_keys", "rms_norm", "kv_produce", "q_produce",
    "q_produce_direct", "o_projection",
]

F64 = np.float64


def rope_theta(d: int, base: float):
    """Pair frequencies of plain RoPE (reading R2): theta_k = base^(-2k/d)."""
    k = np.arange(d // 2, dtype=F64)
    return float(base) ** (-2.0 * k / d)


def yarn_theta(d: int, base: float, scale: float, alpha: float, beta: float, orig_ctx: int):
    """Pair frequencies after YaRN's interpolation by parts (reading R11).

    r_k = orig_ctx * theta_k / (2 pi) is the number of turns pair k makes
    over the original context; g_k = clip((r_k - alpha) / (beta - alpha), 0, 1);
    theta'_k = (1 - g_k) * theta_k / scale + g_k * theta_k.
    """
    theta = rope_theta(d, base)
    r = float(orig_ctx) * theta / (2.0 * np.pi)
    g = np.clip((r - float(alpha)) / (float(beta) - float(alpha)), 0.0, 1.0)
    return (1.0 - g) * theta / float(scale) + g * theta


def rope_rotate(x, pos, base: float, theta=None):
    """Apply the position rotation R_pos to the trailing axis of ``x``.

    blog §2.2.2: RoPE multiplies a vector by a position-dependent rotation
    matrix so that (R_m q)^T (R_n k) depends on n - m only.  Reading R2: the
    matrix is block diagonal with 2x2 rotations on adjacent pairs, pair k
    turned by angle pos * theta_k, theta_k = base^(-2k/d), d = x.shape[-1]
    (or the given pair frequencies ``theta``, e.g. YaRN's, reading R11).

    ``pos`` broadcasts against ``x.shape[:-1]``.
    """
    x = np.asarray(x, dtype=F64)
    d = x.shape[-1]
    if d % 2:
        raise ValueError("RoPE width must be even")
    if d == 0:
        return x.copy()
    theta = rope_theta(d, base) if theta is None else np.asarray(theta, dtype=F64)
    if theta.shape != (d // 2,):
        raise ValueError("theta must hold one frequency per pair")
    ang = np.asarray(pos, dtype=F64)[..., None] * theta
    c, s = np.cos(ang), np.sin(ang)
    even, odd = x[..., 0::2], x[..., 1::2]
    out = np.empty(np.broadcast_shapes(x.shape, ang.shape[:-1] + (d,)), dtype=F64)
    out[..., 0::2] = even * c - odd * s
    out[..., 1::2] = even * s + odd * c
    return out


def visible_keys(seq_len: int, q_len: int) -> np.ndarray:
    """Keys visible to each of the q_len query rows of one sequence (reading R4)."""
    return np.array([seq_len - (q_len - 1 - m) for m in range(q_len)], dtype=np.int64)


def _softmax_two_pass(s):
    """eq. 7's Softmax_j over the last axis, two passes (max, then normalised exp).

    Returns (p, lse).  An empty axis gives an empty p and lse = -inf (R6).
    """
    if s.shape[-1] == 0:
        return s.copy(), np.full(s.shape[:-1], -np.inf)
    m = s.max(axis=-1, keepdims=True)
    e = np.exp(s - m)
    z = e.sum(axis=-1, keepdims=True)
    return e / z, (m + np.log(z))[..., 0]


def mla_attention_naive(c_kv, k_r, q_nope, q_rope, w_uk, w_uv, key_pos, q_pos,
                        n_visible, scale: float, base: float, theta=None):
    """MLA attention of one sequence in the literal, non-absorbed form.

    Inputs (any float type, used as float64):
      c_kv [L, d_c]   cached latents c^KV_j (eq. 9's output; given)
      k_r  [L, d_R]   decoupled RoPE key before rotation, shared by all heads
      q_nope [M, n_h, d_h], q_rope [M, n_h, d_R]  the M query rows
      w_uk, w_uv [n_h, d_h, d_c]
      key_pos [L], q_pos [M], n_visible [M] (row m sees keys 0..n_visible[m]-1)
      theta: optional RoPE pair frequencies (default base^(-2k/d_R))
    Steps, per head i:
      k^C_{j,i} = W^UK_i c^KV_j and v^C_{j,i} = W^UV_i c^KV_j  (eq. 10, 11)
      k^R_j = R_{pos j} k_r_j, q^R_i = R_{q pos} q_rope_i       (blog §2.2.2)
      q_i = [q_nope_i; q^R_i], k_{j,i} = [k^C_{j,i}; k^R_j]      (blog §2.2.2)
      o_i = sum_j Softmax_j(scale * q_i . k_{j,i}) v^C_{j,i}     (eq. 7)
    Returns out [M, n_h, d_h] (eq. 7's o_{t,i}, before W^O), lse [M, n_h] and
    the diagnostic o_lat [M, n_h, d_c] = sum_j p_j c^KV_j.
    """
    c_kv = np.asarray(c_kv, F64)
    k_r = np.asarray(k_r, F64)
    q_nope = np.asarray(q_nope, F64)
    q_rope = np.asarray(q_rope, F64)
    w_uk = np.asarray(w_uk, F64)
    w_uv = np.asarray(w_uv, F64)
    M, n_h, d_h = q_nope.shape
    d_c = c_kv.shape[1]
    k_rot = rope_rotate(k_r, np.asarray(key_pos), base, theta)           # [L, d_R]
    q_rot = rope_rotate(q_rope, np.asarray(q_pos)[:, None], base, theta) # [M, n_h, d_R]
    out = np.zeros((M, n_h, d_h))
    o_lat = np.zeros((M, n_h, d_c))
    lse = np.full((M, n_h), -np.inf)
    n_visible = np.asarray(n_visible, dtype=np.int64)
    for i in range(n_h):
        k_c = c_kv @ w_uk[i].T          # [L, d_h]   eq. 10 for every cached token
        v_c = c_kv @ w_uv[i].T          # [L, d_h]   eq. 11
        keys = np.concatenate([k_c, k_rot], axis=1)   # [L, d_h + d_R]
        for m in range(M):
            n = int(n_visible[m])
            if n <= 0:
                continue
            q = np.concatenate([q_nope[m, i], q_rot[m, i]])
            s = (keys[:n] @ q) * scale
            p, l = _softmax_two_pass(s)
            out[m, i] = p @ v_c[:n]
            o_lat[m, i] = p @ c_kv[:n]
            lse[m, i] = l
    return out, lse, o_lat


# ---------------------------------------------------------------------------
# The absorbed steps, each with its plain definition.  Together they equal
# mla_attention_naive by associativity (blog §2.2.1.1 / §2.2.2: W^UK moves to
# the query side and W^UV to the output side).
# ---------------------------------------------------------------------------

def kv_cache_rows(c_kv, k_r, pos, base: float, theta=None):
    """The cached row of each token: [c^KV_j ; R_{pos j} k_r_j] (readings R3, R4).

    blog §2.2.2: per token the cache keeps c^KV and the already rotated k^R,
    (d_c + d_R) elements.  Returns float64 [N, d_c + d_R].
    """
    c_kv = np.asarray(c_kv, F64)
    return np.concatenate([c_kv, rope_rotate(k_r, np.asarray(pos), base, theta)], axis=1)


def absorb_query(q_nope, q_rope, w_uk, q_pos, base: float, theta=None):
    """Latent-space query of every row and head: [W^UK_i^T q_nope_i ; R_p q_rope_i].

    By eq. 10, q_nope_i . k^C_{j,i} = q_nope_i . (W^UK_i c_j) = (W^UK_i^T q_nope_i) . c_j,
    so scoring the absorbed query against the cached latent equals the
    non-absorbed score.  Returns float64 [T, n_h, d_c + d_R].
    """
    q_nope = np.asarray(q_nope, F64)
    w_uk = np.asarray(w_uk, F64)
    T, n_h, _ = q_nope.shape
    q_abs = np.empty((T, n_h, w_uk.shape[2]))
    for i in range(n_h):
        q_abs[:, i, :] = q_nope[:, i, :] @ w_uk[i]      # row-vector form of W^T q
    q_rot = rope_rotate(q_rope, np.asarray(q_pos)[:, None], base, theta)
    return np.concatenate([q_abs, q_rot], axis=2)


def latent_attention(q_lat, rows, n_visible, scale: float, d_c: int):
    """Attention of latent queries over cached rows (the absorbed eq. 7).

    q_lat [M, n_h, W] with W = d_c + d_R, rows [L, W].  Row m sees rows
    0..n_visible[m]-1.  s = scale * q_lat . row; p = Softmax_j(s);
    o_lat = sum_j p_j row_j[:d_c].  Returns (o_lat [M, n_h, d_c], lse [M, n_h]).
    """
    q_lat = np.asarray(q_lat, F64)
    rows = np.asarray(rows, F64)
    M, n_h, _ = q_lat.shape
    o_lat = np.zeros((M, n_h, d_c))
    lse = np.full((M, n_h), -np.inf)
    for m in range(M):
        n = int(n_visible[m])
        if n <= 0:
            continue
        s = (q_lat[m] @ rows[:n].T) * scale                 # [n_h, n]
        p, l = _softmax_two_pass(s)
        o_lat[m] = p @ rows[:n, :d_c]
        lse[m] = l
    return o_lat, lse


def split_ranges(n_keys: int, block_size: int, num_splits: int):
    """Key ranges of the split-KV partition of one sequence.

    The sequence's blocks are cut into num_splits contiguous runs of
    c = ceil(nblk / num_splits) blocks (the last runs may be short or empty);
    split s covers keys [s*c*bs, min((s+1)*c*bs, n_keys)).  Empty splits are
    returned as (e, e) with e = min(s*c*bs, n_keys).
    """
    if num_splits < 1 or block_size < 1 or n_keys < 0:
        raise ValueError("bad split arguments")
    nblk = -(-n_keys // block_size)
    c = -(-nblk // num_splits) if nblk else 0
    out = []
    for s in range(num_splits):
        lo = min(s * c * block_size, n_keys)
        hi = min((s + 1) * c * block_size, n_keys)
        out.append((lo, hi))
    return out


def combine_splits(o_parts, lse_parts):
    """Merge softmax partials of disjoint key sets.

    With lse_s = log sum_{j in s} exp(s_j) and o_s = the normalised output of
    split s, the full softmax output is sum_s exp(lse_s - LSE) o_s with
    LSE = log sum_s exp(lse_s): an exact identity of softmax over a partition.
    Splits with lse = -inf (no keys) get weight 0; all-empty gives o = 0,
    LSE = -inf.  o_parts [S, ..., d], lse_parts [S, ...].
    """
    o_parts = np.asarray(o_parts, F64)
    lse_parts = np.asarray(lse_parts, F64)
    mx = lse_parts.max(axis=0)
    finite = np.isfinite(mx)
    safe = np.where(finite, mx, 0.0)
    w = np.where(np.isfinite(lse_parts), np.exp(lse_parts - safe), 0.0)
    z = w.sum(axis=0)
    lse = np.where(finite, safe + np.log(np.where(finite, z, 1.0)), -np.inf)
    zz = np.where(finite, z, 1.0)
    o = (w[..., None] * o_parts).sum(axis=0) / zz[..., None]
    o = np.where(finite[..., None], o, 0.0)
    return o, lse


def out_projection(o_lat, w_uv):
    """o_i = W^UV_i o_lat_i for every row and head (eq. 11 moved past the softmax sum).

    o_lat [T, n_h, d_c], w_uv [n_h, d_h, d_c] -> [T, n_h, d_h].
    """
    o_lat = np.asarray(o_lat, F64)
    w_uv = np.asarray(w_uv, F64)
    T, n_h, _ = o_lat.shape
    out = np.empty((T, n_h, w_uv.shape[1]))
    for i in range(n_h):
        out[:, i, :] = o_lat[:, i, :] @ w_uv[i].T
    return out


# ---------------------------------------------------------------- producers
def rms_norm(x, gain, eps: float):
    """The latent RMSNorm (reading R8) over the last axis of x."""
    x = np.asarray(x, F64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return np.asarray(gain, F64) * x / np.sqrt(ms + float(eps))


def kv_produce(h, w_dkv, kv_gain, w_kr, pos, base: float, eps: float, theta=None):
    """Cache rows of new tokens from their hidden states h [T, d_model].

    c^KV_t = RMSNorm(W^DKV h_t)          (notes §2.1.2 eq. 9, blog part 3 §3.1.1; R8)
    k^R_t  = W^KR h_t, rotated at pos_t  (blog §2.2.2; R9)
    Returns (c_kv [T, d_c], k_r [T, d_R] before rotation, rows [T, d_c + d_R]),
    rows being what kv_cache_rows caches for them.
    """
    h = np.asarray(h, F64)
    c_kv = rms_norm(h @ np.asarray(w_dkv, F64).T, kv_gain, eps)
    k_r = h @ np.asarray(w_kr, F64).T
    return c_kv, k_r, kv_cache_rows(c_kv, k_r, pos, base, theta)


def q_produce(h, w_dq, q_gain, w_uq, w_qr, n_h: int, eps: float):
    """Per-head queries of tokens h [T, d_model] through the compressed query.

    c^Q_t = RMSNorm(W^DQ h_t)    (notes §2.1.2 eq. 12, blog part 3 §3.1.1; R8)
    q^C_t = W^UQ c^Q_t           (eq. 13), split into heads of d_h
    q^R_t = W^QR c^Q_t           (blog §2.2.2; R9), before rotation
    Returns (c_q [T, d_c'], q_nope [T, n_h, d_h], q_rope [T, n_h, d_R]).
    """
    h = np.asarray(h, F64)
    c_q = rms_norm(h @ np.asarray(w_dq, F64).T, q_gain, eps)
    T = h.shape[0]
    q_nope = (c_q @ np.asarray(w_uq, F64).T).reshape(T, n_h, -1)
    q_rope = (c_q @ np.asarray(w_qr, F64).T).reshape(T, n_h, -1)
    return c_q, q_nope, q_rope


def q_produce_direct(h, w_qc, w_qr, n_h: int):
    """Per-head queries of a model without query compression (reading R10).

    q^C_t = W^QC h_t  (eq. 1's q = W^Q h, split into heads of d_h)
    q^R_t = W^QR h_t  (blog §2.2.2 with h in place of c^Q), before rotation
    Returns (q_nope [T, n_h, d_h], q_rope [T, n_h, d_R]).
    """
    h = np.asarray(h, F64)
    T = h.shape[0]
    q_nope = (h @ np.asarray(w_qc, F64).T).reshape(T, n_h, -1)
    q_rope = (h @ np.asarray(w_qr, F64).T).reshape(T, n_h, -1)
    return q_nope, q_rope


def o_projection(out, w_o):
    """The layer output of eq. 8 (notes §2.1.1): u_t = W^O [o_{t,1}; ...; o_{t,n_h}],
    the heads' outputs out [T, n_h, d_h] concatenated head after head, and
    W^O [d_model, n_h * d_h] stored [d_out, d_in].  Returns u [T, d_model]."""
    out = np.asarray(out, F64)
    T = out.shape[0]
    return out.reshape(T, -1) @ np.asarray(w_o, F64).T


# ------------------------------------------------------- quantised latent cache

E4M3_MAX = 448.0


def e4m3_value(code):
    """Value of OCP FP8 E4M3 bytes (R12): bit 7 sign, bits 6-3 exponent (bias
    7), bits 2-0 mantissa; exponent 0 holds subnormals m/8 * 2^-6; exponent 15
    with mantissa 7 is NaN (the format has no infinities)."""
    code = np.asarray(code, dtype=np.int64)
    sign = np.where(code & 0x80, -1.0, 1.0)
    e = (code >> 3) & 0xF
    m = (code & 0x7).astype(F64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * 2.0 ** (e.astype(F64) - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


def e4m3_round(y):
    """The E4M3 value nearest to y, ties to even, clamped to +-448 (R12).

    In the binade [2^E, 2^(E+1)) the values are spaced 2^(E-3); below 2^-6
    (subnormals) the spacing is 2^-9.  y / spacing is then 8 + mantissa (or
    the subnormal mantissa), so rounding it half-to-even picks the even
    mantissa on a tie."""
    y = np.asarray(y, F64)
    a = np.abs(y)
    _, ex = np.frexp(a)                       # a = f 2^ex, f in [0.5, 1)
    E = np.maximum(ex.astype(F64) - 1.0, -6.0)
    q = 2.0 ** (E - 3.0)
    r = np.minimum(np.rint(a / q) * q, E4M3_MAX)
    return np.copysign(r, y)


def e4m3_code(v):
    """Byte of an exact E4M3 value v (the inverse of e4m3_value on finite values)."""
    v = np.asarray(v, F64)
    a = np.abs(v)
    _, ex = np.frexp(a)
    E = ex - 1
    normal = a >= 2.0 ** -6
    e_field = np.where(normal, E + 7, 0)
    m_field = np.where(normal, (a / 2.0 ** E.astype(F64) - 1.0) * 8.0, a / 2.0 ** -9)
    code = (np.signbit(v).astype(np.int64) << 7) | (e_field.astype(np.int64) << 3) \
        | np.rint(m_field).astype(np.int64)
    return code.astype(np.uint8)


def quantize_rows(rows, d_c: int):
    """Quantise float32 cache rows [N, d_c + d_R] (R12).

    Returns codes uint8 [N, d_c + d_R] and scales float32 [N, 2] (latent part,
    RoPE part)."""
    rows = np.asarray(rows, dtype=np.float32)
    codes = np.empty(rows.shape, dtype=np.uint8)
    scales = np.empty((rows.shape[0], 2), dtype=np.float32)
    for k, (lo, hi) in enumerate([(0, d_c), (d_c, rows.shape[1])]):
        x = rows[:, lo:hi]
        amax = np.max(np.abs(x), axis=1)
        s = amax / np.float32(E4M3_MAX)                     # float32 division
        s = np.where(amax > 0, s, np.float32(1.0)).astype(np.float32)
        y = x / s[:, None]                                  # float32 division
        codes[:, lo:hi] = e4m3_code(e4m3_round(y.astype(F64)))
        scales[:, k] = s
    return codes, scales


def dequantize_rows(codes, scales, d_c: int):
    """The rows the quantised cache stands for: s * code, float64 (exact)."""
    v = e4m3_value(codes)
    s = np.asarray(scales, F64)
    out = v.copy()
    out[:, :d_c] *= s[:, 0:1]
    out[:, d_c:] *= s[:, 1:2]
    return out


def kv_cache_rows_fp8(c_kv, k_r, pos, base: float, theta=None):
    """Quantised cache rows of tokens at positions pos (R3, R12): the float32
    row [c^KV ; R_pos k^R] (rotation in float64, then rounded to float32),
    quantised.  Returns (codes uint8 [L, d_c + d_R], scales float32 [L, 2])."""
    c_kv = np.asarray(c_kv, F64)
    rows = kv_cache_rows(c_kv, k_r, pos, base, theta).astype(np.float32)
    return quantize_rows(rows, c_kv.shape[1])
