"""LOCKS oracle: a plain, slow, fp64 CPU statement of the decode hot path.

TEST INFRASTRUCTURE. Only the tests, the smoke check of the entry module and the
benchmark's CPU-baseline leg may import or run this module. The product library
(kv_cache_page_amd) never imports it, and the two share no code, header, table
or constant generator: everything below is written from the pages.

Pages followed (cited by title + section/equation/algorithm):
  [N] "LOCKS 阅读笔记" -- zhongzhuzhou.org reading notes (2026-07-29) on
      "LOCKS: Page-Local Compact Key Summaries for Efficient Long-Context
      Decoding" (arXiv 2607.24555).
  [S] "Resumo Técnico: LOCKS" -- gist.science technical summary of the same
      paper.

What the method computes, per KV head, per decode step:
  build   (once per full page; [N] §4.1 eq. 2-3, §4.3 Algorithm 1)
  score   (every full page, from the summary only; [N] §4.2 eq. 4)
  shares  (per-query page-mass shares, group average; [N] §4.2 eq. 5)
  select  (sink + most recent + top-(k-2); [N] §4.2, §4.4 Algorithm 2)
  attend  (softmax attention restricted to the selected pages; [N] §3.1 eq. 1,
           §4.4 Algorithm 2 last step)

Readings where the pages leave a step open (each one is also listed in the
design notes of the repository):
  R1 quantiser   symmetric absmax. scale = fp16(RNE(fp32(absmax) / qmax)),
                 qmax = 7 for int4 and 127 for int8; an infinite fp16 scale is
                 replaced by the largest finite fp16 (65504).
                 code = clamp(rint_half_even(fp32(x) / fp32(scale)), -qmax, qmax),
                 i.e. the integer decision is taken in fp32 from the stored
                 scale. absmax == 0 gives scale 0 and all-zero codes.
  R2 granularity basis: one scale per basis column (r scales); coefficients:
                 one scale per token row c_i (B scales); centroid: one scale.
  R3 scale type  fp16.
  R4 slot layout [Vq | Cq | muq | scales | zero pad to a multiple of 16 bytes]
                 Vq: r columns of d/2 bytes, two's-complement int4. Within a
                 column, each little-endian 32-bit word covers 8 consecutive
                 dims 8t..8t+7 and its bytes hold the dim pairs (0,1), (4,5),
                 (2,3), (6,7) in that order, low nibble = first dim of the pair.
                 Cq: B x r int8, row-major (token i at offset i*r).
                 muq: d int8 in dim order.
                 scales: r basis scales, B coefficient scales, 1 centroid
                 scale, fp16 little-endian.
  R5 eigen order descending eigenvalues; canonical sign: each kept basis
                 vector v_k (and its coefficient column) is negated if needed
                 so that its entry of largest |value| is positive, ties going
                 to the lowest dim index.
  R6 zero sigma  component k (k < r) is active iff lambda_k > 1e-6 * trace(G)
                 and lambda_k > 1e-12 * sum_i |k_i|^2 (the floor keeps rounding
                 residue of the centring of equal keys from counting as a
                 direction); an inactive component has v_k = 0, c_{.k} = 0.
  R7 shares      Z_g sums over all summarised (full) pages of the head,
                 including the sink and a full last page; the partial last
                 page has no summary and is not scored.
  R8 sink/recent sink = logical page 0, recent = logical page P-1 (the page
                 holding the newest token, possibly partial). P == 1 gives {0}.
  R9 budget      k counts distinct pages including sink and recent; k >= P
                 selects every page. Equal keys rank the lower page first.
  R17 deferred   the pages put the build of a filled page outside the decode
      build      critical path. In the deferred reading the step whose token
                 completes page P-1 scores only the pages full before that
                 token, F' = floor((len - 1) / B): the just-completed page is
                 this step's unsummarised recent page (selected, not in Z_g)
                 and is summarised after the step.
  R18 basis      the rank x precision ablation of [N] §6 compares int8, int4
      precision  and int2 bases. A b-bit basis uses the R1 quantiser with
                 qmax = 2^(b-1) - 1 (127, 7, 1), one scale per column as R2.
                 Layout of Vq (R4 for int4): int8, one byte per dim in dim
                 order; int2, four dims per byte in dim order, two's-
                 complement two-bit fields, lowest bits first. Coefficients
                 and centroid stay int8.
  R19 merge      [N] §4.2 names two alternatives to the share average of
      rules      eq. 5 for the group's single page set: group-max (a page any
                 query head rates highly) and group-mass (another pooling).
                 Readings: group-max key_j = max_g m_g(j) on the same
                 normalised shares; group-mass key_j = sum_g exp(s_jg) /
                 sum_g Z_g, the pooled unnormalised mass. Selection as R8-R9.
                 Per-head, the "per-head oracle" that [N] §4.2 and the §6
                 ablation compare against (G selections per group): query
                 head g takes its own sink/recent/top-(k-2) by its own share
                 m_g(j) and attends only its own pages.
"""
from __future__ import annotations

import math

import numpy as np

QMAX_INT4 = 7
QMAX_INT8 = 127
BASIS_BITS = (2, 4, 8)
MERGE_RULES = ("share", "max", "mass", "per_head")


def qmax_of(bits):
    """Reading R18: the symmetric b-bit quantiser's largest code."""
    if bits not in BASIS_BITS:
        raise ValueError(f"basis bits must be one of {BASIS_BITS}")
    return 2 ** (bits - 1) - 1
ACTIVE_REL = 1e-6
ACTIVE_FLOOR = 1e-12
FP16_MAX = 65504.0


# ----------------------------------------------------------------------------
# Build: centre, Gram, eigendecomposition, basis/coefficients
# ([N] §4.1 eq. 2-3, §4.3 Algorithm 1). Every function takes a leading page
# axis: keys (n, B, d); a single page is n = 1.
# ----------------------------------------------------------------------------

def centre(keys):
    """Page centroid and deviations: k_i = mu + delta_i with sum_i delta_i = 0
    ([N] §4.1 eq. 2; Algorithm 1 first steps). keys: (n, B, d)."""
    keys = np.asarray(keys, dtype=np.float64)
    mu = keys.mean(axis=-2)
    return mu, keys - mu[..., None, :]


def gram(D):
    """B x B Gram matrix D D^T of the stacked deviations ([N] §4.1 eq. 3)."""
    return D @ np.swapaxes(D, -1, -2)


def eig_descending(G):
    """Eigenpairs of the symmetric Gram, eigenvalues in descending order
    ([N] §4.1 eq. 3; Algorithm 1 eigendecomposition step)."""
    lam, U = np.linalg.eigh(G)
    return lam[..., ::-1], U[..., ::-1]


def spectral_summary(keys, r, active_rel=ACTIVE_REL):
    """Unquantised rank-r summaries ([N] §4.1, Algorithm 1), keys (n, B, d).

    Returns a dict of arrays with a leading page axis:
      mu (n, d); V (n, d, r) = D^T U_r Sigma_r^{-1}; C (n, B, r) = U_r Sigma_r
      (rows are the c_i); lam (n, B) Gram eigenvalues, descending;
      tau (n,) = sum of lam_k for k >= r (the spectral tail); active (n, r);
      dropped (n,) = tail plus the energy of inactive kept components.
    Inactive components (reading R6) get v_k = 0 and c_.k = 0; active ones
    carry the canonical sign of reading R5."""
    keys = np.asarray(keys, dtype=np.float64)
    n, B, d = keys.shape
    assert 1 <= r <= B
    mu, D = centre(keys)
    G = gram(D)
    lam, U = eig_descending(G)
    trace = np.trace(G, axis1=1, axis2=2)
    energy = np.sum(keys * keys, axis=(1, 2))
    lam_r = lam[:, :r]
    active = (lam_r > active_rel * trace[:, None]) & (lam_r > ACTIVE_FLOOR * energy[:, None])
    sigma = np.sqrt(np.where(active, lam_r, 1.0))
    Ur = U[:, :, :r]
    V = np.swapaxes(D, 1, 2) @ Ur / sigma[:, None, :]            # (n, d, r)
    C = Ur * sigma[:, None, :]                                   # (n, B, r)
    V = np.where(active[:, None, :], V, 0.0)
    C = np.where(active[:, None, :], C, 0.0)
    top = np.argmax(np.abs(V), axis=1)                           # first max over d
    sign = np.where(np.take_along_axis(V, top[:, None, :], axis=1)[:, 0, :] < 0.0, -1.0, 1.0)
    V = V * sign[:, None, :]
    C = C * sign[:, None, :]
    tau = np.sum(np.clip(lam[:, r:], 0.0, None), axis=1)
    dropped = tau + np.sum(np.where(active, 0.0, np.clip(lam_r, 0.0, None)), axis=1)
    return dict(mu=mu, V=V, C=C, lam=lam, tau=tau, active=active, dropped=dropped)


# ----------------------------------------------------------------------------
# Quantisation (readings R1-R3; [N] §4.1 storage paragraph, Algorithm 1 last
# steps: basis int4 per column, coefficients and centroid int8 per row)
# ----------------------------------------------------------------------------

def fp16_scale(absmax, qmax):
    """Reading R1: scale = fp16(RNE(fp32(absmax) / qmax)); inf -> 65504."""
    s = (np.asarray(absmax, dtype=np.float32) / np.float32(qmax)).astype(np.float16)
    return np.where(np.isfinite(s), s, np.float16(FP16_MAX)).astype(np.float16)


def quantise(x, qmax, axis):
    """Symmetric absmax quantisation with one scale per slice along `axis`
    (reading R1). Returns (int64 codes shaped like x, fp16 scales)."""
    x = np.asarray(x, dtype=np.float64)
    scale = fp16_scale(np.max(np.abs(x), axis=axis), qmax)
    s32 = np.expand_dims(scale.astype(np.float32), axis)
    safe = np.where(s32 == 0, np.float32(1.0), s32)
    codes = np.rint(x.astype(np.float32) / safe)
    codes = np.where(s32 == 0, 0.0, np.clip(codes, -qmax, qmax))
    return codes.astype(np.int64), scale


def quantise_summary(summary, basis_bits=4):
    """int4 basis (int8 or int2 in the ablation, reading R18) with one scale per
    column, int8 coefficients with one scale per token row c_i, int8 centroid
    with one scale (readings R1-R3)."""
    Vq, sV = quantise(summary["V"], qmax_of(basis_bits), axis=1)   # (n, d, r), (n, r)
    Cq, sC = quantise(summary["C"], QMAX_INT8, axis=2)      # (n, B, r), (n, B)
    muq, smu = quantise(summary["mu"], QMAX_INT8, axis=1)   # (n, d), (n,)
    return dict(Vq=Vq, sV=sV, Cq=Cq, sC=sC, muq=muq, smu=smu)


def dequantise(qs):
    """Codes times their fp16 scale, widened to fp64."""
    V = qs["Vq"] * qs["sV"].astype(np.float64)[:, None, :]
    C = qs["Cq"] * qs["sC"].astype(np.float64)[:, :, None]
    mu = qs["muq"] * qs["smu"].astype(np.float64)[:, None]
    return dict(V=V, C=C, mu=mu)


# ----------------------------------------------------------------------------
# Slot bytes (reading R4)
# ----------------------------------------------------------------------------

def slot_layout(r, B=16, d=128, basis_bits=4):
    """Byte offsets of the summary slot (readings R4, R18)."""
    qmax_of(basis_bits)
    off_v = 0
    off_c = off_v + r * d * basis_bits // 8
    off_mu = off_c + B * r
    off_s = off_mu + d
    payload = off_s + 2 * (r + B + 1)
    stride = (payload + 127) // 128 * 128
    return dict(v=off_v, c=off_c, mu=off_mu, s_v=off_s, s_c=off_s + 2 * r,
                s_mu=off_s + 2 * (r + B), payload=payload, stride=stride)


# nibble position (0..7, low nibble of byte 0 first) that holds dim 8t + j of
# word t: the bytes carry the dim pairs (0,1), (4,5), (2,3), (6,7)
NIBBLE_OF_DIM = np.array([0, 1, 4, 5, 2, 3, 6, 7])


def pack_slots(qs, B=16, d=128, basis_bits=4):
    """Write slots byte-exactly from codes and scales (readings R4, R18).
    Returns uint8 (n, stride)."""
    n, _, r = qs["Vq"].shape
    L = slot_layout(r, B, d, basis_bits)
    out = np.zeros((n, L["stride"]), dtype=np.uint8)
    vbytes = r * d * basis_bits // 8
    cols = np.swapaxes(qs["Vq"], 1, 2)                               # (n, r, d): column k, dim
    if basis_bits == 4:
        # per column k, words t, nibble positions
        cols = cols.reshape(n, r, d // 8, 8) & 0xF                   # dim j of word t
        nib = np.zeros_like(cols)
        nib[..., NIBBLE_OF_DIM] = cols                               # nibble position p
        packed = (nib[..., 0::2] | (nib[..., 1::2] << 4)).astype(np.uint8)  # (n, r, d/8, 4)
    elif basis_bits == 8:
        packed = (cols & 0xFF).astype(np.uint8)
    else:
        f = cols.reshape(n, r, d // 4, 4) & 0x3                      # four dims per byte
        packed = (f[..., 0] | f[..., 1] << 2 | f[..., 2] << 4 | f[..., 3] << 6).astype(np.uint8)
    out[:, L["v"]:L["v"] + vbytes] = packed.reshape(n, vbytes)
    out[:, L["c"]:L["c"] + B * r] = (qs["Cq"].reshape(n, B * r) & 0xFF).astype(np.uint8)
    out[:, L["mu"]:L["mu"] + d] = (qs["muq"] & 0xFF).astype(np.uint8)
    scales = np.concatenate([qs["sV"], qs["sC"], qs["smu"][:, None]], axis=1).astype("<f2")
    out[:, L["s_v"]:L["payload"]] = scales.view(np.uint8)
    return out


def unpack_slots(buf, r, B=16, d=128, basis_bits=4):
    """Read codes and scales back from slot bytes (readings R4, R18)."""
    buf = np.asarray(buf, dtype=np.uint8)
    n = buf.shape[0]
    L = slot_layout(r, B, d, basis_bits)
    vb = buf[:, L["v"]:L["v"] + r * d * basis_bits // 8]
    if basis_bits == 4:
        packed = vb.reshape(n, r, d // 8, 4).astype(np.int64)
        nib = np.zeros(packed.shape[:-1] + (8,), dtype=np.int64)
        nib[..., 0::2] = packed & 0xF
        nib[..., 1::2] = packed >> 4
        nib = np.where(nib >= 8, nib - 16, nib)
        cols = nib[..., NIBBLE_OF_DIM]                              # dim order
    elif basis_bits == 8:
        cols = vb.view(np.int8).astype(np.int64)
    else:
        packed = vb.reshape(n, r, d // 4).astype(np.int64)
        f = np.stack([(packed >> (2 * e)) & 0x3 for e in range(4)], axis=-1)
        cols = np.where(f >= 2, f - 4, f)
    Vq = np.swapaxes(cols.reshape(n, r, d), 1, 2)
    Cq = buf[:, L["c"]:L["c"] + B * r].view(np.int8).astype(np.int64).reshape(n, B, r)
    muq = buf[:, L["mu"]:L["mu"] + d].view(np.int8).astype(np.int64)
    sc = np.ascontiguousarray(buf[:, L["s_v"]:L["payload"]]).view("<f2").astype(np.float16)
    return dict(Vq=Vq, sV=sc[:, :r], Cq=Cq, sC=sc[:, r:r + B], muq=muq, smu=sc[:, r + B])


def build_slots(keys, r, B=16, d=128, basis_bits=4):
    """Algorithm 1 of [N] §4.3 end to end for full pages keys (n, B, d):
    summary, codes, slot bytes. Returns (slots (n, stride), summary, codes)."""
    s = spectral_summary(keys, r)
    qs = quantise_summary(s, basis_bits)
    return pack_slots(qs, B, d, basis_bits), s, qs


# ----------------------------------------------------------------------------
# Score, shares, select ([N] §4.2 eq. 4-5, §4.4 Algorithm 2)
# ----------------------------------------------------------------------------

def logsumexp(x, axis):
    x = np.asarray(x, dtype=np.float64)
    m = np.max(x, axis=axis, keepdims=True)
    m = np.where(np.isfinite(m), m, 0.0)
    return np.squeeze(m, axis=axis) + np.log(np.sum(np.exp(x - m), axis=axis))


def page_scores(q, mu, V, C):
    """Reconstructed page log-mass, [N] §4.2 eq. 4:
      s_hat_j(q_g) = LSE_i ( (q_g . mu_j + (V_j^T q_g) . c_i) / sqrt(d) ).
    q: (G, d); mu: (P, d); V: (P, d, r); C: (P, B, r). Returns (P, G)."""
    q = np.asarray(q, dtype=np.float64)
    d = q.shape[1]
    a = mu @ q.T                                   # (P, G)   q_g . mu_j
    proj = np.einsum("pdr,gd->pgr", V, q)          # (P, G, r) V_j^T q_g
    inner = np.einsum("pgr,pbr->pgb", proj, C)     # (P, G, B) (V^T q).c_i
    logits = (a[:, :, None] + inner) / math.sqrt(d)
    return logsumexp(logits, axis=2)


def exact_page_lse(q, K):
    """Exact page log-mass LSE_i(q_g . k_i / sqrt(d)) from the full keys: the
    quantity the summary approximates, and the ranking that Lemma 1 of [N]
    §3.1 calls worst-case optimal. q: (G, d); K: (P, B, d). Returns (P, G)."""
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    logits = np.einsum("pbd,gd->pgb", K, q) / math.sqrt(q.shape[1])
    return logsumexp(logits, axis=2)


def share_keys(s, rule="share"):
    """Per-query shares m_g(j) = exp(s_jg) / sum_j' exp(s_j'g) and their group
    average m_bar_j = (1/G) sum_g m_g(j) ([N] §4.2 eq. 5), returned in the log
    domain: key_j = log m_bar_j. s: (F, G) over all summarised pages
    (reading R7). rule "max" and "mass" are the alternatives of reading R19:
    log max_g m_g(j), and log (sum_g exp(s_jg) / sum_g Z_g); "per_head" keeps
    every query head's own log share log m_g(j).
    Returns (key (F,) -- (F, G) for "per_head" --, log Z (G,))."""
    s = np.asarray(s, dtype=np.float64)
    G = s.shape[1]
    logZ = logsumexp(s, axis=0)
    if rule == "share":
        key = logsumexp(s - logZ[None, :], axis=1) - math.log(G)
    elif rule == "max":
        key = np.max(s - logZ[None, :], axis=1)
    elif rule == "mass":
        key = logsumexp(s, axis=1) - logsumexp(logZ, axis=0)
    elif rule == "per_head":
        key = s - logZ[None, :]
    else:
        raise ValueError(f"merge rule must be one of {MERGE_RULES}")
    return key, logZ


def select_pages(key, P, k):
    """Sink + most recent + top-(k-2) by key ([N] §4.2 and §4.4 Algorithm 2;
    readings R8, R9). key: (F,) with F >= P-1. Returns the ascending list."""
    if P <= 0:
        return []
    if k >= P:
        return list(range(P))
    chosen = {0, P - 1}
    cand = sorted(range(1, P - 1), key=lambda j: (-float(key[j]), j))
    chosen.update(cand[: max(k - 2, 0)])
    return sorted(chosen)


def attend(q, K, V):
    """Softmax attention of every query over the given tokens:
    o_g = sum_t softmax_t(q_g . k_t / sqrt(d)) v_t. Returns (o (G, d), lse (G,)).
    With K, V restricted to the selected pages this is the renormalised output
    o_S of [N] §3.1 eq. 1 (Algorithm 2 last step)."""
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    logits = (q @ K.T) / math.sqrt(q.shape[1])      # (G, T)
    lse = logsumexp(logits, axis=1)
    w = np.exp(logits - lse[:, None])
    return w @ V, lse


# ----------------------------------------------------------------------------
# Fixed shared sketch ([N] §3.3, Proposition 1): the family of scoring rules
# that see a page only through the query, its centroid and the sketched keys
# W^T k_i for one projection W (d x rho) shared by all pages.
# ----------------------------------------------------------------------------

def shared_sketch_scores(q, K, W):
    """A member of that family: the rank-rho reconstruction of every key in the
    shared basis W (orthonormal columns), k_i ~ mu + W W^T (k_i - mu), scored
    like eq. 4: LSE_i((q . mu + (W^T q) . (W^T (k_i - mu))) / sqrt(d)). It
    depends on the page only through mu and the sketches W^T k_i.
    q: (G, d); K: (P, B, d); W: (d, rho). Returns (P, G)."""
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    mu = K.mean(axis=1)                                    # (P, d)
    sk = K @ W - (mu @ W)[:, None, :]                      # (P, B, rho) = W^T (k_i - mu)
    a = mu @ q.T                                           # (P, G)
    inner = np.einsum("pbr,gr->pgb", sk, q @ W)            # (P, G, B)
    logits = (a[:, :, None] + inner) / math.sqrt(q.shape[1])
    return logsumexp(logits, axis=2)


def blind_direction_pair(K, W, u, c, a=0, b=1):
    """The construction of Proposition 1: keys K (B, d) of one page, u a unit
    vector orthogonal to span(W); returns K' with c u added to key a and
    subtracted from key b (the centroid and every W^T k_i are unchanged)."""
    Kp = np.array(K, dtype=np.float64, copy=True)
    Kp[a] += c * u
    Kp[b] -= c * u
    return Kp


# ----------------------------------------------------------------------------
# One decode step for one (sequence, KV head)
# ----------------------------------------------------------------------------

def n_pages(seq_len, B=16):
    return (seq_len + B - 1) // B


def n_full_pages(seq_len, B=16):
    return seq_len // B


def decode_head(q, Kp, Vp, seq_len, k, slots=None, r=8, mode="quantised", B=16, deferred=False,
                basis_bits=4, merge="share"):
    """Score -> share -> select -> attend for one (seq, KV head).

    q: (G, d). Kp, Vp: (>=P, B, d) logical pages (the tail page may be
    partial). slots: (F, stride) uint8 summary slots of the full pages, or
    None to build them here. mode: "quantised" scores from the codes (eq. 4 as
    deployed), "unquantised" from the fp64 summary, "exact" ranks by the
    exact page LSE (the Lemma 1 selector of [N] §3.1). deferred: reading R17,
    only the pages full before the current token are summarised and scored.
    basis_bits: the stored basis precision (reading R18); merge: the group
    rule that turns scores into selection keys (reading R19).
    Returns dict(scores (F, G), key (F,), sel (list), out (G, d), lse (G,));
    with merge "per_head", key is (F, G) and sel holds one list per query
    head, whose output attends only that head's own pages."""
    q = np.asarray(q, dtype=np.float64)
    G, d = q.shape
    P = n_pages(seq_len, B)
    F = n_full_pages(max(seq_len - 1, 0), B) if deferred else n_full_pages(seq_len, B)
    Kp = np.asarray(Kp, dtype=np.float64)[:P]
    Vp = np.asarray(Vp, dtype=np.float64)[:P]
    if F > 0:
        if mode == "exact":
            scores = exact_page_lse(q, Kp[:F])
        elif mode == "unquantised":
            s = spectral_summary(Kp[:F], r)
            scores = page_scores(q, s["mu"], s["V"], s["C"])
        else:
            if slots is None:
                slots, _, _ = build_slots(Kp[:F], r, B, d, basis_bits)
            dq = dequantise(unpack_slots(slots[:F], r, B, d, basis_bits))
            scores = page_scores(q, dq["mu"], dq["V"], dq["C"])
        key, _ = share_keys(scores, merge)
    else:
        scores = np.zeros((0, G))
        key = np.zeros((0, G)) if merge == "per_head" else np.zeros(0)

    def attend_pages(qq, sel):
        toks_k, toks_v = [], []
        for j in sel:
            m = B if j < P - 1 else seq_len - B * (P - 1)
            toks_k.append(Kp[j, :m]); toks_v.append(Vp[j, :m])
        if not sel:
            return np.zeros((qq.shape[0], d)), np.full(qq.shape[0], -np.inf)
        return attend(qq, np.concatenate(toks_k), np.concatenate(toks_v))

    if merge == "per_head":
        sel = [select_pages(key[:, g], P, k) for g in range(G)]
        per = [attend_pages(q[g:g + 1], sel[g]) for g in range(G)]
        out = np.concatenate([o for o, _ in per])
        lse = np.concatenate([l for _, l in per])
    else:
        sel = select_pages(key, P, k)
        out, lse = attend_pages(q, sel)
    return dict(scores=scores, key=key, sel=sel, out=out, lse=lse)
