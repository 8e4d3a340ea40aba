"""Plain fp64 definition of paged (split-KV) decode attention, GQA and MLA.

TEST INFRASTRUCTURE ONLY (see the package docstring): never called by the
product path.

What is computed.  Split-KV decode reaches exactly the plain softmax-attention
result: splitting the keys and merging the partial results by their
log-sum-exp is an exact re-association (module docstring of the page
"vllm.models.flint.ops.decode_attention": per-split unnormalised O, m and l
merged into one result).  So the oracle is the plain definition written out in
float64, with the page-gather through the block table, the causal row limit,
the sliding window and the sinks as the pages state them.  The split/merge
functions exist only so the tests can check that merging partials reproduces
the one-split result.

Parity status per function (what pins it, see tests/test_oracle_pins.py):

* ``bf16_bits_to_f64``            pinned: exact spot values, round trip.
* ``fp8_e4m3fn_table`` / bits      pinned: OCP e4m3fn spot values, and all
                                   256 codes against torch's float8_e4m3fn.
* ``row_key_range``                pinned: closed-form causal cases.
* ``attend``                       pinned: brute-force masked dense softmax,
                                   torch fp64 SDPA, closed forms with q = 0.
* ``gqa_decode``                   pinned: worked block-table example of
                                   "Atención paginada", marker keys,
                                   permutation invariance, window and sink
                                   special cases.
* ``gqa_verify``                   pinned: reduces to ``gqa_decode`` at
                                   qlen = 1; each row equals a one-token
                                   decode over its own prefix (hand-computed
                                   limits); dense causal brute force with a
                                   window and sinks; empty rows; the FP8
                                   cache equals the bf16 cache of its
                                   dequantised values (torch's e4m3fn
                                   decoding, power-of-two per-head scales).
* ``varlen_row_requests``          pinned: the row -> request map of the
                                   worked varlen example (golden fixture).
* ``gqa_verify_varlen``            pinned: equals ``gqa_verify`` bitwise when
                                   every request has the same qlen; dense
                                   causal brute force with per-request qlen
                                   (0 included), window and sinks.
* ``mla_verify``                   pinned: dense causal brute force, marker
                                   keys at the row limit, empty rows.
* ``kv_append``                    pinned: the worked example's placement
                                   of each new token, every other byte
                                   unchanged, append-then-decode reads the
                                   new token as the last key.
* ``gqa_partials``/``merge_partials`` pinned: equality across split counts,
                                   LSE consistency.
* ``verify_num_kv_splits``         pinned: hand-evaluated values.
"""

from __future__ import annotations

import numpy as np

LOG2E = 1.4426950408889634
LN2 = 0.6931471805599453


# ---------------------------------------------------------------------------
# Exact decoding of the storage formats
# ---------------------------------------------------------------------------

def bf16_bits_to_f64(bits) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float64, exactly.

    A bfloat16 value is the upper half of an IEEE binary32 word, so shifting
    the 16 bits into the high half and reinterpreting gives the exact value.
    """
    b = np.asarray(bits)
    if b.dtype != np.uint16:
        b = b.view(np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def fp8_e4m3fn_table() -> np.ndarray:
    """Value of every OCP FP8 E4M3 ("fn": finite, no infinities) code, fp64.

    Format: 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits.
    Exponent field 0 encodes subnormals m/8 * 2**-6; fields 1..15 encode
    (1 + m/8) * 2**(e - 7); the single pattern S.1111.111 is NaN (there is no
    infinity), so the largest finite magnitude is 1.75 * 2**8 = 448.  The
    cache of the MLA verify op may be stored in this format and is dequantised
    by one scalar ``k_scale`` ("vllm.v1.attention.ops.triton_decode_attention",
    ``decode_attention_fwd_verify``, parameter ``k_scale``).
    """
    table = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        exp = (code >> 3) & 0xF
        man = code & 0x7
        if exp == 0xF and man == 0x7:
            table[code] = np.nan
        elif exp == 0:
            table[code] = sign * (man / 8.0) * 2.0 ** (-6)
        else:
            table[code] = sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)
    return table


_FP8_TABLE = fp8_e4m3fn_table()


def fp8_bits_to_f64(codes) -> np.ndarray:
    """FP8 E4M3FN codes (uint8) -> float64 through the table above."""
    c = np.asarray(codes)
    if c.dtype != np.uint8:
        c = c.view(np.uint8)
    return _FP8_TABLE[c]


# ---------------------------------------------------------------------------
# Which keys a query row attends
# ---------------------------------------------------------------------------

def row_key_range(seq_len: int, qlen: int = 1, t: int = 0, real_len=None,
                  window: int = 0) -> tuple[int, int]:
    """Key positions ``[lo, hi)`` attended by verify row ``t`` of a request.

    * Row limit: ``hi = max(min(L - qlen + 1 + t, L_real), 0)``, with
      ``L_real = L`` when no real length is given
      ("vllm.v1.attention.ops.triton_decode_attention",
      ``decode_attention_fwd_verify``, parameter ``real_seq_lens``).  With one
      query token (qlen = 1, t = 0) this is ``hi = L``: the decode query sees
      all ``seq_lens[b]`` keys, which include the current token
      ("vllm.models.flint.ops.decode_attention", ``flint_decode_attention``,
      parameter ``seq_lens``).
    * Sliding window: attend the last ``window`` positions,
      ``lo = max(hi - window, 0)`` (same page, ``_FlintDecodeAttention.kernel``:
      ``start_tok = max(seq_len - window, 0)``; parameter ``window``).  A
      window <= 0 means full attention.
    """
    L = int(seq_len)
    L_real = L if real_len is None else int(real_len)
    hi = max(min(L - qlen + 1 + t, L_real), 0)
    lo = max(hi - int(window), 0) if window and window > 0 else 0
    return lo, hi


# ---------------------------------------------------------------------------
# The attention definition
# ---------------------------------------------------------------------------

def attend(q, K, V, sm_scale: float, sinks=None):
    """Softmax attention of query rows over one key set, in float64.

    ``q`` [n, d], ``K`` [m, d], ``V`` [m, dv]; ``sinks`` is None or [n] sink
    logits.  Returns ``(O [n, dv], lse [n])`` with

        x_j = sm_scale * q . K_j
        LSE = log(sum_j exp(x_j))                      (natural log)
        O   = sum_j exp(x_j) V_j / (sum_j exp(x_j) + exp(sink))

    The sink is a logit already in the scaled domain that enters only the
    denominator ("vllm.models.flint.ops.decode_attention", module docstring:
    the sink adds exp2(sink * log2(e) - m * c) to the final denominator, with
    c = scale * log2(e), i.e. exp(sink - scale * m) relative to the running
    max).  LSE is taken over the keys only, so it is -inf for a row with no
    key ("vllm.v1.attention.ops.triton_decode_attention", parameter ``lse``)
    and partial LSEs stay mergeable.  A row with no key has O = 0
    ("vllm.models.flint.ops.decode_attention", parameter ``seq_lens``:
    0 writes zeros).
    """
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    n = q.shape[0]
    dv = V.shape[1]
    if K.shape[0] == 0:
        return np.zeros((n, dv)), np.full(n, -np.inf)
    x = sm_scale * (q @ K.T)                        # [n, m]
    M = x.max(axis=1, keepdims=True)
    e = np.exp(x - M)
    s = e.sum(axis=1)
    lse = M[:, 0] + np.log(s)
    denom = s.copy()
    if sinks is not None:
        denom = denom + np.exp(np.asarray(sinks, dtype=np.float64) - M[:, 0])
    O = (e @ V) / denom[:, None]
    return O, lse


# ---------------------------------------------------------------------------
# GQA paged decode
# ---------------------------------------------------------------------------

def _gather_positions(block_table_row, positions, page_size):
    """Physical page and in-page slot of each logical key position.

    The block table row lists, in order, the physical pages holding a
    sequence's cache; position j lives in page ``row[j // page_size]`` at slot
    ``j % page_size`` ("Atención paginada", Ruta de decodificación: the block
    table has shape (batch_size, max_blocks_per_seq) and each row holds the
    physical locations of the request's cache blocks; -1 marks unallocated
    blocks, which an attended position never reaches).
    """
    pos = np.asarray(positions, dtype=np.int64)
    pages = np.asarray(block_table_row, dtype=np.int64)[pos // page_size]
    if pages.size and pages.min() < 0:
        raise ValueError("an attended position maps to an unallocated (-1) block")
    return pages, pos % page_size


def gqa_decode(q_bits, kv_bits, block_table, seq_lens, sm_scale, sinks=None,
               window: int = 0):
    """Paged GQA decode, one query token per request, in float64.

    Inputs (raw storage, exactly as the kernel reads it):

    * ``q_bits``      uint16 [B, Hq, D] bf16 queries;
    * ``kv_bits``     uint16 [num_pages, Hkv, P, 2D] bf16 HND cache with K in
      ``[..., :D]`` and V in ``[..., D:]``
      ("vllm.models.flint.ops.decode_attention", ``flint_decode_attention``,
      parameter ``kv_cache``);
    * ``block_table`` int [B, max_blocks]; ``seq_lens`` int [B];
    * ``sinks``       None or float [Hq] sink logits; ``window`` <= 0 for full
      attention.

    Query head h reads kv head ``h // G`` with ``G = Hq / Hkv`` (contiguous
    groups: the same page's kernel maps kv head kvh to query heads
    ``kvh * 8 + 0..7``).  Returns ``(O [B, Hq, D], LSE [B, Hq])``.
    """
    q = bf16_bits_to_f64(q_bits)
    kv = np.asarray(kv_bits)
    B, Hq, D = q.shape
    _, Hkv, P, two_d = kv.shape
    assert two_d == 2 * D and Hq % Hkv == 0
    G = Hq // Hkv
    O = np.zeros((B, Hq, D))
    lse = np.full((B, Hq), -np.inf)
    for b in range(B):
        lo, hi = row_key_range(int(seq_lens[b]), window=window)
        pages, slots = _gather_positions(block_table[b], np.arange(lo, hi), P)
        for kvh in range(Hkv):
            rows = bf16_bits_to_f64(kv[pages, kvh, slots, :])      # [n, 2D]
            hs = slice(kvh * G, (kvh + 1) * G)
            sk = None if sinks is None else np.asarray(sinks, np.float64)[hs]
            O[b, hs], lse[b, hs] = attend(q[b, hs], rows[:, :D], rows[:, D:],
                                          sm_scale, sk)
    return O, lse


def gqa_verify(q_bits, kv_bits, block_table, seq_lens, qlen: int, sm_scale,
               sinks=None, window: int = 0, real_seq_lens=None, kv_dtype: str = "bf16",
               k_scale=1.0, v_scale=1.0):
    """Paged GQA causal verify: qlen query tokens per request, in float64.

    The verify form of GQA decode.  The rows, their limits and the output
    layout are those of "vllm.v1.attention.ops.triton_decode_attention",
    ``decode_attention_fwd_verify`` (q [B * qlen, H, D] with the verify
    tokens of a request contiguous; row t of request b attends keys below
    ``hi = max(min(L - qlen + 1 + t, L_real), 0)``; one block-table row per
    request); the cache layout, the query-head grouping, the sinks and the
    sliding window are those of ``gqa_decode`` ("vllm.models.flint.ops.
    decode_attention").  The window of row t covers its last ``window``
    keys, ``[max(hi - window, 0), hi)``.

    An FP8 cache (``kv_dtype = "fp8_e4m3fn"``, uint8 codes) holds K and V
    scaled by ``k_scale`` and ``v_scale``: value = code value * scale, as the
    scalar ``k_scale`` dequantises an FP8 cache in
    "vllm.v1.attention.ops.triton_decode_attention" (parameter ``k_scale``);
    GQA's K and V are separate tensors, so each has its own scale, a scalar
    or one per kv head.

    Returns ``(O [B * qlen, Hq, D], LSE [B * qlen, Hq])``.  With qlen = 1 and
    no real lengths this is ``gqa_decode``.
    """
    q = bf16_bits_to_f64(q_bits)
    kv = np.asarray(kv_bits)
    rows, Hq, D = q.shape
    _, Hkv, P, two_d = kv.shape
    assert two_d == 2 * D and Hq % Hkv == 0 and rows % qlen == 0
    G = Hq // Hkv
    ks = np.broadcast_to(np.asarray(k_scale, np.float64), (Hkv,))
    vs = np.broadcast_to(np.asarray(v_scale, np.float64), (Hkv,))

    def decode_rows(raw, kvh):
        if kv_dtype == "bf16":
            return bf16_bits_to_f64(raw)
        if kv_dtype == "fp8_e4m3fn":
            vals = fp8_bits_to_f64(raw)
            vals[:, :D] *= ks[kvh]
            vals[:, D:] *= vs[kvh]
            return vals
        raise ValueError(kv_dtype)
    B = rows // qlen
    O = np.zeros((rows, Hq, D))
    lse = np.full((rows, Hq), -np.inf)
    for b in range(B):
        L = int(seq_lens[b])
        L_real = None if real_seq_lens is None else int(real_seq_lens[b])
        for t in range(qlen):
            r = b * qlen + t
            lo, hi = row_key_range(L, qlen, t, L_real, window)
            pages, slots = _gather_positions(block_table[b], np.arange(lo, hi), P)
            for kvh in range(Hkv):
                kvrows = decode_rows(kv[pages, kvh, slots, :], kvh)    # [n, 2D]
                hs = slice(kvh * G, (kvh + 1) * G)
                sk = None if sinks is None else np.asarray(sinks, np.float64)[hs]
                O[r, hs], lse[r, hs] = attend(q[r, hs], kvrows[:, :D], kvrows[:, D:],
                                              sm_scale, sk)
    return O, lse


# ---------------------------------------------------------------------------
# MLA causal verify
# ---------------------------------------------------------------------------

def varlen_row_requests(cu_seqlens_q) -> np.ndarray:
    """Request index of every query row of a variable-length batch.

    The rows of request b are ``cu_seqlens_q[b] .. cu_seqlens_q[b + 1] - 1``:
    cumulative query lengths map each query token to its sequence ("Atención
    paginada", Ruta Varlen, Mecanismo de indexación and its example).
    """
    cu = np.asarray(cu_seqlens_q, dtype=np.int64)
    return np.repeat(np.arange(len(cu) - 1), np.diff(cu))


def gqa_verify_varlen(q_bits, kv_bits, block_table, seq_lens, cu_seqlens_q, sm_scale,
                      sinks=None, window: int = 0, real_seq_lens=None,
                      kv_dtype: str = "bf16", k_scale=1.0, v_scale=1.0):
    """Paged GQA causal verify with a query length per request, in float64.

    Request b has ``qlen_b = cu_seqlens_q[b + 1] - cu_seqlens_q[b]`` query
    tokens in rows ``cu_seqlens_q[b] + t`` ("Atención paginada", Ruta
    Varlen: cumulative query lengths index the rows; a request may have no
    query token).  Row t attends the keys ``row_key_range(L, qlen_b, t,
    L_real, window)``: the verify rule of "vllm.v1.attention.ops.
    triton_decode_attention" with the request's own qlen.  Cache, grouping,
    sinks, window and FP8 scales as in ``gqa_verify``.

    Returns ``(O [total_rows, Hq, D], LSE [total_rows, Hq])``.
    """
    q = bf16_bits_to_f64(q_bits)
    kv = np.asarray(kv_bits)
    rows, Hq, D = q.shape
    _, Hkv, P, two_d = kv.shape
    cu = np.asarray(cu_seqlens_q, dtype=np.int64)
    assert two_d == 2 * D and Hq % Hkv == 0 and cu[-1] == rows and np.all(np.diff(cu) >= 0)
    G = Hq // Hkv
    ks = np.broadcast_to(np.asarray(k_scale, np.float64), (Hkv,))
    vs = np.broadcast_to(np.asarray(v_scale, np.float64), (Hkv,))
    O = np.zeros((rows, Hq, D))
    lse = np.full((rows, Hq), -np.inf)
    for b in range(len(cu) - 1):
        L = int(seq_lens[b])
        L_real = None if real_seq_lens is None else int(real_seq_lens[b])
        n = int(cu[b + 1] - cu[b])
        for t in range(n):
            r = int(cu[b]) + t
            lo, hi = row_key_range(L, n, t, L_real, window)
            pages, slots = _gather_positions(block_table[b], np.arange(lo, hi), P)
            for kvh in range(Hkv):
                raw = kv[pages, kvh, slots, :]
                if kv_dtype == "bf16":
                    kvrows = bf16_bits_to_f64(raw)
                elif kv_dtype == "fp8_e4m3fn":
                    kvrows = fp8_bits_to_f64(raw)
                    kvrows[:, :D] *= ks[kvh]
                    kvrows[:, D:] *= vs[kvh]
                else:
                    raise ValueError(kv_dtype)
                hs = slice(kvh * G, (kvh + 1) * G)
                sk = None if sinks is None else np.asarray(sinks, np.float64)[hs]
                O[r, hs], lse[r, hs] = attend(q[r, hs], kvrows[:, :D], kvrows[:, D:],
                                              sm_scale, sk)
    return O, lse


def mla_verify(q_bits, kv, block_table, seq_lens, real_seq_lens, qlen: int,
               sm_scale: float, Lv: int, kv_dtype: str = "bf16",
               k_scale: float = 1.0, page_size=None):
    """Causal MLA verify over a per-request block table, in float64.

    Follows "vllm.v1.attention.ops.triton_decode_attention",
    ``decode_attention_fwd_verify``:

    * ``q_bits`` uint16 [B * qlen, H, Lk]; the qlen verify rows of a request
      are contiguous (parameter ``q``);
    * ``kv`` is the paged latent cache, [num_pages, P, 1, Lk] or
      [num_pages * P, 1, Lk] (parameter ``k_buffer``), as uint16 bf16 bits or
      uint8 FP8 E4M3FN codes dequantised by the scalar ``k_scale``;
    * V is ``K[..., :Lv]``: the same latent row, only its first Lv dims
      (parameter ``v_buffer``);
    * the block table has one row per request, shared by its qlen rows
      (parameter ``req_to_token``: not repeated);
    * row t of request b attends ``[0, hi)`` with
      ``hi = max(min(L - qlen + 1 + t, L_real), 0)``.

    Returns ``(O [B * qlen, H, Lv], LSE [B * qlen, H])``.
    """
    q = bf16_bits_to_f64(q_bits)
    kv = np.asarray(kv)
    if kv.ndim == 3:
        if page_size is None:
            raise ValueError("page_size is required for a 3D cache")
        kv = kv.reshape(-1, page_size, 1, kv.shape[-1])
    P = kv.shape[1]
    rows, H, Lk = q.shape
    assert rows % qlen == 0 and kv.shape[-1] == Lk and kv.shape[2] == 1
    B = rows // qlen
    O = np.zeros((rows, H, Lv))
    lse = np.full((rows, H), -np.inf)
    for b in range(B):
        L = int(seq_lens[b])
        L_real = None if real_seq_lens is None else int(real_seq_lens[b])
        his = [row_key_range(L, qlen, t, L_real)[1] for t in range(qlen)]
        n_max = max(his)
        pages, slots = _gather_positions(block_table[b], np.arange(n_max), P)
        raw = kv[pages, slots, 0, :]                                 # [n, Lk]
        if kv_dtype == "bf16":
            lat = bf16_bits_to_f64(raw)
        elif kv_dtype == "fp8_e4m3fn":
            lat = fp8_bits_to_f64(raw) * float(k_scale)
        else:
            raise ValueError(kv_dtype)
        for t in range(qlen):
            r = b * qlen + t
            O[r], lse[r] = attend(q[r], lat[: his[t]], lat[: his[t], :Lv], sm_scale)
    return O, lse


# ---------------------------------------------------------------------------
# KV append (the cache write that precedes decode / verify)
# ---------------------------------------------------------------------------

def kv_append(cache, block_table, seq_lens, qlen: int, src0, src1=None):
    """Write the qlen newest tokens of every request into the paged cache.

    The decode kernel of "Atención paginada" (Ruta de decodificación,
    "Comportamiento de la caché") updates the paged cache in place through
    the block table: token position j of request b lives at slot ``j % P`` of
    page ``block_table[b][j // P]``.  Following "vllm.models.flint.ops.
    decode_attention" (the current token's K/V is written before the decode
    kernel reads the cache, and ``seq_lens`` counts it), the tokens written
    are the last qlen positions of each request: token t (row ``b * qlen + t``
    of the sources) goes to position ``seq_lens[b] - qlen + t``.

    ``cache``  [num_pages, H, P, n] storage elements (any dtype: a byte copy);
    ``src0``   [B * qlen, H, n0] elements copied to ``cache[..., :n0]``;
    ``src1``   None or [B * qlen, H, n1] copied to ``cache[..., n0:n0 + n1]``
               (GQA: K then V of an HND cache; MLA: the latent row alone).

    A token whose position is negative, or whose page entry lies outside the
    block table row or outside ``[0, num_pages)``, is not written (nothing is
    ever written outside the cache).  Returns the updated copy of ``cache``.
    """
    out = np.array(cache, copy=True)
    num_pages, H, P, _ = out.shape
    s0 = np.asarray(src0)
    n0 = s0.shape[2]
    s1 = None if src1 is None else np.asarray(src1)
    bt = np.asarray(block_table)
    B = bt.shape[0]
    for b in range(B):
        for t in range(qlen):
            pos = int(seq_lens[b]) - qlen + t
            if pos < 0 or pos // P >= bt.shape[1]:
                continue
            page = int(bt[b, pos // P])
            if page < 0 or page >= num_pages:
                continue
            r = b * qlen + t
            out[page, :, pos % P, :n0] = s0[r]
            if s1 is not None:
                out[page, :, pos % P, n0:n0 + s1.shape[2]] = s1[r]
    return out


# ---------------------------------------------------------------------------
# Split partials and their merge (used by the self-checks and merge tests)
# ---------------------------------------------------------------------------

def gqa_partials(q_bits, kv_bits, block_table, seq_lens, sm_scale, boundaries,
                 window: int = 0):
    """Per-split partials of GQA decode for explicit key-range partitions.

    ``boundaries(b, lo, hi)`` returns the split edges
    ``lo = e_0 <= e_1 <= ... <= e_S = hi`` (any partition, page-aligned or
    not).  Split s attends ``[e_s, e_{s+1})`` and yields its normalised output
    ``O_s = sum exp(x) V / sum exp(x)`` and natural-log ``lse_s`` (-inf and
    O_s = 0 for an empty split).  This is the fp32 partial layout of the
    verify op's workspace, [rows, H, S, Lv + 1] holding (O_s, lse_s)
    ("vllm.v1.attention.ops.triton_decode_attention", parameter
    ``attn_logits``), information-equivalent to the (O, m, l) partials of
    "vllm.models.flint.ops.decode_attention".  Sinks are not applied here;
    they enter once, at the merge.

    Returns ``(O_parts [B, Hq, S, D], lse_parts [B, Hq, S])``; every request
    must produce the same S.
    """
    q = bf16_bits_to_f64(q_bits)
    kv = np.asarray(kv_bits)
    B, Hq, D = q.shape
    _, Hkv, P, _ = kv.shape
    G = Hq // Hkv
    outs = []
    for b in range(B):
        lo, hi = row_key_range(int(seq_lens[b]), window=window)
        edges = list(boundaries(b, lo, hi))
        assert edges[0] == lo and edges[-1] == hi
        assert all(edges[i] <= edges[i + 1] for i in range(len(edges) - 1))
        S = len(edges) - 1
        Ob = np.zeros((Hq, S, D))
        lb = np.full((Hq, S), -np.inf)
        for s in range(S):
            pages, slots = _gather_positions(block_table[b],
                                             np.arange(edges[s], edges[s + 1]), P)
            for kvh in range(Hkv):
                rows = bf16_bits_to_f64(kv[pages, kvh, slots, :])
                hs = slice(kvh * G, (kvh + 1) * G)
                Ob[hs, s], lb[hs, s] = attend(q[b, hs], rows[:, :D], rows[:, D:],
                                              sm_scale)
        outs.append((Ob, lb))
    S0 = outs[0][1].shape[1]
    assert all(o[1].shape[1] == S0 for o in outs)
    return np.stack([o[0] for o in outs]), np.stack([o[1] for o in outs])


def merge_partials(O_parts, lse_parts, sinks=None):
    """Merge split partials by their log-sum-exp.

    For one (row, head) with partials ``(O_s, lse_s)``, s = 0..S-1:

        M   = max_s lse_s
        w_s = exp(lse_s - M)                (0 for an empty split)
        O   = sum_s w_s O_s / (sum_s w_s + exp(sink - M))
        LSE = M + log(sum_s w_s)

    and ``O = 0``, ``LSE = -inf`` when every split is empty.  This is the
    combine the pages do on unnormalised partials ("vllm.models.flint.ops.
    decode_attention", ``combine_splits``: per-head max over splits, split
    weights exp2(m_s c - m c), weighted l and O, then the sink term in the
    final denominator), restated for normalised partials and natural logs.

    ``O_parts`` [..., S, Dv], ``lse_parts`` [..., S]; ``sinks`` broadcasts
    against ``lse_parts[..., 0]`` (e.g. [H] for [rows, H, S]).
    """
    O_parts = np.asarray(O_parts, dtype=np.float64)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    M = lse_parts.max(axis=-1)
    empty = ~np.isfinite(M)
    M_safe = np.where(empty, 0.0, M)
    w = np.where(np.isfinite(lse_parts), np.exp(lse_parts - M_safe[..., None]), 0.0)
    wsum = w.sum(axis=-1)
    contrib = np.where(w[..., None] > 0, O_parts, 0.0) * w[..., None]
    num = contrib.sum(axis=-2)
    denom = wsum.copy()
    if sinks is not None:
        denom = denom + np.exp(np.asarray(sinks, dtype=np.float64) - M_safe)
    with np.errstate(divide="ignore", invalid="ignore"):
        O = np.where(empty[..., None], 0.0, num / np.where(empty, 1.0, denom)[..., None])
        lse = np.where(empty, -np.inf, M_safe + np.log(np.where(empty, 1.0, wsum)))
    return O, lse


# ---------------------------------------------------------------------------
# Static split cap of the verify op
# ---------------------------------------------------------------------------

def _cdiv(a: int, b: int) -> int:
    return -(-a // b)


def verify_num_kv_splits(max_seq_len: int, batch: int, qlen: int, num_heads: int,
                         sm_count: int, block_h: int, occupancy: float = 1.0,
                         min_work_per_split: int = 64, max_splits: int = 8) -> int:
    """Static upper bound on the KV split count, from static sizes only.

    Restates the rule of "vllm.v1.attention.ops.triton_decode_attention",
    ``verify_num_kv_splits``:

    * a "program" is one (request, row-block) pair, with
      ``ceil(qlen * num_heads / block_h)`` row-blocks per request (the plainest
      reading of the ``verify_row_blocks`` helper the page calls but does not
      show);
    * the ideal split count is ``ceil(max_seq_len / min_work_per_split)``;
    * the number of resident programs ("slots") is ``occupancy * sm_count``;
    * if one split of every request fits in one dispatch round, take as many
      splits as fill that round; otherwise take the n <= min(ideal,
      max_splits) minimising rounds(n) / n, preferring the smallest n within
      5% of the best;
    * the result is clamped to ``[1, min(ideal, 2 * sm_count)]``.
    """
    # programs in flight for one split of every request
    programs = max(1, batch) * _cdiv(qlen * num_heads, block_h)
    ideal = _cdiv(max(1, max_seq_len), max(1, min_work_per_split))
    slots = max(1, int(occupancy * sm_count))
    if programs <= slots:
        # a single round holds one split of every request: fill that round
        n = slots // programs
    else:
        # rounds each split costs, for 1 .. limit splits; the fewest splits
        # whose cost is within 5% of the lowest
        limit = max(1, min(ideal, max_splits))
        cost = {}
        for k in range(1, limit + 1):
            cost[k] = _cdiv(k * programs, slots) / k
        lowest = min(cost.values())
        n = 1
        while cost[n] > lowest * 1.05:
            n += 1
    n = min(n, ideal, 2 * sm_count)
    return max(n, 1)


__all__ = [
    "LN2", "LOG2E", "attend", "bf16_bits_to_f64", "fp8_e4m3fn_table",
    "fp8_bits_to_f64", "gqa_decode", "gqa_partials", "merge_partials",
    "mla_verify", "row_key_range", "verify_num_kv_splits",
]
