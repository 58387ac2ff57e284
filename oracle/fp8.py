"""FP8 (E4M3) KV cache: encoding, quantised append and decode attention --
TEST INFRASTRUCTURE.

What it follows:
  * "让 Agent 跑得快：LLM 推理服务", section 四 (FP8 量化): FP8 is one byte per
    value, half of bf16, so a bandwidth-bound decode moves half the bytes;
    "LLM推理工程实战", section 5.3 (KV Cache量化): the KV cache itself can be
    stored quantised (vLLM's kv_cache_dtype=fp8), attention reading the
    dequantised values.

Readings where the pages leave a step open:
  * The FP8 format is OCP E4M3 without infinities: sign, 4 exponent bits
    (bias 7), 3 mantissa bits; exponent 0 holds the subnormals m * 2^-9;
    S.1111.111 is NaN, so the largest finite magnitude is 448.
  * One scale per cache (k_scale for K, v_scale for V), given by the caller,
    as in vLLM's fp8 KV cache: value = code_value * scale.  Or, as a second
    form, one scale per (physical block, KV head) for each of K and V: every
    scale argument below takes either a number or a [num_blocks,
    num_kv_heads] array, and a value stored in block b for KV head h means
    code_value * scale[b, h].  The caller chooses the scales (finite, > 0),
    for instance from a block's absolute maximum; the append quantises with
    the scale of the block a slot lies in.
  * Quantising x (a bf16 value): y = x / scale in IEEE binary32 (one correctly
    rounded division), clamped to [-448, 448], then rounded to the nearest
    E4M3 value, ties to the even code (the one with an even mantissa).
    Inputs must be finite.
  * Decode attention over the FP8 cache is the bf16 decode of the other
    oracle functions applied to the dequantised keys and values:
    out = softmax_t(scale * <q, k_scale * Kc[t]>) . (v_scale * Vc[t]).
  * Chunked prefill over the FP8 cache is the same with a chunk of Lq query
    rows per sequence at positions ctx - Lq .. ctx - 1, each seeing the keys
    up to its own position when causal ("LLM 推理优化技术全景", Chunked
    Prefill), as the bf16 chunk oracle does.
"""
import numpy as np

E4M3_MAX = 448.0
NAN_CODE = 0x7F


def e4m3_value(code):
    """Real value(s) of E4M3 code(s) (uint8 array or int), float64; NaN for
    the two NaN codes."""
    c = np.asarray(code, dtype=np.int64)
    s = np.where(c >> 7 == 1, -1.0, 1.0)
    e = (c >> 3) & 15
    m = (c & 7).astype(np.float64)
    mag = np.where(e == 0, np.ldexp(m / 8.0, -6), np.ldexp(1.0 + m / 8.0, e - 7))
    mag = np.where((e == 15) & ((c & 7) == 7), np.nan, mag)
    return s * mag


def e4m3_encode(y):
    """Nearest E4M3 code of float32 value(s) y with |y| <= 448, ties to the
    even code.  Arithmetic in float64, exact for float32 inputs."""
    y = np.asarray(y, dtype=np.float32).astype(np.float64)
    if np.any(~np.isfinite(y)) or np.any(np.abs(y) > E4M3_MAX):
        raise ValueError("e4m3_encode takes finite values within +-448")
    a = np.abs(y)
    sign = np.where(np.signbit(y), 0x80, 0)
    code = np.zeros(a.shape, dtype=np.int64)
    sub = a < 2.0 ** -6
    # subnormal range: multiples of 2^-9; a count of 8 is the smallest normal
    # (code 8), which the code arithmetic below gives for free
    code[sub] = np.round(a[sub] * 2.0 ** 9).astype(np.int64)
    nrm = ~sub
    mant, exp = np.frexp(a[nrm])          # a = mant * 2^exp, mant in [0.5, 1)
    e = exp - 1                           # a = (2 mant) * 2^e, 2 mant in [1, 2)
    steps = np.round((2.0 * mant - 1.0) * 8.0).astype(np.int64)  # 0 .. 8, half-even
    code[nrm] = ((e + 7) << 3) + steps     # steps = 8 carries into the exponent
    return (sign | code).astype(np.uint8)


def scale_table(scale, num_blocks, num_kv_heads):
    """A cache's scale as a [num_blocks, num_kv_heads] float64 array: a
    number is the same scale everywhere; an array must have that shape.
    Every scale must be finite and > 0."""
    a = np.asarray(scale, dtype=np.float64)
    if a.ndim == 0:
        a = np.full((num_blocks, num_kv_heads), float(a))
    if a.shape != (num_blocks, num_kv_heads):
        raise ValueError(f"scale table of shape {a.shape}, want {(num_blocks, num_kv_heads)}")
    if not np.all(np.isfinite(a) & (a > 0)):
        raise ValueError("scales must be finite and > 0")
    return a


def quantise(x_bf16_bits, scale):
    """bf16 values (uint16 bit patterns, any shape) -> E4M3 codes, with a
    scale (a number, or binary32 values broadcast against the input)."""
    bits = np.asarray(x_bf16_bits).astype(np.uint16).astype(np.uint32) << 16
    x = bits.view(np.float32)
    y = x / np.asarray(scale, dtype=np.float32)     # one binary32 division
    y = np.clip(y, np.float32(-E4M3_MAX), np.float32(E4M3_MAX))
    return e4m3_encode(y)


def kv_append_fp8(k_new, v_new, slot_mapping, k_cache, v_cache, k_scale, v_scale):
    """Quantised append: token t's K/V rows (bf16 bits [T, Hkv, D]) are
    quantised with the scales of the block their slot s = slot_mapping[t]
    lies in (block s // bs, one scale per KV head) and written at slot s of
    the code pools ([NB, bs, Hkv, D] uint8), skipped when s < 0.  Returns
    new pools."""
    kc, vc = np.array(k_cache, dtype=np.uint8), np.array(v_cache, dtype=np.uint8)
    nb, bs, hkv, d = kc.shape
    slots = np.asarray(slot_mapping, dtype=np.int64)
    ks, vs = scale_table(k_scale, nb, hkv), scale_table(v_scale, nb, hkv)
    k_new, v_new = np.asarray(k_new), np.asarray(v_new)
    if k_new.shape != (slots.shape[0], hkv, d) or v_new.shape != k_new.shape:
        raise ValueError("shape mismatch")
    flat_k = kc.reshape(nb * bs, hkv, d)
    flat_v = vc.reshape(nb * bs, hkv, d)
    for t, s in enumerate(slots):
        if s < 0:
            continue
        if s >= nb * bs:
            raise ValueError(f"slot {s} outside the pool")
        blk = s // bs
        flat_k[s] = quantise(k_new[t], ks[blk][:, None])
        flat_v[s] = quantise(v_new[t], vs[blk][:, None])
    return kc, vc


def dequantise_rows(codes, scales, ids, n):
    """The first n token rows of a sequence whose blocks are `ids`, as values:
    code value x the scale of (block, KV head).  codes [NB, bs, Hkv, D],
    scales [NB, Hkv]; returns [n, Hkv, D] float64."""
    nb, bs, hkv, d = codes.shape
    vals = e4m3_value(codes[ids]) * scales[ids][:, None, :, None]
    return vals.reshape(len(ids) * bs, hkv, d)[:n]


def paged_decode_fp8(q_bf16_bits, k_codes, v_codes, k_scale, v_scale, block_table,
                     context_lens, scale):
    """fp64 decode attention over FP8 pools: for sequence i and query head h
    (KV head h // (Hq / Hkv)), gather the first context_lens[i] token rows
    through the block table, dequantise (code value x cache scale), then
    softmax(scale * q.K) . V with the stable three-sweep softmax.  The scales
    are numbers or [NB, Hkv] tables (see scale_table).  A row with no keys is
    all zeros.  Returns [B, Hq, D] float64."""
    qb = np.asarray(q_bf16_bits).astype(np.uint16).astype(np.uint32) << 16
    q = qb.view(np.float32).astype(np.float64)
    kc, vc = np.asarray(k_codes, dtype=np.uint8), np.asarray(v_codes, dtype=np.uint8)
    bt = np.asarray(block_table, dtype=np.int64)
    ctx = np.asarray(context_lens, dtype=np.int64)
    nb, bs, hkv, d = kc.shape
    b, hq, d2 = q.shape
    if d2 != d or hq % hkv or bt.shape[0] != b or ctx.shape != (b,):
        raise ValueError("shape mismatch")
    g = hq // hkv
    ks, vs = scale_table(k_scale, nb, hkv), scale_table(v_scale, nb, hkv)
    out = np.zeros((b, hq, d), dtype=np.float64)
    for i in range(b):
        n = int(ctx[i])
        if n == 0:
            continue
        nblk = -(-n // bs)
        ids = bt[i, :nblk]
        if np.any(ids < 0) or np.any(ids >= nb):
            raise ValueError(f"sequence {i}: block id outside the pool")
        k = dequantise_rows(kc, ks, ids, n)
        v = dequantise_rows(vc, vs, ids, n)
        for h in range(hq):
            kv = h // g
            s = float(scale) * (k[:, kv, :] @ q[i, h])
            p = np.exp(s - s.max())
            out[i, h] = (p @ v[:, kv, :]) / p.sum()
    return out


def paged_prefill_fp8(q_bf16_bits, k_codes, v_codes, k_scale, v_scale, block_table,
                      context_lens, cu_q_lens, scale, causal=True):
    """fp64 chunked attention over FP8 pools: sequence i has query rows
    cu_q_lens[i] .. cu_q_lens[i + 1] - 1; row r sits at position
    context_lens[i] - Lq_i + r and sees keys 0 .. position (all
    context_lens[i] keys when not causal), dequantised (code value x its
    scale: a number, or an [NB, Hkv] table), with the stable three-sweep
    softmax.  Returns [sum Lq, Hq, D] float64."""
    qb = np.asarray(q_bf16_bits).astype(np.uint16).astype(np.uint32) << 16
    q = qb.view(np.float32).astype(np.float64)
    kc, vc = np.asarray(k_codes, dtype=np.uint8), np.asarray(v_codes, dtype=np.uint8)
    bt = np.asarray(block_table, dtype=np.int64)
    ctx = np.asarray(context_lens, dtype=np.int64)
    cu = np.asarray(cu_q_lens, dtype=np.int64)
    nb, bs, hkv, d = kc.shape
    t, hq, d2 = q.shape
    if d2 != d or hq % hkv or bt.shape[0] != ctx.shape[0] or cu.shape[0] != ctx.shape[0] + 1:
        raise ValueError("shape mismatch")
    if cu[-1] != t:
        raise ValueError("cu_q_lens does not end at the number of query rows")
    g = hq // hkv
    ks, vs = scale_table(k_scale, nb, hkv), scale_table(v_scale, nb, hkv)
    out = np.zeros((t, hq, d), dtype=np.float64)
    for i in range(ctx.shape[0]):
        n, lq = int(ctx[i]), int(cu[i + 1] - cu[i])
        if lq == 0 or n == 0:
            continue
        if lq > n:
            raise ValueError(f"sequence {i}: {lq} query rows over {n} keys")
        nblk = -(-n // bs)
        ids = bt[i, :nblk]
        if np.any(ids < 0) or np.any(ids >= nb):
            raise ValueError(f"sequence {i}: block id outside the pool")
        k = dequantise_rows(kc, ks, ids, n)
        v = dequantise_rows(vc, vs, ids, n)
        for r in range(lq):
            seen = n - lq + r + 1 if causal else n
            for h in range(hq):
                kv = h // g
                s_ = float(scale) * (k[:seen, kv, :] @ q[cu[i] + r, h])
                p_ = np.exp(s_ - s_.max())
                out[cu[i] + r, h] = (p_ @ v[:seen, kv, :]) / p_.sum()
    return out
