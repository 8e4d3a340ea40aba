"""Seeded synthetic workloads for the five decode configurations.

Structure (lengths, block tables, pool sizes) is drawn with NumPy's PCG64 so it
is identical on every machine; values are drawn with torch's generator, on the
CPU for small cases or directly on the GPU for the multi-GB page pools, and
are bf16 (round-to-nearest-even from fp32 N(0, 1) samples) or FP8 E4M3FN
codes.  Nothing here computes attention.

Recipe (one line per configuration, seeds: structure ``2000 + n``, values
``1000 + n`` for configuration n):

1. ``tiny_gqa``    B=3, seq_lens [30, 32, 70], page 32, 4 blocks per row,
   Hq=8, Hkv=1, D=128.  Rows hold cdiv(L + 1, 32) = 1/2/3 distinct random
   pages of an 8-page pool (room for the next token, as in the worked example
   of "Atención paginada"), -1 padded.
2. ``gqa_sinks``   B=64, Hq=64, Hkv=8, D=128, page 16, L ~ U[1024, 8192],
   40000-page pool, block table = consecutive chunks of one seeded pool
   permutation, 512 blocks per row, per-head sinks N(0, 1).
3. ``gqa_window``  as 2 with window 128 and L ~ U[4096, 32768]; the pool is
   max(40000, sum of pages) pages, 2048 blocks per row.
4. ``mla_verify``  B=32, qlen=4, H=128, Lk=576, Lv=512, page 16,
   L ~ U[2048, 16384], real length L - U{0, 1, 2}; q and cache 0.1 N(0, 1);
   pool = sum of pages, permuted, 1024 blocks per row; FP8 variant quantises
   the bf16 cache with k_scale = amax / 448.
5. ``gqa_skewed``  B=256, Hq=32, Hkv=8, D=128, page 16,
   L = floor(exp(U[ln 16, ln 131072])) with 4 seeded requests at L = 0;
   pool = sum of pages, permuted, 8192 blocks per row, no sinks.
6. ``gqa_verify``  GQA causal verify: as 2 (sinks, L ~ U[1024, 8192]) with
   qlen = 2 verify tokens per request (q [B * 2, Hq, D]) and real length
   L - U{0, 1}.
7. ``gqa_verify4`` as 6 with qlen = 4 (32 score columns per kv head) and
   real length L - U{0, 3}.

Never-attended cache slots (unreferenced pages, slots past L, slots before a
window) can be NaN-poisoned so that any stray read shows up in the output.
"""

from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

BF16_NAN_BITS = 0x7FC0
FP8_NAN_CODE = 0x7F

CONFIGS = {
    "tiny_gqa": dict(index=1, B=3, Hq=8, Hkv=1, D=128, P=32, fixed_lens=[30, 32, 70],
                     max_blocks=4, pool=8, window=0, sinks=False),
    "gqa_sinks": dict(index=2, B=64, Hq=64, Hkv=8, D=128, P=16, len_range=(1024, 8192),
                      max_blocks=512, pool=40000, window=0, sinks=True),
    "gqa_window": dict(index=3, B=64, Hq=64, Hkv=8, D=128, P=16, len_range=(4096, 32768),
                       max_blocks=2048, pool=40000, window=128, sinks=True),
    "mla_verify": dict(index=4, B=32, qlen=4, H=128, Lk=576, Lv=512, P=16,
                       len_range=(2048, 16384), real_drop=(0, 2), max_blocks=1024),
    "gqa_skewed": dict(index=5, B=256, Hq=32, Hkv=8, D=128, P=16,
                       loguniform=(16, 131072), zero_lens=4, max_blocks=8192,
                       pool=0, window=0, sinks=False),
    "gqa_verify": dict(index=6, B=64, Hq=64, Hkv=8, D=128, P=16, len_range=(1024, 8192),
                       max_blocks=512, pool=40000, window=0, sinks=True, qlen=2,
                       real_drop=(0, 1)),
    "gqa_verify4": dict(index=7, B=64, Hq=64, Hkv=8, D=128, P=16, len_range=(1024, 8192),
                        max_blocks=512, pool=40000, window=0, sinks=True, qlen=4,
                        real_drop=(0, 3)),
}


def bf16_bits_from_f32(x) -> np.ndarray:
    """fp32 values -> bfloat16 bit patterns (uint16), round to nearest even."""
    t = torch.as_tensor(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def fp8_codes_from_f32(x) -> np.ndarray:
    """fp32 values (|x| <= 448) -> FP8 E4M3FN codes (uint8), nearest even."""
    t = torch.as_tensor(np.ascontiguousarray(x, dtype=np.float32)).clamp(-448.0, 448.0)
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _cdiv(a: int, b: int) -> int:
    return -(-a // b)


def _chunked_block_table(lens_pages, pool, max_blocks, rng):
    """Consecutive chunks of one seeded permutation of the pool, -1 padded."""
    total = int(np.sum(lens_pages))
    if total > pool:
        raise ValueError(f"pool of {pool} pages cannot hold {total} pages")
    perm = rng.permutation(pool).astype(np.int32)
    bt = np.full((len(lens_pages), max_blocks), -1, dtype=np.int32)
    off = 0
    for b, n in enumerate(lens_pages):
        if n > max_blocks:
            raise ValueError(f"request {b} needs {n} blocks > {max_blocks}")
        bt[b, :n] = perm[off:off + n]
        off += n
    return bt


@dataclasses.dataclass
class GqaWorkload:
    name: str
    B: int
    Hq: int
    Hkv: int
    D: int
    P: int
    seq_lens: np.ndarray          # int32 [B]
    block_table: np.ndarray       # int32 [B, max_blocks]
    num_pages: int
    window: int
    has_sinks: bool
    value_seed: int
    qlen: int = 1                              # verify tokens per request
    real_seq_lens: np.ndarray | None = None    # int32 [B] or None

    @property
    def sm_scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    @property
    def max_blocks(self) -> int:
        return int(self.block_table.shape[1])

    @property
    def rows(self) -> int:
        return self.B * self.qlen

    def row_range(self, b: int, t: int):
        """Keys [lo, hi) of verify token t of request b (t = 0 for decode)."""
        L = int(self.seq_lens[b])
        Lr = L if self.real_seq_lens is None else int(self.real_seq_lens[b])
        hi = max(min(L - self.qlen + 1 + t, Lr), 0)
        lo = max(hi - self.window, 0) if self.window > 0 else 0
        return lo, hi

    def key_range(self, b: int):
        """Keys any row of request b attends: the union of its rows' ranges."""
        lo, _ = self.row_range(b, 0)
        _, hi = self.row_range(b, self.qlen - 1)
        return lo, hi

    def attended_mask(self) -> np.ndarray:
        """bool [num_pages, P]: True where some request attends that slot."""
        m = np.zeros((self.num_pages, self.P), dtype=bool)
        for b in range(self.B):
            lo, hi = self.key_range(b)
            if hi <= lo:
                continue
            pos = np.arange(lo, hi)
            m[self.block_table[b, pos // self.P], pos % self.P] = True
        return m

    def kv_bytes(self) -> int:
        """Attended K and V bytes: sum_b n_b * Hkv * 2 * D * 2 B."""
        n = sum(max(hi - lo, 0) for lo, hi in (self.key_range(b) for b in range(self.B)))
        return int(n) * self.Hkv * 2 * self.D * 2

    def page_bytes(self) -> int:
        """Bytes of the whole pages that hold attended slots."""
        pages = 0
        for b in range(self.B):
            lo, hi = self.key_range(b)
            if hi > lo:
                pages += _cdiv(hi, self.P) - lo // self.P
        return pages * self.Hkv * self.P * 2 * self.D * 2

    def flops(self) -> int:
        n = sum(max(hi - lo, 0) for b in range(self.B) for t in range(self.qlen)
                for lo, hi in (self.row_range(b, t),))
        return int(n) * self.Hq * 4 * self.D

    def values(self, device="cpu", poison=True, fp8=False):
        """Draw q, the page pool and sinks as torch tensors on ``device``.

        Returns dict(q bf16 [B * qlen, Hq, D], kv bf16 [pages, Hkv, P, 2D],
        sinks fp32 [Hq] or None).  With ``poison`` every never-attended slot
        holds bf16 NaN.  With ``fp8`` the cache is FP8 E4M3FN codes (uint8)
        of the bf16 values divided by per-kv-head scales, k_scale / v_scale
        [Hkv] fp32 = amax / 448 of that head's attended K / V values (NaN
        code 0x7F where never attended, with ``poison``).
        """
        dev = torch.device(device)
        g = torch.Generator(device=dev)
        g.manual_seed(self.value_seed)
        q = torch.randn((self.rows, self.Hq, self.D), generator=g, device=dev,
                        dtype=torch.float32).to(torch.bfloat16)
        kv = torch.empty((self.num_pages, self.Hkv, self.P, 2 * self.D),
                         dtype=torch.bfloat16, device=dev)
        chunk = max(1, (1 << 26) // (self.Hkv * self.P * 2 * self.D))
        for p0 in range(0, self.num_pages, chunk):
            p1 = min(self.num_pages, p0 + chunk)
            kv[p0:p1] = torch.randn((p1 - p0, self.Hkv, self.P, 2 * self.D), generator=g,
                                    device=dev, dtype=torch.float32).to(torch.bfloat16)
        sinks = None
        if self.has_sinks:
            sinks = torch.randn((self.Hq,), generator=g, device=dev, dtype=torch.float32)
        if fp8:
            mask = torch.from_numpy(~self.attended_mask()).to(dev)
            ks = torch.empty(self.Hkv, dtype=torch.float32, device=dev)
            vs = torch.empty(self.Hkv, dtype=torch.float32, device=dev)
            codes = torch.empty(kv.shape, dtype=torch.uint8, device=dev)
            for h in range(self.Hkv):
                x = kv[:, h].float().masked_fill(mask[:, :, None], 0.0)
                ka, va = float(x[..., :self.D].abs().max()), float(x[..., self.D:].abs().max())
                ks[h] = ka / 448.0 if ka > 0 else 1.0
                vs[h] = va / 448.0 if va > 0 else 1.0
                x = kv[:, h].float()
                x[..., :self.D] /= ks[h]
                x[..., self.D:] /= vs[h]
                codes[:, h] = x.clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8)
            if poison:
                codes.masked_fill_(mask[:, None, :, None], FP8_NAN_CODE)
            return dict(q=q, kv=codes, sinks=sinks, k_scale=ks, v_scale=vs)
        if poison:
            mask = torch.from_numpy(~self.attended_mask()).to(dev)
            kv.view(torch.int16).masked_fill_(mask[:, None, :, None],
                                              np.int16(BF16_NAN_BITS))
        return dict(q=q, kv=kv, sinks=sinks)


def gqa_workload(name: str, batch=None, len_range=None, seed_offset: int = 0,
                 fixed_lens=None, loguniform=None, zero_lens=None, qlen=None,
                 real_drop=None, fixed_real=None, heads=None, window=None,
                 page_size=None, pool=None) -> GqaWorkload:
    """Structure of a GQA configuration, optionally shrunk for oracle-sized tests.

    ``batch``/``len_range``/``fixed_lens``/``loguniform`` override the
    configuration's batch size and length distribution (same shapes
    otherwise); ``seed_offset`` gives independent draws.  ``qlen``,
    ``real_drop`` (real length = L - U{d0..d1}) and ``fixed_real`` make it a
    verify workload; ``heads`` = (Hq, Hkv), ``window`` and ``page_size``
    override those sizes; ``pool`` = "tight" sizes the page pool to the pages
    the requests use (plus 5).
    """
    c = CONFIGS[name]
    idx = c["index"]
    rng = np.random.Generator(np.random.PCG64(2000 + idx + 7919 * seed_offset))
    B = c["B"] if batch is None else int(batch)
    P = c["P"] if page_size is None else int(page_size)
    fl = fixed_lens if fixed_lens is not None else c.get("fixed_lens")
    if fl is not None:
        lens = np.asarray(fl, dtype=np.int64)
        B = len(lens)
    elif loguniform is not None or (len_range is None and "loguniform" in c):
        lo_l, hi_l = loguniform if loguniform is not None else c["loguniform"]
        lens = np.floor(np.exp(rng.uniform(math.log(lo_l), math.log(hi_l), size=B)))
        lens = np.minimum(lens.astype(np.int64), hi_l)
        nz = c.get("zero_lens", 0) if zero_lens is None else zero_lens
        if nz:
            lens[rng.choice(B, size=min(nz, B), replace=False)] = 0
    else:
        lo_l, hi_l = len_range if len_range is not None else c["len_range"]
        lens = rng.integers(lo_l, hi_l, size=B, endpoint=True).astype(np.int64)
    if name == "tiny_gqa":
        pages_per = [_cdiv(int(L) + 1, P) for L in lens]
    else:
        pages_per = [_cdiv(int(L), P) for L in lens]
    max_blocks = max(c["max_blocks"], max(pages_per) if pages_per else 1)
    if len_range is not None or batch is not None or loguniform is not None:
        max_blocks = max(max(pages_per) if pages_per else 1, 1) + 3
    pool_n = max(c["pool"], int(np.sum(pages_per)))
    if name == "tiny_gqa":
        pool_n = c["pool"]
    if pool == "tight":
        pool_n = int(np.sum(pages_per)) + 5
    pool = pool_n
    bt = _chunked_block_table(pages_per, pool, max_blocks, rng)
    ql = c.get("qlen", 1) if qlen is None else int(qlen)
    real = None
    rd = real_drop if real_drop is not None else c.get("real_drop")
    if fixed_real is not None:
        real = np.asarray(fixed_real, dtype=np.int64)
    elif rd is not None:
        real = lens - rng.integers(rd[0], rd[1], size=B, endpoint=True)
    Hq, Hkv = (c["Hq"], c["Hkv"]) if heads is None else heads
    return GqaWorkload(name=name, B=B, Hq=Hq, Hkv=Hkv, D=c["D"], P=P,
                       seq_lens=lens.astype(np.int32), block_table=bt, num_pages=pool,
                       window=c["window"] if window is None else int(window),
                       has_sinks=c["sinks"], value_seed=1000 + idx + 7919 * seed_offset,
                       qlen=ql, real_seq_lens=None if real is None else real.astype(np.int32))


@dataclasses.dataclass
class MlaWorkload:
    name: str
    B: int
    qlen: int
    H: int
    Lk: int
    Lv: int
    P: int
    seq_lens: np.ndarray
    real_seq_lens: np.ndarray | None
    block_table: np.ndarray
    num_pages: int
    value_seed: int

    @property
    def sm_scale(self) -> float:
        return 1.0 / math.sqrt(192.0)

    @property
    def rows(self) -> int:
        return self.B * self.qlen

    def row_hi(self, b: int, t: int) -> int:
        L = int(self.seq_lens[b])
        Lr = L if self.real_seq_lens is None else int(self.real_seq_lens[b])
        return max(min(L - self.qlen + 1 + t, Lr), 0)

    def request_keys(self, b: int) -> int:
        return max(self.row_hi(b, t) for t in range(self.qlen))

    def attended_mask(self) -> np.ndarray:
        m = np.zeros((self.num_pages, self.P), dtype=bool)
        for b in range(self.B):
            n = self.request_keys(b)
            if n:
                pos = np.arange(n)
                m[self.block_table[b, pos // self.P], pos % self.P] = True
        return m

    def kv_bytes(self, elem_bytes: int = 2) -> int:
        """Latent rows read once per request: sum_b max_t hi * Lk * elem."""
        return sum(self.request_keys(b) for b in range(self.B)) * self.Lk * elem_bytes

    def flops(self) -> int:
        keys = sum(self.row_hi(b, t) for b in range(self.B) for t in range(self.qlen))
        return int(keys) * self.H * 2 * (self.Lk + self.Lv)

    def values(self, device="cpu", poison=True, fp8=False):
        """q bf16 [rows, H, Lk]; latent cache [pages, P, 1, Lk] as bf16, or as
        FP8 E4M3FN codes (uint8) plus the fp32 k_scale = amax / 448 of the
        attended bf16 values when ``fp8``."""
        dev = torch.device(device)
        g = torch.Generator(device=dev)
        g.manual_seed(self.value_seed)
        q = (0.1 * torch.randn((self.rows, self.H, self.Lk), generator=g, device=dev,
                               dtype=torch.float32)).to(torch.bfloat16)
        kv = torch.empty((self.num_pages, self.P, 1, self.Lk), dtype=torch.bfloat16,
                         device=dev)
        chunk = max(1, (1 << 26) // (self.P * self.Lk))
        for p0 in range(0, self.num_pages, chunk):
            p1 = min(self.num_pages, p0 + chunk)
            kv[p0:p1] = (0.1 * torch.randn((p1 - p0, self.P, 1, self.Lk), generator=g,
                                           device=dev, dtype=torch.float32)).to(torch.bfloat16)
        mask = torch.from_numpy(~self.attended_mask()).to(dev)
        out = dict(q=q)
        if fp8:
            att = kv.float().masked_fill(mask[:, :, None, None], 0.0)
            amax = float(att.abs().max())
            k_scale = amax / 448.0 if amax > 0 else 1.0
            codes = (kv.float() / k_scale).clamp(-448.0, 448.0).to(torch.float8_e4m3fn)
            codes = codes.view(torch.uint8)
            if poison:
                codes.masked_fill_(mask[:, :, None, None], FP8_NAN_CODE)
            out.update(kv=codes, k_scale=k_scale)
        else:
            if poison:
                kv.view(torch.int16).masked_fill_(mask[:, :, None, None],
                                                  np.int16(BF16_NAN_BITS))
            out.update(kv=kv, k_scale=1.0)
        return out


def mla_workload(name: str = "mla_verify", batch=None, len_range=None, qlen=None,
                 heads=None, seed_offset: int = 0, fixed_lens=None,
                 fixed_real=None, no_real=False, page_size=None) -> MlaWorkload:
    c = CONFIGS[name]
    idx = c["index"]
    rng = np.random.Generator(np.random.PCG64(2000 + idx + 7919 * seed_offset))
    B = c["B"] if batch is None else int(batch)
    P = c["P"] if page_size is None else int(page_size)
    ql = c["qlen"] if qlen is None else int(qlen)
    if fixed_lens is not None:
        lens = np.asarray(fixed_lens, dtype=np.int64)
        B = len(lens)
    else:
        lo_l, hi_l = len_range if len_range is not None else c["len_range"]
        lens = rng.integers(lo_l, hi_l, size=B, endpoint=True).astype(np.int64)
    real = None
    if fixed_real is not None:
        real = np.asarray(fixed_real, dtype=np.int64)
    elif not no_real:
        d0, d1 = c["real_drop"]
        real = lens - rng.integers(d0, d1, size=B, endpoint=True)
    pages_per = [_cdiv(max(int(L), 0), P) for L in lens]
    max_blocks = max(max(pages_per) if pages_per else 1, 1)
    if batch is None and len_range is None and fixed_lens is None:
        max_blocks = max(max_blocks, c["max_blocks"])
    else:
        max_blocks += 3
    pool = max(int(np.sum(pages_per)), 1)
    bt = _chunked_block_table(pages_per, pool, max_blocks, rng)
    return MlaWorkload(name=name, B=B, qlen=ql, H=c["H"] if heads is None else int(heads),
                       Lk=c["Lk"], Lv=c["Lv"], P=P, seq_lens=lens.astype(np.int32),
                       real_seq_lens=None if real is None else real.astype(np.int32),
                       block_table=bt, num_pages=pool,
                       value_seed=1000 + idx + 7919 * seed_offset)
