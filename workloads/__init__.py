"""Seeded synthetic inputs for the attention library and its oracle.

This module holds no attention arithmetic: it draws random numbers, rounds
them to the storage precision, builds masks' valid lengths and paged block
tables, and describes the five workloads.  Both the GPU tests and the fp64
oracle are fed from here, so both see bit-identical inputs.

Storage precision: bf16 values are produced by round-to-nearest-even of fp32
draws (any multiplier such as x0.5 is applied in fp32 before rounding) and are
returned as raw uint16 bits plus their exact float64 value.

Seeds: ``numpy.random.default_rng([cfg, tensor_id])`` (PCG64) with tensor ids
Q=0, K=1, V=2, dO=3, lengths=4, block permutation=5, K cache=6, V cache=7.
"""

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

TID_Q, TID_K, TID_V, TID_DO, TID_LEN, TID_PERM, TID_KC, TID_VC = range(8)


def rng(cfg_seed, tensor_id):
    return np.random.default_rng([int(cfg_seed), int(tensor_id)])


def bf16_bits(x):
    """fp32 array -> uint16 bf16 bits, round to nearest even (NaN kept NaN)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r = np.where(nan, np.uint16(0x7FC0), r)
    return r


def bf16_value(bits):
    """uint16 bf16 bits -> float32 array holding the same value exactly."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def e4m3_value(codes):
    """uint8 FP8 E4M3 codes (OCP "E4M3FN": 1 sign bit, 4 exponent bits with
    bias 7, 3 mantissa bits; no infinities; S.1111.111 is NaN) -> float64."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    mant = (c & 7).astype(np.float64)
    mag = np.where(e == 0, mant / 8.0 * 2.0 ** -6,
                   (1.0 + mant / 8.0) * np.exp2(e - 7.0))
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return sign * mag


_E4M3_POS = e4m3_value(np.arange(0x7F, dtype=np.uint8))   # 0 .. 448, ascending
E4M3_MAX = float(_E4M3_POS[-1])


def e4m3_codes(x):
    """float array -> uint8 E4M3 codes: nearest value, ties to the even code
    (even mantissa), magnitudes beyond 448 saturated to 448."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), E4M3_MAX)
    hi = np.clip(np.searchsorted(_E4M3_POS, a), 1, 0x7E)
    lo = hi - 1
    dlo, dhi = a - _E4M3_POS[lo], _E4M3_POS[hi] - a
    pick = np.where(dlo < dhi, lo, np.where(dhi < dlo, hi,
                                            np.where(lo % 2 == 0, lo, hi)))
    return (pick | np.where(x < 0, 0x80, 0)).astype(np.uint8)


def to_device(t, device="cuda"):
    """Copy a generated Tensor to a torch GPU tensor with the same bits."""
    import torch
    if t.dtype == "fp8":
        return torch.from_numpy(np.ascontiguousarray(t.store)).to(device)
    if t.dtype == "bf16":
        x = torch.from_numpy(np.ascontiguousarray(t.store).view(np.int16))
        return x.view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(t.store)).to(device)


@dataclass
class Tensor:
    """A generated tensor: storage bits (bf16) or fp32 data, plus exact fp64."""
    dtype: str            # "bf16", "f32" or "fp8"
    store: np.ndarray     # uint16 bits (bf16), float32 (f32), uint8 E4M3 (fp8)
    exact: np.ndarray     # float64 copy of the stored values

    @property
    def shape(self):
        return self.store.shape


def normal(shape, cfg_seed, tensor_id, dtype, mult=1.0):
    """iid N(0,1) * mult, drawn in fp32, stored in ``dtype``."""
    x = rng(cfg_seed, tensor_id).standard_normal(size=shape, dtype=np.float32)
    if mult != 1.0:
        x = (x * np.float32(mult)).astype(np.float32)
    if dtype == "bf16":
        bits = bf16_bits(x)
        return Tensor("bf16", bits, bf16_value(bits).astype(np.float64))
    if dtype == "f32":
        return Tensor("f32", x, x.astype(np.float64))
    raise ValueError(dtype)


def normal_fp8(shape, cfg_seed, tensor_id, mult=1.0, transpose=False):
    """iid N(0,1) * mult drawn in fp32 (as ``normal``) and quantized to FP8
    E4M3 per (batch, head): descale = amax / 448 (fp32), codes =
    E4M3(x / descale).  Returns (Tensor, descale float32 [B*H]).  The
    Tensor's ``exact`` is codes * descale in float64 with the logical
    [B,H,N,d] shape; with transpose=True its ``store`` is [B,H,d,ldv], the
    key axis last and padded with zero codes to ldv = N rounded up to 16.
    """
    B, H, N, d = shape
    x = rng(cfg_seed, tensor_id).standard_normal(size=shape, dtype=np.float32)
    if mult != 1.0:
        x = (x * np.float32(mult)).astype(np.float32)
    amax = np.abs(x).reshape(B * H, -1).max(axis=1).astype(np.float64)
    descale = np.maximum(amax / E4M3_MAX, 2.0 ** -100).astype(np.float32)
    ds = descale.astype(np.float64).reshape(B, H, 1, 1)
    codes = e4m3_codes(x.astype(np.float64) / ds)
    exact = e4m3_value(codes) * ds
    store = codes
    if transpose:
        ldv = -(-N // 16) * 16
        store = np.zeros((B, H, d, ldv), np.uint8)
        store[..., :N] = np.swapaxes(codes, 2, 3)
    return Tensor("fp8", store, exact), descale


def uniform_int(n, lo, hi, cfg_seed, tensor_id):
    """n integers uniform on [lo, hi] inclusive (int32)."""
    return rng(cfg_seed, tensor_id).integers(lo, hi + 1, size=n).astype(np.int32)


@dataclass
class Paged:
    """A paged KV cache plus block table: V [num_blocks, Hkv, block_size, d],
    K [num_blocks, Hkv, d/32, block_size, 32] (grouped, see paged_cache)."""
    k_cache: Tensor
    v_cache: Tensor
    block_table: np.ndarray   # int32 [B, max_blocks], -1 where unused
    seq_lens: np.ndarray      # int32 [B]
    block_size: int


def block_sparse_mask(H, N, band=2, stride=8):
    """Structured 128 x 128 block mask [H, nb, nb] (uint8): a local band
    |i - j| <= band plus every stride-th key block (global columns), the
    same for every head."""
    nb = -(-N // 128)
    i = np.arange(nb)[:, None]
    j = np.arange(nb)[None, :]
    m = (np.abs(i - j) <= band) | (j % stride == 0)
    return np.broadcast_to(m.astype(np.uint8), (H, nb, nb)).copy()


def paged_cache(seq_lens, Hkv, d, block_size, max_blocks, cfg_seed,
                poison_tails=True):
    """Random paged cache: every sequence's blocks are a slice of one random
    permutation of all physical blocks; slots past a sequence's length in its
    last block hold NaN when ``poison_tails`` (so a kernel that reads them
    into its arithmetic is caught), else ordinary N(0,1) values.

    V is stored [num_blocks, Hkv, block_size, d]; K in groups of 32 head-dim
    elements, [num_blocks, Hkv, d/32, block_size, 32] (element 32g + j of
    token u of a head's block at [.., g, u, j]), the library's K cache
    layout.  Both draw their values as [num_blocks, Hkv, block_size, d]
    arrays from their seeded streams, so the layout changes where a value
    sits, not the value."""
    if d % 32:
        raise ValueError("paged caches need d divisible by 32")
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    B = seq_lens.size
    nblk = [-(-int(L) // block_size) for L in seq_lens]
    total = max(1, sum(nblk))
    perm = rng(cfg_seed, TID_PERM).permutation(total).astype(np.int32)
    table = np.full((B, max_blocks), -1, dtype=np.int32)
    off = 0
    for b in range(B):
        table[b, :nblk[b]] = perm[off:off + nblk[b]]
        off += nblk[b]
    shape = (total, Hkv, block_size, d)
    kc = rng(cfg_seed, TID_KC).standard_normal(size=shape, dtype=np.float32)
    vc = rng(cfg_seed, TID_VC).standard_normal(size=shape, dtype=np.float32)
    if poison_tails:
        for b in range(B):
            L = int(seq_lens[b])
            if nblk[b] and L % block_size:
                last = table[b, nblk[b] - 1]
                kc[last, :, L % block_size:] = np.nan
                vc[last, :, L % block_size:] = np.nan
    kc = np.ascontiguousarray(
        kc.reshape(total, Hkv, block_size, d // 32, 32).transpose(0, 1, 3, 2, 4))
    kb, vb = bf16_bits(kc), bf16_bits(vc)
    return Paged(Tensor("bf16", kb, bf16_value(kb).astype(np.float64)),
                 Tensor("bf16", vb, bf16_value(vb).astype(np.float64)),
                 table, seq_lens, block_size)


@dataclass
class Workload:
    """One attention workload (a forward/backward problem or a decode batch)."""
    name: str
    seed: int
    kind: str                 # "attn" or "decode"
    dtype: str                # "bf16" or "f32"
    B: int
    H: int
    N: int
    d: int
    causal: bool = False
    qkv_mult: float = 1.0
    kv_len_range: Optional[tuple] = None   # (lo, hi) inclusive, key padding
    backward: bool = False
    # varlen only: sequence lengths ~ U{lo..hi}; N is the longest allowed
    seq_range: Optional[tuple] = None
    # dense only: dropout on P with this drop probability (seed = the
    # workload seed, offset 0)
    p_drop: float = 0.0
    # decode only
    Hkv: int = 0
    ctx_range: Optional[tuple] = None
    block_size: int = 16
    splits: int = 8
    notes: str = field(default="")

    def qkv(self):
        shape = (self.B, self.H, self.N, self.d)
        return tuple(normal(shape, self.seed, t, self.dtype, self.qkv_mult)
                     for t in (TID_Q, TID_K, TID_V))

    def fp8_inputs(self):
        """(q, k, v_t, q_descale, k_descale, v_descale) for an FP8 forward:
        Q and K [B,H,N,d] E4M3, V transposed [B,H,d,ldv] (see normal_fp8)."""
        shape = (self.B, self.H, self.N, self.d)
        q, qd = normal_fp8(shape, self.seed, TID_Q, self.qkv_mult)
        k, kd = normal_fp8(shape, self.seed, TID_K, self.qkv_mult)
        v, vd = normal_fp8(shape, self.seed, TID_V, self.qkv_mult,
                           transpose=True)
        return q, k, v, qd, kd, vd

    def dout(self):
        return normal((self.B, self.H, self.N, self.d), self.seed, TID_DO,
                      self.dtype)

    def kv_len(self):
        if self.kv_len_range is None:
            return None
        lo, hi = self.kv_len_range
        return uniform_int(self.B, lo, hi, self.seed, TID_LEN)

    def decode_inputs(self, poison_tails=True):
        lens = uniform_int(self.B, self.ctx_range[0], self.ctx_range[1],
                           self.seed, TID_LEN)
        max_blocks = -(-self.ctx_range[1] // self.block_size)
        cache = paged_cache(lens, self.Hkv, self.d, self.block_size,
                            max_blocks, self.seed, poison_tails)
        q = normal((self.B, self.H, self.d), self.seed, TID_Q, self.dtype)
        return q, cache

    def varlen_lens(self):
        lo, hi = self.seq_range
        return uniform_int(self.B, lo, hi, self.seed, TID_LEN)

    def varlen_inputs(self):
        """(cu_seqlens int32 [B+1], q, k, v [H, total, d]): the sequences
        packed back to back along the token axis, head-major."""
        lens = self.varlen_lens()
        cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        shape = (self.H, int(cu[-1]), self.d)
        q, k, v = (normal(shape, self.seed, t, self.dtype, self.qkv_mult)
                   for t in (TID_Q, TID_K, TID_V))
        return cu, q, k, v

    def varlen_dout(self):
        total = int(np.sum(self.varlen_lens()))
        return normal((self.H, total, self.d), self.seed, TID_DO, self.dtype)

    def prefill_inputs(self, poison_tails=True):
        """Chunked prefill against a paged cache: context lengths ~ U(ctx),
        new-token chunks ~ U(seq_range) (capped by the context); returns
        (cu_seqlens_q, q [Hq, total_q, d], cache) where the cache holds all
        seq_lens tokens, new ones included."""
        ctx = uniform_int(self.B, self.ctx_range[0], self.ctx_range[1],
                          self.seed, TID_LEN)
        qlen = np.minimum(uniform_int(self.B, self.seq_range[0],
                                      self.seq_range[1], self.seed, TID_PERM),
                          ctx)
        cu = np.concatenate([[0], np.cumsum(qlen)]).astype(np.int32)
        max_blocks = -(-self.ctx_range[1] // self.block_size)
        cache = paged_cache(ctx, self.Hkv, self.d, self.block_size,
                            max_blocks, self.seed, poison_tails)
        q = normal((self.H, int(cu[-1]), self.d), self.seed, TID_Q,
                   self.dtype)
        return cu, q, cache

    def prefill_flops(self):
        """4*Hq*d per (new token, visible cached key): new token i of a
        chunk of q tokens after c earlier ones sees c + i + 1 keys."""
        cu, _, cache = self.prefill_inputs(poison_tails=False)
        tot = 0.0
        for b in range(self.B):
            qn = int(cu[b + 1] - cu[b])
            L = int(cache.seq_lens[b])
            tot += qn * (L - qn) + qn * (qn + 1) / 2
        return 4.0 * self.H * self.d * tot

    def fwd_flops(self):
        """4*B*H*N^2*d, halved when causal (nominal N^2 under key padding);
        for a packed ragged batch the sum of 4*H*L^2*d over its sequences."""
        if self.kind == "varlen":
            sq = float(np.sum(np.asarray(self.varlen_lens(), np.float64) ** 2))
            f = 4.0 * self.H * sq * self.d
        elif self.kind == "sparse":   # computed (unmasked) blocks only
            mask = block_sparse_mask(self.H, self.N)
            rows = np.minimum(128, self.N - 128 * np.arange(mask.shape[1]))
            cnt = float(np.einsum("hij,i,j->", mask.astype(np.float64), rows,
                                  rows))
            f = 4.0 * self.B * cnt * self.d
        else:
            f = 4.0 * self.B * self.H * self.N * self.N * self.d
        return f / 2 if self.causal else f

    def bwd_flops(self):
        """Five N^2 d contractions: 2.5x the forward count."""
        return 2.5 * self.fwd_flops()


# The five workloads.  Shapes follow BERT-large / GPT-2-medium / long-context
# attention layers; the data are synthetic (no datasets or trained weights).
WORKLOADS = {
    "tiny_f32": Workload("tiny_f32", 1, "attn", "f32", 1, 1, 256, 64),
    "bert_large_padded": Workload(
        "bert_large_padded", 2, "attn", "bf16", 16, 16, 512, 64,
        kv_len_range=(256, 512), backward=True),
    "gpt2_medium_causal_1k": Workload(
        "gpt2_medium_causal_1k", 3, "attn", "bf16", 8, 16, 1024, 64,
        causal=True, qkv_mult=0.5, backward=True),
    "gpt2_medium_causal_4k": Workload(
        "gpt2_medium_causal_4k", 31, "attn", "bf16", 2, 16, 4096, 64,
        causal=True, qkv_mult=0.5, backward=True),
    # The 4K GPT-2-medium step with attention dropout 0.1 (GPT-2's training
    # setting for attention probabilities).
    "gpt2_medium_causal_4k_dropout": Workload(
        "gpt2_medium_causal_4k_dropout", 32, "attn", "bf16", 2, 16, 4096, 64,
        causal=True, qkv_mult=0.5, backward=True, p_drop=0.1),
    "long_causal_16k_d128": Workload(
        "long_causal_16k_d128", 4, "attn", "bf16", 1, 16, 16384, 128,
        causal=True),
    # A causal prefill batch packed without padding: 16 prompts of 64..4096
    # tokens, GPT-2-medium-shaped heads.
    "varlen_causal_prefill": Workload(
        "varlen_causal_prefill", 6, "varlen", "bf16", 16, 16, 4096, 64,
        causal=True, qkv_mult=0.5, backward=True, seq_range=(64, 4096)),
    # Chunked prefill in serving: 8 sequences with 1K-8K cached tokens each,
    # a new chunk of 256-1024 of them attending the whole prefix (GQA 4:1).
    "paged_chunked_prefill": Workload(
        "paged_chunked_prefill", 7, "prefill", "bf16", 8, 32, 1024, 128,
        causal=True, Hkv=8, ctx_range=(1024, 8192), seq_range=(256, 1024)),
    # Block-sparse attention at 16K: a 5-block local band plus every 8th key
    # block (about 16% of the blocks), non-causal.
    "block_sparse_16k": Workload(
        "block_sparse_16k", 8, "sparse", "bf16", 1, 16, 16384, 64,
        qkv_mult=0.5, backward=True),
    # FP8 (E4M3) forward on the 16K causal d = 128 shape, per-head scales.
    "long_causal_16k_d128_fp8": Workload(
        "long_causal_16k_d128_fp8", 9, "fp8", "fp8", 1, 16, 16384, 128,
        causal=True),
    "long_causal_64k_d64": Workload(
        "long_causal_64k_d64", 41, "attn", "bf16", 1, 2, 65536, 64,
        causal=True),
    "paged_gqa_decode": Workload(
        "paged_gqa_decode", 5, "decode", "bf16", 16, 32, 1, 128, Hkv=8,
        ctx_range=(1024, 8192), block_size=16, splits=8),
}
