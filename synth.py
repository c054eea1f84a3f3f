"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module only draws random numbers and rounds them to the operand dtype;
it holds none of the arithmetic of the method and imports neither the oracle
nor the GPU binding, so both sides can take their inputs from here.

Recipe (every draw is float32 from a seeded torch.Generator, scaled in float32,
then rounded to bfloat16 with round-to-nearest-even when the operand is bf16):

* mm (fp32): generator(seed): W = randn(K, N), then the fixed request row
  mine = randn(1, K), then for each batch size M in the listed order the M-1
  distractor rows randn(M-1, K); the batch is cat(mine, distractors).  This is
  the draw order of the handbook's split-K experiment (K=4096, N=256, seed 0).
* every other workload: generator(seed) draws the shared operands first
  (weights, bias), then the fixed request (sample / row / slice 0); the
  distractors of batch size B come from generator(1000 + B), on the CPU for
  small batches or on the GPU (torch's device generator) for large ones.

Shapes and distributions follow the pages' workloads:
  addmm  X randn [M, 4096], W 0.02*randn [4096, 14336], bias 0.02*randn [14336]
  conv   x 2*rand-1 [B, 3, 224, 224], w 0.02*randn [1152, 3, 14, 14],
         bias 0.02*randn [1152]
  attn   Q, K, V randn [B, 8, 1024, 128] flattened to [8B, 1024, 128]
  decode q randn [B, 32, 64], K, V randn [B, 32, 8192, 64]
  paged prefill: q randn [total_q, H, D] (request b's rows cu_q[b] .. cu_q[b+1]-1,
         the first at position prefix_b), then the K and V caches as for paged
         decode holding each request's prefix_b + q_len_b tokens.
  paged decode: the same q, K, V draws per request; each request's tokens are
         stored in pages of P tokens of a cache [num_pages, H, P, D], pages
         handed out in a seeded random permutation (so a request's pages are
         scattered), block_table [B, max_pages] int32 (unused entries -1),
         seq_lens [B] int32.
"""
import torch

BF16 = torch.bfloat16


def _gen(seed, device="cpu"):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _randn(shape, g, device="cpu", scale=None):
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if scale is not None:
        t.mul_(scale)
    return t


def _uniform_pm1(shape, g, device="cpu"):
    t = torch.rand(shape, generator=g, device=device, dtype=torch.float32)
    return t.mul_(2.0).sub_(1.0)


# ----------------------------------------------------------------- mm (fp32)
def mm_inputs(Ms=(1, 8, 63, 64, 200), K=4096, N=256, seed=0):
    """Returns W [K, N] and {M: X [M, K]} with X[M][0] the same row for all M."""
    g = _gen(seed)
    W = _randn((K, N), g)
    mine = _randn((1, K), g)
    X = {}
    for M in Ms:
        X[M] = torch.cat([mine, _randn((M - 1, K), g)]) if M > 1 else mine.clone()
    return W, X


# ------------------------------------------------------------------- addmm
def addmm_shared(K=4096, N=14336, seed=0, dtype=BF16):
    g = _gen(seed)
    W = _randn((K, N), g, scale=0.02).to(dtype)
    bias = _randn((N,), g, scale=0.02).to(dtype)
    x0 = _randn((1, K), g).to(dtype)
    return W, bias, x0


def addmm_batch(x0, M, device="cpu", dtype=BF16):
    """[M, K] batch whose row 0 is x0; distractors from generator(1000 + M)."""
    K = x0.shape[1]
    x0 = x0.to(device)
    if M == 1:
        return x0.clone()
    g = _gen(1000 + M, device)
    rest = _randn((M - 1, K), g, device=device).to(dtype)
    return torch.cat([x0, rest])


# -------------------------------------------------------------------- conv
def conv_shared(Cout=1152, Cin=3, Kh=14, Kw=14, H=224, W=224, seed=0, dtype=BF16):
    g = _gen(seed)
    w = _randn((Cout, Cin, Kh, Kw), g, scale=0.02).to(dtype)
    bias = _randn((Cout,), g, scale=0.02).to(dtype)
    x0 = _uniform_pm1((1, Cin, H, W), g).to(dtype)
    return w, bias, x0


def conv_batch(x0, B, device="cpu", dtype=BF16):
    x0 = x0.to(device)
    if B == 1:
        return x0.clone()
    g = _gen(1000 + B, device)
    rest = _uniform_pm1((B - 1,) + tuple(x0.shape[1:]), g, device=device).to(dtype)
    return torch.cat([x0, rest])


# --------------------------------------------------------------- attention
def attn_shared(H=8, T=1024, D=128, seed=0, dtype=BF16):
    """Q, K, V of batch element b = 0: each [1, H, T, D]."""
    g = _gen(seed)
    return tuple(_randn((1, H, T, D), g).to(dtype) for _ in range(3))


def attn_batch(qkv0, B, device="cpu", dtype=BF16):
    """Flattened [B*H, T, D] Q, K, V whose first H slices are batch element 0."""
    out = []
    g = _gen(1000 + B, device) if B > 1 else None
    for t0 in qkv0:
        t0 = t0.to(device)
        if B > 1:
            t = torch.cat([t0, _randn((B - 1,) + tuple(t0.shape[1:]), g, device=device).to(dtype)])
        else:
            t = t0.clone()
        out.append(t.reshape(-1, t0.shape[2], t0.shape[3]))
    return tuple(out)


# ------------------------------------------------------------------ decode
def decode_shared(H=32, S=8192, D=64, seed=0, dtype=BF16):
    """q [1, H, D], K and V [1, H, S, D] of request 0."""
    g = _gen(seed)
    q = _randn((1, H, D), g).to(dtype)
    k = _randn((1, H, S, D), g).to(dtype)
    v = _randn((1, H, S, D), g).to(dtype)
    return q, k, v


def decode_batch(qkv0, B, device="cpu", dtype=BF16, block=16):
    """[B, ...] q, K, V whose request 0 is qkv0; distractors from generator(1000 + B),
    drawn `block` requests at a time to bound the float32 staging memory."""
    q0, k0, v0 = (t.to(device) for t in qkv0)
    if B == 1:
        return q0.clone(), k0.clone(), v0.clone()
    g = _gen(1000 + B, device)
    H, S, D = k0.shape[1], k0.shape[2], k0.shape[3]
    q = torch.empty((B, H, D), dtype=dtype, device=device)
    k = torch.empty((B, H, S, D), dtype=dtype, device=device)
    v = torch.empty((B, H, S, D), dtype=dtype, device=device)
    q[0], k[0], v[0] = q0[0], k0[0], v0[0]
    q[1:] = _randn((B - 1, H, D), g, device=device).to(dtype)
    for b0 in range(1, B, block):
        b1 = min(B, b0 + block)
        k[b0:b1] = _randn((b1 - b0, H, S, D), g, device=device).to(dtype)
        v[b0:b1] = _randn((b1 - b0, H, S, D), g, device=device).to(dtype)
    return q, k, v


# ----------------------------------------------------------------- helpers
def randn(shape, seed, dtype=torch.float32, scale=None, device="cpu"):
    """Generic seeded draw for parity cases of arbitrary shape."""
    return _randn(shape, _gen(seed, device), device=device, scale=scale).to(dtype)


def randint(shape, lo, hi, seed, dtype=torch.float32):
    """Small integers in [lo, hi], exact in bfloat16 and float32."""
    g = _gen(seed)
    return torch.randint(lo, hi + 1, shape, generator=g).to(dtype)


def uniform(shape, seed, lo=0.0, hi=1.0, dtype=torch.float32):
    g = _gen(seed)
    t = torch.rand(shape, generator=g, dtype=torch.float32)
    return (t * (hi - lo) + lo).to(dtype)


def paged_decode_inputs(seq_lens, H=32, D=64, P=16, seed=0, device="cpu", dtype=BF16, spare_pages=7,
                        with_seq=True, block_pages=2048):
    """q [B, H, D]; k_cache, v_cache [num_pages, H, P, D]; block_table [B, max_pages]
    int32; seq_lens [B] int32; and, if with_seq, the contiguous K, V of each
    request (lists of [H, S_b, D] views) holding the same values.  Page ids are a
    seeded random permutation of 0 .. num_pages-1 (spare pages stay random).
    Drawn on `device`, `block_pages` pages at a time (bounded float32 staging)."""
    B = len(seq_lens)
    g = _gen(seed, device)
    npg = [(int(s) + P - 1) // P for s in seq_lens]
    max_pages = max(max(npg), 1)
    num_pages = sum(npg) + spare_pages
    q = _randn((B, H, D), g, device=device).to(dtype)
    k_cache = torch.empty((num_pages, H, P, D), dtype=dtype, device=device)
    v_cache = torch.empty((num_pages, H, P, D), dtype=dtype, device=device)
    for cache in (k_cache, v_cache):
        for p0 in range(0, num_pages, block_pages):
            p1 = min(num_pages, p0 + block_pages)
            cache[p0:p1] = _randn((p1 - p0, H, P, D), g, device=device).to(dtype)
    perm = torch.randperm(num_pages, generator=g, device=device)
    bt = torch.full((B, max_pages), -1, dtype=torch.int32, device=device)
    k_seq, v_seq = [], []
    used = 0
    for b in range(B):
        pages = perm[used:used + npg[b]]
        used += npg[b]
        bt[b, :npg[b]] = pages.to(torch.int32)
        if with_seq:
            S = int(seq_lens[b])
            k_seq.append(k_cache[pages].permute(1, 0, 2, 3).reshape(H, -1, D)[:, :S])
            v_seq.append(v_cache[pages].permute(1, 0, 2, 3).reshape(H, -1, D)[:, :S])
    sl = torch.tensor([int(s) for s in seq_lens], dtype=torch.int32, device=device)
    return q, k_cache, v_cache, bt, sl, k_seq, v_seq


def request_kv(k_cache, v_cache, block_table, seq_lens, b):
    """The contiguous K, V [1, H, S_b, D] of request b of a paged cache (a gather)."""
    S = int(seq_lens[b])
    P = k_cache.shape[2]
    pages = block_table[b, :(S + P - 1) // P].long()
    H, D = k_cache.shape[1], k_cache.shape[3]
    k = k_cache[pages].permute(1, 0, 2, 3).reshape(H, -1, D)[:, :S]
    v = v_cache[pages].permute(1, 0, 2, 3).reshape(H, -1, D)[:, :S]
    return k[None].contiguous(), v[None].contiguous()


def paged_prefill_inputs(prefix_lens, q_lens, H=8, D=128, P=16, seed=0, device="cpu", dtype=BF16,
                         spare_pages=5, block_pages=2048):
    """Chunked-prefill inputs: q [total_q, H, D]; cu_q [B+1] int32; q_pos0 [B] int32
    (= prefix_lens); k_cache, v_cache [num_pages, H, P, D] holding each request's
    prefix_b + q_len_b tokens; block_table [B, max_pages] int32 (pages a seeded
    permutation, unused entries -1)."""
    B = len(q_lens)
    g = _gen(seed, device)
    kv = [int(a) + int(n) for a, n in zip(prefix_lens, q_lens)]
    cu = [0]
    for n in q_lens:
        cu.append(cu[-1] + int(n))
    q = _randn((cu[-1], H, D), g, device=device).to(dtype)
    npg = [(n + P - 1) // P for n in kv]
    max_pages = max(max(npg), 1)
    num_pages = sum(npg) + spare_pages
    k_cache = torch.empty((num_pages, H, P, D), dtype=dtype, device=device)
    v_cache = torch.empty((num_pages, H, P, D), dtype=dtype, device=device)
    for cache in (k_cache, v_cache):
        for p0 in range(0, num_pages, block_pages):
            p1 = min(num_pages, p0 + block_pages)
            cache[p0:p1] = _randn((p1 - p0, H, P, D), g, device=device).to(dtype)
    perm = torch.randperm(num_pages, generator=g, device=device)
    bt = torch.full((B, max_pages), -1, dtype=torch.int32, device=device)
    used = 0
    for b in range(B):
        bt[b, :npg[b]] = perm[used:used + npg[b]].to(torch.int32)
        used += npg[b]
    cu_q = torch.tensor(cu, dtype=torch.int32, device=device)
    q_pos0 = torch.tensor([int(a) for a in prefix_lens], dtype=torch.int32, device=device)
    return q, cu_q, q_pos0, k_cache, v_cache, bt
