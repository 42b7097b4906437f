"""Seeded synthetic inputs for the grouped MoE backward GEMMs.

This module only draws inputs (random values, group sizes, MXFP8 encodings of
random values).  It holds none of the method's arithmetic, and both the CPU
oracle and the HIP path take their inputs from it.

Shapes and distributions follow the workloads the library is measured on
(tokens grouped in multiples of 256, as the pages require of offsets and
padded_offsets):

  wgrad_small   hidden 256, inter 256, 4 experts, counts [256, 0, 512, 256]
  dswiglu       L 8, K 2048, N 1024, M 16384 (multinomial groups)
  wgrad_moe     hidden 4096, inter 2048, 64 experts, 65536 tokens, Zipf(1.2)
  dgeglu        L 32, K 4096, N 1536, M 32768, discrete B, dbias
  dsrelu_mxfp8  L 16, K 7168, N 2048, M 65536, MXFP8 A and B
  dglu_mxfp8    L 32, K 4096, N 1536, M 32768, MXFP8 A and discrete B,
                dSwiGLU with amax (the dGeGLU workload's shape on the
                block-scaled path)
  wgrad_mxfp8   the wgrad_moe shape (hidden 4096, inter 2048, 64 experts,
                65536 Zipf(1.2) tokens) on MXFP8 K-major operands

Every generator takes a seed and a torch device; tensors are created on that
device from a torch.Generator seeded with it, so a run that needs the same
inputs on the CPU (for the oracle) copies them from wherever they were drawn.
"""
import math

import numpy as np
import torch

BLOCK = 256  # group granularity required of offsets / padded_offsets


# --------------------------------------------------------------------------
# group sizes
# --------------------------------------------------------------------------

def multinomial_groups(total_rows, groups, seed, block=BLOCK):
    """Group sizes in multiples of `block` summing to total_rows: the
    total_rows/block blocks are dealt to the groups by a seeded multinomial
    draw with equal probabilities (empty groups can occur)."""
    assert total_rows % block == 0
    rng = np.random.default_rng(seed)
    counts = rng.multinomial(total_rows // block, [1.0 / groups] * groups)
    return (counts * block).astype(np.int64)


def zipf_groups(total_rows, groups, s, seed, block=BLOCK):
    """Zipf(s)-skewed group sizes in multiples of `block`: weights (r+1)^-s
    over ranks r < groups, total_rows/block blocks apportioned by largest
    remainder (ties to the lower rank), then a seeded permutation of the
    groups."""
    nb = total_rows // block
    w = np.array([(r + 1.0) ** -s for r in range(groups)])
    quota = w / w.sum() * nb
    base = np.floor(quota).astype(np.int64)
    rem = quota - base
    order = sorted(range(groups), key=lambda r: (-rem[r], r))
    for r in order[: nb - int(base.sum())]:
        base[r] += 1
    perm = np.random.default_rng(seed).permutation(groups)
    counts = np.empty(groups, np.int64)
    counts[perm] = base
    return counts * block


def cumulative(counts):
    """int32 cumulative ends of consecutive groups (the offsets array)."""
    return np.cumsum(np.asarray(counts, np.int64)).astype(np.int32)


# --------------------------------------------------------------------------
# value draws
# --------------------------------------------------------------------------

def _gen(seed, device):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def normal(shape, std, gen, device, dtype=torch.bfloat16):
    """N(0, std) drawn in fp32, then cast (round to nearest even) to dtype."""
    x = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x.to(dtype)


def uniform(shape, lo, hi, gen, device):
    x = torch.rand(shape, generator=gen, device=device, dtype=torch.float32)
    return x.mul_(hi - lo).add_(lo)


def small_ints(shape, lo, hi, gen, device, dtype=torch.bfloat16):
    """Integers in [lo, hi] (exactly representable in bf16)."""
    return torch.randint(lo, hi + 1, shape, generator=gen, device=device).to(dtype)


FP8_MAX = {torch.float8_e4m3fn: 448.0, torch.float8_e5m2: 57344.0}


def mx_encode(x, block=32, fmt=torch.float8_e4m3fn):
    """OCP MXFP8 encoding of an fp32 matrix (rows, K): one E8M0 scale per
    `block` consecutive K values of each row and FP8 codes (E4M3, or E5M2
    with fmt=torch.float8_e5m2).  The scale exponent is
    e = ceil(log2(amax / max)) over the block, max the format's largest
    value (so no code saturates), the stored byte is e + 127, and each code
    is the FP8 value nearest to x / 2^e (torch's cast, ties to even).  An
    all-zero block takes e = -127 (byte 0).  Returns (codes as fmt, scales
    as torch.uint8)."""
    rows, K = x.shape
    assert K % block == 0
    xb = x.reshape(rows, K // block, block)
    amax = xb.abs().amax(dim=2)
    e = torch.ceil(torch.log2(amax / FP8_MAX[fmt]))
    e = torch.where(amax > 0, e, torch.full_like(e, -127.0)).clamp_(-127, 127)
    q = (xb / torch.exp2(e).unsqueeze(2)).to(fmt)
    return q.reshape(rows, K), (e + 127).to(torch.uint8)


# --------------------------------------------------------------------------
# workloads
# --------------------------------------------------------------------------

def wgrad_inputs(hidden, inter, counts, a_major="k", b_major="n", seed=0,
                 device="cpu", ints=False):
    """Inputs of the grouped wgrad.

    A is the logical (hidden, T) matrix and B the logical (T, inter) one,
    both N(0,1) in bf16 (or small integers in [-2, 2] with ints=True).
    Storage: A K-major is a (hidden, T) row-major tensor, A M-major a
    (T, hidden) row-major tensor; B N-major a (T, inter) row-major tensor,
    B K-major an (inter, T) row-major tensor.  Returns a dict with the stored
    tensors `a`, `b`, the offsets (int32) and the sizes."""
    counts = np.asarray(counts, np.int64)
    T = int(counts.sum())
    g = _gen(seed, device)
    draw = (lambda s: small_ints(s, -2, 2, g, device)) if ints else \
        (lambda s: normal(s, 1.0, g, device))
    a = draw((hidden, T) if a_major == "k" else (T, hidden))
    b = draw((T, inter) if b_major == "n" else (inter, T))
    return dict(a=a.contiguous(), b=b.contiguous(), a_major=a_major, b_major=b_major,
                offsets=torch.from_numpy(cumulative(counts)).to(device),
                counts=counts, hidden=hidden, inter=inter, tokens_sum=T)


def wgrad_mx_inputs(hidden, inter, counts, seed=0, device="cpu", scale_spread=0, ints=False,
                    ab_dtype=torch.float8_e4m3fn):
    """Inputs of the block-scaled (MXFP8) grouped wgrad.

    A is the logical (hidden, T) matrix, stored K-major; B the logical
    (T, inter) matrix, stored K-major as an (inter, T) array.  Both are N(0,1)
    values (integers in [-2, 2] with ints=True) MXFP8-encoded along T by
    mx_encode (one E8M0 scale per 32 tokens of a row); scale_spread > 0
    multiplies each row by 2^j, j uniform in [-scale_spread, scale_spread],
    before encoding.  Returns the codes `a` (hidden, T), `b` (inter, T), the
    scales `sfa` (hidden, T/32), `sfb` (inter, T/32), the offsets and sizes."""
    counts = np.asarray(counts, np.int64)
    T = int(counts.sum())
    g = _gen(seed, device)

    def draw(rows):
        if ints:
            x = torch.randint(-2, 3, (rows, T), generator=g, device=device).float()
        else:
            x = torch.randn((rows, T), generator=g, device=device, dtype=torch.float32)
        if scale_spread:
            j = torch.randint(-scale_spread, scale_spread + 1, (rows, 1), generator=g,
                              device=device).float()
            x = x * torch.exp2(j)
        return mx_encode(x, fmt=ab_dtype)

    a, sfa = draw(hidden)
    b, sfb = draw(inter)
    return dict(a=a, sfa=sfa, b=b, sfb=sfb,
                offsets=torch.from_numpy(cumulative(counts)).to(device),
                counts=counts, hidden=hidden, inter=inter, tokens_sum=T)


def to_ragged(x, counts, per=1):
    """The "tensor_ragged" storage of a K-major (rows, K) tensor whose K axis
    is split into consecutive per-expert slices of counts[e] // per columns:
    the per-expert (rows, count) blocks, each K-contiguous, concatenated in
    expert order (a flat tensor).  Pure data movement: per = 32 relays out a
    scale array whose columns cover 32 tokens each."""
    cols = [int(c) // per for c in counts]
    parts, start = [], 0
    for c in cols:
        parts.append(x[:, start:start + c].reshape(-1))
        start += c
    assert start == x.shape[1]
    return torch.cat(parts) if parts else x.reshape(-1)[:0]


def wgrad_initial(num_experts, hidden, inter, dtype, seed, device="cpu"):
    """Initial outputs for accumulate mode: N(0,1) in the output dtype."""
    g = _gen(seed, device)
    return normal((num_experts, hidden, inter), 1.0, g, device, dtype)


def dglu_inputs(L, K, N, counts, a_std=0.02, b_std=0.02, c_std=2.0,
                c_dtype=torch.bfloat16, m_extra=0, seed=0, device="cpu",
                discrete=False, b_major="k", ints=False):
    """Inputs of the grouped dgrad + dGLU.

    A (M, K) bf16 K-major, B per expert (N, K) (dense: one (L, N, K) tensor,
    i.e. the (N, K, L) layout with strides (K, 1, N*K); discrete: L separate
    tensors), C (M, 2N) N(0, c_std), prob U(0,1), alpha and beta U(0.5,1.5).
    M = sum(counts) + m_extra (rows past the last group are never touched).
    b_major "n" stores each expert's B as a (K, N) row-major tensor."""
    counts = np.asarray(counts, np.int64)
    valid_m = int(counts.sum())
    M = valid_m + m_extra
    g = _gen(seed, device)
    if ints:
        a = small_ints((M, K), -2, 2, g, device)
        bshape = (N, K) if b_major == "k" else (K, N)
        bl = [small_ints(bshape, -2, 2, g, device) for _ in range(L)]
    else:
        a = normal((M, K), a_std, g, device)
        bshape = (N, K) if b_major == "k" else (K, N)
        bl = [normal(bshape, b_std, g, device) for _ in range(L)]
    b_dense = None
    if not discrete:
        assert b_major == "k"
        b_dense = torch.stack(bl).contiguous()
        bl = [b_dense[i] for i in range(L)]
    c = normal((M, 2 * N), c_std, g, device, c_dtype)
    prob = uniform((M,), 0.0, 1.0, g, device)
    alpha = uniform((L,), 0.5, 1.5, g, device)
    beta = uniform((L,), 0.5, 1.5, g, device)
    return dict(a=a, b_dense=b_dense, b_list=bl, b_major=b_major, c=c, prob=prob,
                alpha=alpha, beta=beta,
                padded_offsets=torch.from_numpy(cumulative(counts)).to(device),
                counts=counts, L=L, K=K, N=N, M=M, valid_m=valid_m)


def dsrelu_inputs(L, K, N, counts, c_dtype=torch.bfloat16, m_extra=0, seed=0,
                  device="cpu", discrete=False, scale_spread=0, ab_dtype=torch.float8_e4m3fn):
    """Inputs of the grouped block-scaled dgrad + dsReLU.

    A (M, K) and B (N, K) per expert are N(0,1) values MXFP8-encoded by
    mx_encode (E4M3 codes, one E8M0 scale per 32 K values of each row);
    scale_spread > 0 additionally multiplies each row by 2^j for j drawn
    uniformly from [-scale_spread, scale_spread], so the scales vary.
    C (M, N) N(0,1), prob U(0,1), alpha U(0.5,1.5)."""
    counts = np.asarray(counts, np.int64)
    valid_m = int(counts.sum())
    M = valid_m + m_extra
    g = _gen(seed, device)

    def draw(rows):
        x = torch.randn((rows, K), generator=g, device=device, dtype=torch.float32)
        if scale_spread:
            j = torch.randint(-scale_spread, scale_spread + 1, (rows, 1), generator=g,
                              device=device).float()
            x = x * torch.exp2(j)
        return mx_encode(x, fmt=ab_dtype)

    a, sfa = draw(M)
    bl, sl = [], []
    for _ in range(L):
        q, s = draw(N)
        bl.append(q)
        sl.append(s)
    b_dense = sfb_dense = None
    if not discrete:
        b_dense = torch.stack(bl).contiguous()
        sfb_dense = torch.stack(sl).contiguous()
        bl = [b_dense[i] for i in range(L)]
        sl = [sfb_dense[i] for i in range(L)]
    c = normal((M, N), 1.0, g, device, c_dtype)
    prob = uniform((M,), 0.0, 1.0, g, device)
    alpha = uniform((L,), 0.5, 1.5, g, device)
    return dict(a=a, sfa=sfa, b_dense=b_dense, sfb_dense=sfb_dense, b_list=bl,
                sfb_list=sl, c=c, prob=prob, alpha=alpha,
                padded_offsets=torch.from_numpy(cumulative(counts)).to(device),
                counts=counts, L=L, K=K, N=N, M=M, valid_m=valid_m)



def dglu_mx_inputs(L, K, N, counts, c_std=2.0, c_dtype=torch.bfloat16, m_extra=0,
                   seed=0, device="cpu", discrete=True, scale_spread=0, ints=False,
                   ab_dtype=torch.float8_e4m3fn):
    """Inputs of the grouped block-scaled dgrad + dGLU.

    A (M, K) and B (N, K) per expert are N(0,1) values (integers in [-2, 2]
    with ints=True, which E4M3 and bf16 both hold exactly) MXFP8-encoded by
    mx_encode; scale_spread > 0 multiplies each row by 2^j, j uniform in
    [-scale_spread, scale_spread], before encoding.  C (M, 2N) N(0, c_std),
    prob U(0,1), alpha and beta U(0.5,1.5)."""
    counts = np.asarray(counts, np.int64)
    valid_m = int(counts.sum())
    M = valid_m + m_extra
    g = _gen(seed, device)

    def draw(rows):
        if ints:
            x = torch.randint(-2, 3, (rows, K), generator=g, device=device).float()
        else:
            x = torch.randn((rows, K), generator=g, device=device, dtype=torch.float32)
        if scale_spread:
            j = torch.randint(-scale_spread, scale_spread + 1, (rows, 1), generator=g,
                              device=device).float()
            x = x * torch.exp2(j)
        return mx_encode(x, fmt=ab_dtype)

    a, sfa = draw(M)
    bl, sl = [], []
    for _ in range(L):
        q, s = draw(N)
        bl.append(q)
        sl.append(s)
    b_dense = sfb_dense = None
    if not discrete:
        b_dense = torch.stack(bl).contiguous()
        sfb_dense = torch.stack(sl).contiguous()
        bl = [b_dense[i] for i in range(L)]
        sl = [sfb_dense[i] for i in range(L)]
    c = normal((M, 2 * N), c_std, g, device, c_dtype)
    prob = uniform((M,), 0.0, 1.0, g, device)
    alpha = uniform((L,), 0.5, 1.5, g, device)
    beta = uniform((L,), 0.5, 1.5, g, device)
    return dict(a=a, sfa=sfa, b_dense=b_dense, sfb_dense=sfb_dense, b_list=bl,
                sfb_list=sl, c=c, prob=prob, alpha=alpha, beta=beta,
                padded_offsets=torch.from_numpy(cumulative(counts)).to(device),
                counts=counts, L=L, K=K, N=N, M=M, valid_m=valid_m)

# The named workloads (sizes and recipes; seeds 1000 + index).
WORKLOADS = {
    "wgrad_small": dict(kind="wgrad", hidden=256, inter=256,
                        counts=[256, 0, 512, 256], a_major="k", b_major="n", seed=1001),
    "dswiglu": dict(kind="dglu", act="dswiglu", L=8, K=2048, N=1024, M=16384,
                    c_std=2.0, discrete=False, dbias=False, seed=1002),
    "wgrad_moe": dict(kind="wgrad", hidden=4096, inter=2048, E=64, T=65536,
                      zipf=1.2, b_major="n", seed=1003),
    "dgeglu": dict(kind="dglu", act="dgeglu", L=32, K=4096, N=1536, M=32768,
                   c_std=4.0, discrete=True, dbias=True, seed=1004),
    "dsrelu_mxfp8": dict(kind="dsrelu", L=16, K=7168, N=2048, M=65536, seed=1005),
    "dglu_mxfp8": dict(kind="dglu_mx", act="dswiglu", L=32, K=4096, N=1536, M=32768,
                       c_std=2.0, discrete=True, dbias=False, seed=1006),
    "wgrad_mxfp8": dict(kind="wgrad_mx", hidden=4096, inter=2048, E=64, T=65536, zipf=1.2,
                        seed=1007),
}


def workload_counts(name):
    w = WORKLOADS[name]
    if w["kind"] in ("wgrad", "wgrad_mx"):
        if "counts" in w:
            return np.asarray(w["counts"], np.int64)
        return zipf_groups(w["T"], w["E"], w["zipf"], w["seed"])
    return multinomial_groups(w["M"], w["L"], w["seed"])


def bits(t):
    """numpy bit patterns of a CPU tensor (uint16 for 16-bit floats, uint8
    for 8-bit ones, the plain array otherwise)."""
    t = t.detach().cpu().contiguous()
    if t.dtype in (torch.bfloat16, torch.float16):
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype in (torch.float8_e4m3fn, torch.float8_e5m2):
        return t.view(torch.uint8).numpy()
    return t.numpy()


def flops_wgrad(hidden, inter, counts):
    return 2.0 * hidden * inter * float(np.sum(counts))


def flops_dgrad(valid_m, N, K):
    return 2.0 * valid_m * N * K


def ceil_div(a, b):
    return -(-a // b)


__all__ = [n for n in dir() if not n.startswith("_") and n not in ("math", "np", "torch")]
