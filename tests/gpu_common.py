"""Helpers for the GPU parity tests: the tolerance check and sampled-oracle
plumbing.  The oracle is only ever fed generator inputs, never HIP outputs."""
import numpy as np
import torch

import oracle

MAX_ABS = 5e-3   # parity bar for fp32 outputs against the fp64 oracle
REL_L2 = 1e-3


def parity(gpu: torch.Tensor, ref: np.ndarray, max_abs=MAX_ABS, rel_l2=REL_L2, what=""):
    g = gpu.detach().to(torch.float64).cpu().numpy()
    assert g.shape == ref.shape, (what, g.shape, ref.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    err = np.abs(g - ref)
    nref = np.linalg.norm(ref)
    rel = np.linalg.norm(g - ref) / nref if nref > 0 else np.linalg.norm(g - ref)
    print(f"[parity] {what}: max_abs={err.max():.3e} rel_l2={rel:.3e}", flush=True)
    assert err.max() <= max_abs, f"{what}: max-abs {err.max():.3e} > {max_abs}"
    assert rel <= rel_l2, f"{what}: rel-L2 {rel:.3e} > {rel_l2}"
    return err.max(), rel


def _bf16_rne(x):
    """fp64 values rounded to nearest even bf16 (through fp32, which is exact
    to within far less than a bf16 ulp here), returned as fp64."""
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).double().numpy()


def _bf16_ulp(x):
    """Spacing of bf16 values at |x| (8 significant bits; bf16's normal range
    starts at 2^-126)."""
    e = np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** -126)))
    return np.exp2(e - 7)


def bf16_parity(gpu_bf16: torch.Tensor, gpu_f32: torch.Tensor, ref: np.ndarray, what="",
                fp32_err=2e-6, min_within=0.999):
    """bf16 output, held to one bf16 ulp of the fp64 oracle rounded to nearest
    even (the reading for a bf16 output): bit-identical to the same kernel's
    fp32 output rounded to nearest even, and per element
    |out - RNE(ref)| <= ulp(RNE(ref)) + fp32_err, where fp32_err bounds the
    fp32 output's own error against the oracle (the rounding of an fp32 value
    and of the exact one can then differ by one ulp, and by more only where
    that error exceeds an ulp, i.e. for values of magnitude below about
    2^8 fp32_err).  fp32_err is that kernel's fp32 error level: 2e-6 for the
    fp32-FMA decode, 1e-3 where P rounds to fp16 (prefill, verify and the
    FP8 paths).  A share min_within of the elements must be within one ulp
    with no allowance at all: 99.9 % for the decode; for the fp16-P kernels,
    whose fp32 error exceeds an ulp on the smallest outputs, the share is
    given by the caller."""
    assert gpu_bf16.dtype == torch.bfloat16
    rounded = gpu_f32.to(torch.bfloat16)
    same = torch.equal(gpu_bf16.view(torch.int16), rounded.view(torch.int16))
    assert same, f"{what}: bf16 output differs from the rounded fp32 output"
    g = gpu_bf16.detach().to(torch.float64).cpu().numpy()
    assert np.all(np.isfinite(g))
    r16 = _bf16_rne(ref)
    ulp = _bf16_ulp(r16)
    err = np.abs(g - r16)
    excess = err - ulp
    within = float(np.mean(err <= ulp))
    print(f"[bf16] {what}: max(|out - RNE(ref)| - ulp)={excess.max():.3e} "
          f"within one ulp {100 * within:.4f} %", flush=True)
    assert excess.max() <= fp32_err, f"{what}: bf16 output beyond one ulp of RNE(oracle)"
    assert within >= min_within, f"{what}: only {100 * within:.3f} % within one ulp"


def compact_subset(batch, seqs):
    """Host copies of the blocks `seqs` use, with their block tables remapped
    onto a compact pool (the oracle is invariant to physical relabelling).
    Returns (k_pool, v_pool, block_table, context_lens, kept_rows_of_q)."""
    w = batch.workload
    bt = batch.block_table.cpu()
    ctx = batch.context_lens.cpu()
    rows = bt[seqs]
    used = torch.unique(rows[rows >= 0]).to(torch.int64)
    remap = torch.full((w.num_blocks,), -1, dtype=torch.int64)
    remap[used] = torch.arange(used.numel())
    nbt = torch.where(rows >= 0, remap[rows.clamp(min=0).to(torch.int64)], torch.tensor(-1))
    dev_used = used.to(batch.k_cache.device)
    k_sub = batch.k_cache.index_select(0, dev_used).cpu()
    v_sub = batch.v_cache.index_select(0, dev_used).cpu()
    return k_sub, v_sub, nbt.to(torch.int32), ctx[seqs]


def oracle_decode_sample(batch, seqs):
    """fp64 oracle for decode rows `seqs` of a (possibly huge) GPU batch."""
    k_sub, v_sub, bt, ctx = compact_subset(batch, seqs)
    q = batch.q.cpu()[seqs]
    return oracle.paged_attention(q, k_sub, v_sub, bt, ctx, batch.workload.scale)


def oracle_prefill_sample(batch, seqs, causal=True):
    """fp64 oracle for sequences `seqs` (all their query rows) of a batch."""
    k_sub, v_sub, bt, ctx = compact_subset(batch, seqs)
    cu = batch.cu_q_lens.cpu()
    q_all = batch.q.cpu()
    rows = torch.cat([torch.arange(int(cu[i]), int(cu[i + 1])) for i in seqs])
    lens = torch.tensor([int(cu[i + 1] - cu[i]) for i in seqs])
    ncu = torch.zeros(len(seqs) + 1, dtype=torch.int32)
    ncu[1:] = torch.cumsum(lens, 0)
    out = oracle.paged_attention(q_all[rows], k_sub, v_sub, bt, ctx, batch.workload.scale,
                                 cu_q_lens=ncu, causal=causal)
    return out, rows
