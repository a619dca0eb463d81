"""GPU parity of the paged entry pools and the token ring ("DeepSeek-V4 深度分析报告" section
3.5: the Classical KV Cache holds compressed entries in blocks of lcm(m, m') = 128 tokens,
the State Cache of fixed size the window rows and the uncompressed tail).

Each case runs one batch twice through the C ABI: with contiguous pools, and with the same
rows scattered into paged pools (32 CSA entries or 1 HCA entry per 128-token block, blocks
placed by a random permutation among garbage rows) and a 256-row token ring per sequence.
Outputs (entries written, scores, idx, out, lse) must be bit-identical, the new entries
must land at their block-table rows, and no other physical row may change.  One case is
also checked against the oracle reading the logical rows through the same table."""

import math

import numpy as np
import pytest
import torch

from long_context_attention_07_amd import configs, ops, synth
from oracle.attention import attend_token
from oracle.indexer import index_scores, topk_select, visible

from harness import DEV, assert_close, check_topk, log

pytestmark = pytest.mark.gpu

RING = 256
BLOCK_TOKENS = 128


@pytest.fixture(autouse=True)
def _needs_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ops.lib()


class Paged:
    """Physical pools of one layer: entry rows through a block table, token rows in rings."""

    def __init__(self, g, x, ratio, n_q, ring=RING):
        self.epb = BLOCK_TOKENS // ratio
        self.R = ring
        E, lens, n = x["E"], x["lens"], len(x["lens"])
        nblk = [max(1, -(-e // self.epb)) for e in E]
        total = sum(nblk) + 7
        perm = [int(v) for v in g.permutation(total)]
        self.table, o = [], 0
        for nb in nblk:
            self.table.append(perm[o:o + nb])
            o += nb
        # logical entry i of sequence b -> physical row
        self.erow = []
        for b in range(n):
            t = self.table[b]
            self.erow.append(torch.tensor([t[i // self.epb] * self.epb + i % self.epb for i in range(E[b])],
                                          dtype=torch.long, device=DEV))
        self.n_rows = total * self.epb
        self.x, self.lens, self.n_q = x, lens, n_q

    def entries(self, pool, garbage_seed):
        """Physical copy of a contiguous entry pool [sum E, ...] (garbage elsewhere)."""
        gen = torch.Generator(device=DEV)
        gen.manual_seed(garbage_seed)
        phys = torch.randint(0, 255, (self.n_rows,) + tuple(pool.shape[1:]), generator=gen, device=DEV,
                             dtype=torch.uint8 if pool.dtype == torch.uint8 else torch.int16)
        phys = phys.to(torch.uint8) if pool.dtype == torch.uint8 else phys.view(pool.dtype)
        phys = phys.contiguous()
        for b in range(len(self.lens)):
            e0 = self.x["entry_off"][b]
            phys[self.erow[b]] = pool[e0:e0 + self.x["E"][b]]
        return phys

    def ring(self, pool, garbage_seed):
        """Token rings [n_seqs * RING, ...] holding each sequence's positions tok_lo .. L-1."""
        gen = torch.Generator(device=DEV)
        gen.manual_seed(garbage_seed)
        R = self.R
        ring = torch.randn((len(self.lens) * R,) + tuple(pool.shape[1:]), generator=gen, device=DEV).to(pool.dtype)
        for b, L in enumerate(self.lens):
            lo, t0 = self.x["tok_lo"][b], self.x["tok_off"][b]
            assert L - lo <= R
            pos = torch.arange(lo, L, device=DEV)
            ring[b * R + pos % R] = pool[t0:t0 + (L - lo)]
        return ring

    def seqs(self, block_entries=None):
        n = len(self.lens)
        return ops.Seqs(self.n_q, self.lens, [0] * n, [b * self.R for b in range(n)], self.x["tok_lo"],
                        block_table=self.table, block_entries=block_entries or self.epb, tok_ring=self.R)


def _csa_run(sq, kv, c, z, kI, cI, zI, qI, q, x, wl, k):
    ops.csa_compress2(sq, wl.ratio, wl.overlap, wl.rope_theta, (c, z, x["bias"], wl.rope_dims, kv),
                      (cI, zI, x["biasI"], 0, kI))
    n_tok = sq.total_q
    idx = torch.full((n_tok, k), -7, dtype=torch.int32, device=DEV)
    ws = torch.empty(ops.csa_workspace_bytes(ops.OP_INDEX_TOPK, sq, k=k, ratio=wl.ratio) // 4 + 1, device=DEV)
    ops.csa_index_topk(sq, qI, x["w"], wl.n_I, kI, wl.ratio, k, idx, ws=ws)
    out = ops.Rows.of(torch.empty((n_tok * wl.n_h, wl.d_c), dtype=torch.bfloat16, device=DEV))
    lse = torch.empty((n_tok, wl.n_h), dtype=torch.float32, device=DEV)
    wsa_b = ops.csa_workspace_bytes(ops.OP_CSA_ATTEND, sq, wl.n_h, wl.d_c, k, wl.ratio, wl.n_win)
    wsa = torch.empty(wsa_b // 4 + 1, device=DEV) if wsa_b else None
    ops.csa_attend(sq, q, wl.n_h, kv, idx, k, c, wl.n_win, x["sink"], 1.0 / math.sqrt(wl.d_c), wl.rope_dims,
                   wl.rope_theta, out, lse, ws=wsa)
    return idx, out.data, lse


@pytest.mark.parametrize("k,n_q_hi", [(512, 1), (1024, 24)])
def test_paged_csa_equals_contiguous(k, n_q_hi):
    """CSA layer (bf16 rows, bf16 indexer): decode (one new token, the pair attention kernel,
    k = 512) and multi-token steps (up to 24 new tokens, the 64-head kernel, k = 1024)."""
    import dataclasses
    wl = dataclasses.replace(configs.CSA_DECODE_BF16, k=k)
    g = synth.rng(70 + k)
    n = 12
    lens = [int(v) for v in synth.log_uniform_ints(g, n, 3000, 200000)]
    n_q = [int(v) for v in g.integers(1, n_q_hi + 1, size=n)]
    lens = [max(L, q) for L, q in zip(lens, n_q)]
    x = synth.decode_inputs(wl, lens, 900 + k, DEV, n_q=n_q)
    log(f"paged CSA k={k}: {n} seqs, ctx {min(lens)}..{max(lens)}, {sum(n_q)} query tokens")
    sq = ops.Seqs(n_q, lens, x["entry_off"], x["tok_off"], x["tok_lo"])
    R = {key: ops.Rows.of(x[key].clone()) for key in ("kv", "c", "z", "kI", "cI", "zI", "qI", "q")}
    idx_a, out_a, lse_a = _csa_run(sq, R["kv"], R["c"], R["z"], R["kI"], R["cI"], R["zI"], R["qI"], R["q"], x, wl, k)

    pg = Paged(g, x, wl.ratio, n_q)
    kv_p0 = pg.entries(x["kv"], 1)
    kI_p0 = pg.entries(x["kI"], 2)
    kv_p, kI_p = kv_p0.clone(), kI_p0.clone()
    c_r, z_r = pg.ring(x["c"], 3), pg.ring(x["z"], 4)
    cI_r, zI_r = pg.ring(x["cI"], 5), pg.ring(x["zI"], 6)
    sp = pg.seqs()
    idx_b, out_b, lse_b = _csa_run(sp, ops.Rows.of(kv_p), ops.Rows.of(c_r), ops.Rows.of(z_r), ops.Rows.of(kI_p),
                                   ops.Rows.of(cI_r), ops.Rows.of(zI_r), R["qI"], R["q"], x, wl, k)
    torch.cuda.synchronize()
    assert torch.equal(idx_a, idx_b), "idx differs between paged and contiguous pools"
    assert torch.equal(out_a.view(torch.int16), out_b.view(torch.int16)), "out bits differ"
    assert torch.equal(lse_a.view(torch.int32), lse_b.view(torch.int32)), "lse bits differ"
    # new entries at their block-table rows, every other physical row untouched
    touched = torch.zeros(pg.n_rows, dtype=torch.bool, device=DEV)
    for b, L in enumerate(lens):
        for i in range((L - n_q[b]) // wl.ratio, L // wl.ratio):
            r = pg.erow[b][i]
            e0 = x["entry_off"][b]
            assert torch.equal(kv_p[r].view(torch.int16), R["kv"].data[e0 + i].view(torch.int16)), f"seq {b} entry {i}"
            assert torch.equal(kI_p[r].view(torch.int16), R["kI"].data[e0 + i].view(torch.int16))
            touched[r] = True
    assert torch.equal(kv_p[~touched].view(torch.int16), kv_p0[~touched].view(torch.int16)), "other rows changed"
    assert torch.equal(kI_p[~touched].view(torch.int16), kI_p0[~touched].view(torch.int16)), "other rows changed"
    log(f"paged CSA k={k}: idx, out, lse and entries bit-identical to contiguous pools")

    # the oracle, reading the logical rows through the block table and the ring on the host
    if k == 512:
        f64 = lambda t: t.detach().float().cpu().numpy().astype(np.float64)  # noqa: E731
        kvh, kIh, ch = f64(kv_p), f64(kI_p), f64(c_r)
        qIh, wh, qh, sink = f64(x["qI"]), f64(x["w"]), f64(x["q"]), f64(x["sink"])
        gi = idx_b.cpu().numpy()
        oh, lh = f64(out_b).reshape(-1, wl.n_h, wl.d_c), lse_b.cpu().numpy()
        for b in range(0, n, 3):
            L = lens[b]
            p = L - 1
            V = visible(p, wl.ratio)
            rows = pg.erow[b].cpu().numpy()
            kI_log = kIh[rows[:V]]
            s = index_scores(qIh[b * wl.n_I:(b + 1) * wl.n_I], wh[b], kI_log)
            check_topk(gi[b], topk_select(s, k), s, k)
            lo = x["tok_lo"][b]
            toks = ch[b * RING + np.arange(lo, L) % RING]
            o, lr = attend_token(qh[b * wl.n_h:(b + 1) * wl.n_h], p, kvh[rows], list(gi[b]), toks, wl.n_win, sink,
                                 1.0 / math.sqrt(wl.d_c), wl.rope_dims, wl.rope_theta, tok_lo=lo)
            assert_close(oh[b], o, 1e-2, f"paged out seq {b}")
            assert_close(lh[b], lr, 1e-2, f"paged lse seq {b}")
        log("paged CSA: oracle through the block table agrees")


def test_paged_hca_equals_contiguous():
    """HCA layer (128:1, one entry per 128-token block): compress and dense attention, split
    launch, with contexts up to 1M."""
    wl = configs.HCA_DECODE_1M_BF16
    g = synth.rng(80)
    n = 6
    lens = [int(v) for v in synth.log_uniform_ints(g, n, 20000, 1 << 20)]
    n_q = [1, 3, 1, 2, 1, 1]
    x = synth.decode_inputs(wl, lens, 950, DEV, n_q=n_q)
    sq = ops.Seqs(n_q, lens, x["entry_off"], x["tok_off"], x["tok_lo"])

    def run(seqs, kv, c, z):
        ops.csa_compress(seqs, c, z, x["bias"], wl.ratio, wl.overlap, wl.rope_dims, wl.rope_theta, kv)
        n_tok = seqs.total_q
        out = ops.Rows.of(torch.empty((n_tok * wl.n_h, wl.d_c), dtype=torch.bfloat16, device=DEV))
        lse = torch.empty((n_tok, wl.n_h), dtype=torch.float32, device=DEV)
        wsb = ops.csa_workspace_bytes(ops.OP_HCA_ATTEND, seqs, wl.n_h, wl.d_c, 0, wl.ratio, wl.n_win)
        ws = torch.empty(wsb // 4 + 1, device=DEV) if wsb else None
        ops.hca_attend(seqs, ops.Rows.of(x["q"]), wl.n_h, kv, wl.ratio, c, wl.n_win, x["sink"],
                       1.0 / math.sqrt(wl.d_c), wl.rope_dims, wl.rope_theta, out, lse, ws=ws)
        return out.data, lse

    kv_c = x["kv"].clone()
    out_a, lse_a = run(sq, ops.Rows.of(kv_c), ops.Rows.of(x["c"]), ops.Rows.of(x["z"]))
    pg = Paged(g, x, wl.ratio, n_q, ring=512)   # HCA sources: the last 128 tokens of a block
    kv_p = pg.entries(x["kv"], 11)
    out_b, lse_b = run(pg.seqs(), ops.Rows.of(kv_p), ops.Rows.of(pg.ring(x["c"], 12)), ops.Rows.of(pg.ring(x["z"], 13)))
    torch.cuda.synchronize()
    assert torch.equal(out_a.view(torch.int16), out_b.view(torch.int16)), "out bits differ"
    assert torch.equal(lse_a.view(torch.int32), lse_b.view(torch.int32)), "lse bits differ"
    for b, L in enumerate(lens):
        for i in range((L - n_q[b]) // wl.ratio, L // wl.ratio):
            assert torch.equal(kv_p[pg.erow[b][i]].view(torch.int16), kv_c[x["entry_off"][b] + i].view(torch.int16))
    log(f"paged HCA: {n} seqs up to {max(lens)} tokens bit-identical to contiguous pools")


def test_paged_mixed_precision_prefill_equals_contiguous():
    """Multi-token prefill chunks with fp8 KV rows and MXFP4 indexer keys (the query-block
    indexer kernel and the 64-head attention kernel), paged with 32 entries per block."""
    from harness import kv_split, mxfp4
    wl = configs.CSA_PREFILL_MIXED
    g = synth.rng(90)
    n_q, lens = [40, 17, 64], [3000, 70000, 9000]
    n = len(lens)
    D, n_h, n_I, d_I, ratio, k = wl.d_c, wl.n_h, wl.n_I, wl.d_I, wl.ratio, wl.k
    E = [L // ratio for L in lens]
    entry_off = list(np.concatenate([[0], np.cumsum(E)[:-1]]).astype(int))
    tok_lo = [max(0, L - q - wl.n_win - 2 * ratio) for L, q in zip(lens, n_q)]
    rows = [L - lo for L, lo in zip(lens, tok_lo)]
    tok_off = list(np.concatenate([[0], np.cumsum(rows)[:-1]]).astype(int))
    kv_rows, _ = kv_split(g.standard_normal((sum(E), D)))
    kI_rows, _ = mxfp4(g.standard_normal((sum(E), d_I)))
    c_rows, _ = kv_split(g.standard_normal((sum(rows), D)))
    z = torch.from_numpy(g.standard_normal((sum(rows), D))).to(torch.bfloat16).to(DEV)
    cI = torch.from_numpy(g.standard_normal((sum(rows), d_I))).to(torch.bfloat16).to(DEV)
    zI = torch.from_numpy(g.standard_normal((sum(rows), d_I))).to(torch.bfloat16).to(DEV)
    qI_rows, _ = mxfp4(g.standard_normal((sum(n_q) * n_I, d_I)))
    q = torch.from_numpy(g.standard_normal((sum(n_q) * n_h, D))).to(torch.bfloat16).to(DEV)
    w = torch.from_numpy((g.standard_normal((sum(n_q), n_I)) / 8).astype(np.float32)).to(DEV)
    sink = torch.from_numpy(g.standard_normal(n_h).astype(np.float32)).to(DEV)
    bias = torch.from_numpy((g.standard_normal((2 * ratio, D)) / math.sqrt(D)).astype(np.float32)).to(DEV)
    biasI = torch.from_numpy((g.standard_normal((2 * ratio, d_I)) / math.sqrt(d_I)).astype(np.float32)).to(DEV)

    def run(seqs, kv, kI, c, z_, cI_, zI_):
        ops.csa_compress2(seqs, ratio, 1, wl.rope_theta, (c, z_, bias, wl.rope_dims, kv), (cI_, zI_, biasI, 0, kI))
        idx = torch.full((sum(n_q), k), -7, dtype=torch.int32, device=DEV)
        ws = torch.empty(ops.csa_workspace_bytes(ops.OP_INDEX_TOPK, seqs, k=k, ratio=ratio) // 4 + 1, device=DEV)
        ops.csa_index_topk(seqs, qI_rows, w, n_I, kI, ratio, k, idx, ws=ws)
        out = ops.Rows.of(torch.empty((sum(n_q) * n_h, D), dtype=torch.bfloat16, device=DEV))
        lse = torch.empty((sum(n_q), n_h), dtype=torch.float32, device=DEV)
        ops.csa_attend(seqs, ops.Rows.of(q), n_h, kv, idx, k, c, wl.n_win, sink, 1.0 / math.sqrt(D), wl.rope_dims,
                       wl.rope_theta, out, lse)
        return idx, out.data, lse

    sq = ops.Seqs(n_q, lens, entry_off, tok_off, tok_lo)
    kv_c = ops.Rows(kv_rows.data.clone(), ops.KV_SPLIT, D, kv_rows.scales.clone())
    kI_c = ops.Rows(kI_rows.data.clone(), ops.MXFP4, d_I, kI_rows.scales.clone())
    a = run(sq, kv_c, kI_c, c_rows, ops.Rows.of(z), ops.Rows.of(cI), ops.Rows.of(zI))
    x = dict(E=E, lens=lens, entry_off=entry_off, tok_off=tok_off, tok_lo=tok_lo)
    pg = Paged(g, x, ratio, n_q)
    kv_p = ops.Rows(pg.entries(kv_rows.data, 21), ops.KV_SPLIT, D, pg.entries(kv_rows.scales.view(torch.uint8), 22)
                    .view(torch.float32))
    kI_p = ops.Rows(pg.entries(kI_rows.data, 23), ops.MXFP4, d_I, pg.entries(kI_rows.scales, 24))
    c_p = ops.Rows(pg.ring(c_rows.data.view(torch.int16), 25).view(torch.uint8), ops.KV_SPLIT, D,
                   pg.ring(c_rows.scales, 26))
    b = run(pg.seqs(), kv_p, kI_p, c_p, ops.Rows.of(pg.ring(z, 27)), ops.Rows.of(pg.ring(cI, 28)),
            ops.Rows.of(pg.ring(zI, 29)))
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]), "idx differs"
    assert torch.equal(a[1].view(torch.int16), b[1].view(torch.int16)), "out bits differ"
    assert torch.equal(a[2].view(torch.int32), b[2].view(torch.int32)), "lse bits differ"
    log("paged prefill chunks (fp8 KV, MXFP4 keys): bit-identical to contiguous pools")


@pytest.mark.parametrize("fmt,epb", [("mxfp4", 32), ("fp8", 32), ("mxfp4", 4), ("bf16", 32), ("bf16", 4)])
def test_paged_decode_indexer_equals_contiguous(fmt, epb):
    """The decode indexer (MXFP4 or fp8 1x128 keys on the scaled matrix cores, or bf16 keys,
    one query row per sequence) over paged key pools gives the contiguous pools' score bits.  64 sequences
    of 524288 tokens (131072 entries each): enough work that the contiguous launch takes
    ranges of 4096 entries while the paged one keeps each range within one block-id load
    (2048 entries of 32-entry blocks), so the two launches also split the rows differently.
    With 4-entry blocks a range spans more blocks than one load holds, and the later rows
    take their block ids from the table one by one.
    (The bf16 kernel's ranges are 448 entries: 4-entry blocks take it past one load too.)
    Key bytes are drawn directly in the format (any e2m1 code; e8m0 scales near 1; e4m3
    codes without the NaN pattern, fp32 row scales; bf16 from N(0,1)), which is all bit
    equality needs."""
    n, L, ratio, n_I, d_I = 64, 524288, 4, 64, 128
    V = L // ratio
    gen = torch.Generator(device=DEV)
    gen.manual_seed(71)

    def rows(count, seed_shift):
        gen.manual_seed(71 + seed_shift)
        if fmt == "bf16":
            data = torch.randn((count, d_I), generator=gen, device=DEV).to(torch.bfloat16)
            return data, None
        if fmt == "mxfp4":
            data = torch.randint(0, 256, (count, d_I // 2), generator=gen, device=DEV, dtype=torch.uint8)
            sc = torch.randint(122, 133, (count, d_I // 32), generator=gen, device=DEV, dtype=torch.uint8)
            return data, sc
        data = torch.randint(0, 256, (count, d_I), generator=gen, device=DEV, dtype=torch.uint8)
        data = torch.where((data & 0x7f) == 0x7f, data - 1, data)  # no NaN code
        sc = torch.rand((count, 1), generator=gen, device=DEV, dtype=torch.float32) * 0.01 + 0.001
        return data, sc

    kind = {"mxfp4": ops.MXFP4, "fp8": ops.FP8_B128, "bf16": ops.BF16}[fmt]
    k_data, k_sc = rows(n * V, 0)
    q_data, q_sc = rows(n * n_I, 1)
    w = (torch.randn((n, n_I), generator=gen, device=DEV) / 8).contiguous()
    qI = ops.Rows(q_data, kind, d_I, q_sc)

    # paged copy: the blocks of all sequences placed by a random permutation among 7 spare ones
    nblk = V // epb
    total = n * nblk + 7
    perm = torch.randperm(total, generator=gen, device=DEV)
    table = perm[: n * nblk].view(n, nblk)
    erow = (table.repeat_interleave(epb, dim=1) * epb + torch.arange(V, device=DEV) % epb).reshape(-1)
    if fmt == "bf16":
        pk_data = torch.randn((total * epb, d_I), generator=gen, device=DEV).to(torch.bfloat16)
        pk_sc = None
    else:
        pk_data = torch.randint(0, 256, (total * epb,) + tuple(k_data.shape[1:]), generator=gen, device=DEV,
                                dtype=torch.uint8)
        if fmt == "fp8":
            pk_data = torch.where((pk_data & 0x7f) == 0x7f, pk_data - 1, pk_data)
        pk_sc = torch.ones((total * epb,) + tuple(k_sc.shape[1:]), device=DEV, dtype=k_sc.dtype)
        pk_sc[erow] = k_sc
    pk_data[erow] = k_data

    lens = [L] * n
    sq_c = ops.Seqs([1] * n, lens, [b * V for b in range(n)], [0] * n, [L - 1] * n)
    sq_p = ops.Seqs([1] * n, lens, [0] * n, [0] * n, [L - 1] * n, block_table=table.cpu().tolist(),
                    block_entries=epb)
    s_c = torch.full((n, V), float("nan"), device=DEV)
    s_p = torch.full((n, V), float("nan"), device=DEV)
    ops.csa_index_score(sq_c, qI, w, n_I, ops.Rows(k_data, kind, d_I, k_sc), ratio, s_c)
    ops.csa_index_score(sq_p, qI, w, n_I, ops.Rows(pk_data, kind, d_I, pk_sc), ratio, s_p)
    torch.cuda.synchronize()
    assert torch.isfinite(s_c).all(), "every visible entry scored, finite"
    assert torch.equal(s_c.view(torch.int32), s_p.view(torch.int32)), "paged scores differ from contiguous"
    log(f"paged {fmt} decode indexer: {n} x {V} scores bit-identical to contiguous pools")
