"""GPU parity of the paged cache layout (uniform mode with token-axis groups or
channel-axis K, Oaken's dense body with per-sequence sparse lists, the
chunk-mixed class pools with one block table per class, and DSQ's 64-token
groups).

Pages are handed out in a seeded random order from a pool larger than the
sequences need.  Codes and scales gathered through the block table must equal
the oracle's bit for bit; decode must equal, bit for bit, the decode of a
contiguous cache holding the same data (same arithmetic in the same order),
and meet the attention bar against the oracle.
"""
import numpy as np
import pytest

import oracle
import synth
from kvq_harness import ATTN_BAR, ATTN_TIGHT, host_bytes, i32_device, rel_err_rows, to_device, unpack_layout

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
K = pytest.importorskip("quantized_kv_cache_05_amd")

SM = 1.0 / np.sqrt(128.0)
LAYOUT = {"k": "K", "v": "V"}

# (bits, symmetric, group, format)
CODECS = [(8, True, 128, 0), (4, False, 64, 0), (2, False, 32, 0), (8, False, 128, 1), (8, False, 128, 2)]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    K.lib()
    yield


def f32bits(a):
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


def make(B, H, S, codec, P=0, pages=0, table=None):
    bits, sym, group, fmt = codec
    return K.QuantKVCache(B, H, S, K.KVQ_MODE_UNIFORM, k_bits=bits, symmetric=sym, k_group=group, fmt=fmt,
                          page_tokens=P, num_pages=pages,
                          block_table=None if table is None else i32_device(table.reshape(-1)))


def decode(cache, q, Hq, lens, max_len, ns):
    B = q.shape[0]
    out = torch.full((B, Hq, 128), float("nan"), dtype=torch.float32, device="cuda")
    ws, n = cache.workspace(Hq, max_len, ns)
    K.kvq_decode_attn(cache.desc, to_device(q), Hq, i32_device(lens), max_len, SM, out, ws, n, ns)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def oracle_rows(x, codec):
    bits, sym, group, fmt = codec
    if fmt:
        q, dq = ((oracle.quant_rows_e4m3, oracle.dequant_rows_e4m3) if fmt == 1 else
                 (oracle.quant_rows_e5m2, oracle.dequant_rows_e5m2))
        c, s = q(x, group)
        return c, s, None, dq(c, s, group)
    c, s, z = oracle.quant_rows(x, group, bits, sym)
    return c, s, z, oracle.dequant_rows(c, s, z, group, sym)


@pytest.mark.parametrize("codec", CODECS)
@pytest.mark.parametrize("P", [64, 256])
@pytest.mark.parametrize("G", [1, 4, 16])
def test_paged_matches_contiguous(codec, P, G):
    bits, sym, group, fmt = codec
    B, H, S, T = 3, 2, 512, 333
    print("case paged codec=%s P=%d G=%d" % (codec, P, G), flush=True)
    w = synth.scaled(synth.WORKLOADS[1], batch=B, kv_heads=H, q_heads=H * G, seq=T + 1, tokens=T + 1)
    k, v, q = w.kv(0), w.kv(1), w.q()
    per_seq = S // P
    used = -(-(T + 1) // P)  # pages each sequence touches
    pool = B * used + 3  # a few pages never handed out
    rng = np.random.default_rng(1000 + P + bits)
    ids = rng.permutation(pool)[:B * used].reshape(B, used)
    table = np.full((B, per_seq), -1, np.int32)
    table[:, :used] = ids
    paged = make(B, H, S, codec, P, pool, table)
    flat = make(B, H, S, codec)
    app = np.array([T, 200, 100])  # single-token appends at different positions
    for cache in (paged, flat):
        K.kvq_quant_append(cache.desc, to_device(k[:, :, :T]), to_device(v[:, :, :T]), T, i32_device([0] * B))
        K.kvq_quant_append(cache.desc, to_device(k[:, :, T:T + 1]), to_device(v[:, :, T:T + 1]), 1,
                           i32_device(app))
    torch.cuda.synchronize()
    assert paged.flags() == 0 and flat.flags() == 0
    RB, NG = 128 * bits // 8, 128 // group
    lens = [T + 1, 201, 101]
    deq = {}
    for name, x in (("k", k), ("v", v)):
        logical = x[:, :, :T + 1].copy()
        for b in range(B):
            logical[b, :, app[b]] = x[b, :, T]
        oc, os_, oz, xh = oracle_rows(logical, codec)
        deq[name] = xh
        codes = host_bytes(paged.buf(name + ".codes")).reshape(pool, H, P, RB)
        scale = host_bytes(paged.buf(name + ".scale")).view(np.float32).reshape(pool, H, P, NG)
        zero = None if (sym or fmt) else host_bytes(paged.buf(name + ".zero")).reshape(pool, H, P, NG)
        for b, L in enumerate(lens):
            t = np.arange(L)
            pg, r = table[b, t // P], t % P
            got = unpack_layout(codes[pg, :, r].transpose(1, 0, 2), bits, LAYOUT[name], sym)
            assert np.array_equal(got, oc[b, :, :L]), (name, b)
            assert np.array_equal(f32bits(scale[pg, :, r].transpose(1, 0, 2)), f32bits(os_[b, :, :L])), (name, b)
            if zero is not None:
                assert np.array_equal(zero[pg, :, r].transpose(1, 0, 2), oz[b, :, :L]), (name, b)
    for ns in (0, 1, 3):
        out_p = decode(paged, q, H * G, lens, T + 1, ns)
        out_f = decode(flat, q, H * G, lens, T + 1, ns)
        assert np.array_equal(out_p.view(np.uint32), out_f.view(np.uint32)), ns
        refs = np.stack([oracle.attention(q[b], deq["k"][b][:, :L], deq["v"][b][:, :L], SM)
                         for b, L in enumerate(lens)])
        err = float(rel_err_rows(out_p, refs).max())
        print("paged %s P%d G%d ns%d: max rel err %.3e" % (codec, P, G, ns, err), flush=True)
        assert err <= ATTN_BAR and err <= ATTN_TIGHT


def test_paged_bad_page_is_flagged():
    codec = (4, False, 64, 0)
    B, H, S, P = 2, 2, 256, 64
    w = synth.scaled(synth.WORKLOADS[1], batch=B, kv_heads=H, q_heads=H, seq=128, tokens=128)
    k, v, q = w.kv(0), w.kv(1), w.q()
    table = np.array([[0, 1, -1, -1], [2, 9, -1, -1]], np.int32)  # page 9 is outside a 4-page pool
    cache = make(B, H, S, codec, P, 4, table)
    K.kvq_quant_append(cache.desc, to_device(k), to_device(v), 128, i32_device([0, 0]))
    torch.cuda.synchronize()
    assert cache.flags() & K.KVQ_FLAG_PAGE_RANGE
    cache.status.zero_()
    out = decode(cache, q, H, [128, 64], 128, 0)  # sequence 1 stops before the bad page
    assert cache.flags() == 0 and np.all(np.isfinite(out))
    decode(cache, q, H, [128, 128], 128, 0)  # now it reads through it: page 0 instead, flagged
    assert cache.flags() & K.KVQ_FLAG_PAGE_RANGE


@pytest.mark.parametrize("P", [64, 128])
@pytest.mark.parametrize("G", [1, 4, 16])
def test_paged_oaken(P, G):
    """Oaken with its dense body in pages and its sparse lists per sequence: the sparse lists equal
    the contiguous cache's byte for byte, every dense row gathered through the block table equals
    the contiguous cache's row, decode equals the contiguous decode bit for bit and meets the
    attention bar against the oracle."""
    from test_gpu_parity import oaken_thresholds
    B, H, S, T = 2, 3, 512, 333
    print("case paged oaken P=%d G=%d" % (P, G), flush=True)
    w = synth.scaled(synth.WORKLOADS[5], batch=B, kv_heads=H, q_heads=H * G, seq=T, tokens=T)
    wc = synth.scaled(synth.WORKLOADS[5], kv_heads=4, seq=256)
    thr_k, thr_v = oaken_thresholds(wc, 0, 20), oaken_thresholds(wc, 1, 20)
    k, v, q = w.kv(0), w.kv(1), w.q()
    per_seq, used = S // P, -(-T // P)
    pool = B * used + 2
    ids = np.random.default_rng(77 + P).permutation(pool)[:B * used].reshape(B, used)
    table = np.full((B, per_seq), -1, np.int32)
    table[:, :used] = ids
    cap = S * 24
    # zero-filled, so that the unwritten tails of the sparse buffers compare equal too
    kw = dict(k_bits=4, k_group=64, k_thr=thr_k, v_thr=thr_v, sparse_cap=cap, zero_fill=True)
    paged = K.QuantKVCache(B, H, S, K.KVQ_MODE_OAKEN, page_tokens=P, num_pages=pool,
                           block_table=i32_device(table.reshape(-1)), **kw)
    flat = K.QuantKVCache(B, H, S, K.KVQ_MODE_OAKEN, **kw)
    for cache in (paged, flat):  # bulk 300 rows, 32 more, then one row (the one-token kernel)
        K.kvq_quant_append(cache.desc, to_device(k[:, :, :300]), to_device(v[:, :, :300]), 300, i32_device([0] * B))
        K.kvq_quant_append(cache.desc, to_device(k[:, :, 300:332]), to_device(v[:, :, 300:332]), 32,
                           i32_device([300] * B))
        K.kvq_quant_append(cache.desc, to_device(k[:, :, 332:]), to_device(v[:, :, 332:]), 1, i32_device([332] * B))
    torch.cuda.synchronize()
    assert paged.flags() == 0 and flat.flags() == 0
    for name in ("k", "v"):
        for f in ("rowptr", "sparse"):
            assert np.array_equal(host_bytes(paged.buf(name + "." + f)), host_bytes(flat.buf(name + "." + f))), (name, f)
        for f, per in (("codes", 64), ("scale", 8), ("zero", 2), ("oscale", 8)):
            pg = host_bytes(paged.buf(name + "." + f)).reshape(pool, H, P, per)
            fl = host_bytes(flat.buf(name + "." + f)).reshape(B, H, S, per)
            for b in range(B):
                t = np.arange(T)
                got = pg[table[b, t // P], :, t % P].transpose(1, 0, 2)
                assert np.array_equal(got, fl[b, :, :T]), (name, f, b)
    deq = {}
    for name, x, thr in (("k", k, thr_k), ("v", v, thr_v)):
        deq[name] = oracle.oaken_dequant_rows(*oracle.oaken_rows(x, thr, 64), thr, 64)
    for lens in ([T, T], [T, 190]):
        refs = np.stack([oracle.attention(q[b], deq["k"][b][:, :L], deq["v"][b][:, :L], SM)
                         for b, L in enumerate(lens)])
        for ns in (0, 1, 3):
            out_p = decode(paged, q, H * G, lens, T, ns)
            out_f = decode(flat, q, H * G, lens, T, ns)
            # same arithmetic in the same order (no atomics touch the output): bit for bit
            assert np.array_equal(out_p.view(np.uint32), out_f.view(np.uint32)), (lens, ns)
            err = float(rel_err_rows(out_p, refs).max())
            print("paged oaken P%d G%d ns%d lens%s: max rel err %.3e" % (P, G, ns, lens, err), flush=True)
            assert err <= ATTN_BAR and err <= ATTN_TIGHT


@pytest.mark.parametrize("P", [64, 128])
@pytest.mark.parametrize("G", [1, 4, 16])
def test_paged_dsq(P, G):
    """DSQ with its groups in pages: streamed appends into a paged and a contiguous cache give the
    same groups (gathered through the block table) and tails byte for byte, decode equals the
    contiguous decode bit for bit and meets the attention bar against the oracle."""
    B, H, S = 2, 2, 512
    sizes = [130, 1, 60, 64, 77]
    T = sum(sizes)
    print("case paged dsq P=%d G=%d" % (P, G), flush=True)
    w = synth.scaled(synth.WORKLOADS[8], batch=B, kv_heads=H, q_heads=H * G, seq=T, tokens=T)
    k, v, q, sc = w.kv(0), w.kv(1), w.q(), w.scores()
    per_seq, used = S // P, -(-T // P)
    pool = B * used + 2
    ids = np.random.default_rng(99 + P).permutation(pool)[:B * used].reshape(B, used)
    table = np.full((B, per_seq), -1, np.int32)
    table[:, :used] = ids
    kw = dict(k_group=32, v_group=32, dsq_sig=13, zero_fill=True)
    paged = K.QuantKVCache(B, H, S, K.KVQ_MODE_DSQ, page_tokens=P, num_pages=pool,
                           block_table=i32_device(table.reshape(-1)), **kw)
    flat = K.QuantKVCache(B, H, S, K.KVQ_MODE_DSQ, **kw)
    L = 0
    for n in sizes:
        for cache in (paged, flat):
            K.kvq_dsq_append(cache.desc, to_device(np.ascontiguousarray(k[:, :, L:L + n])),
                             to_device(np.ascontiguousarray(v[:, :, L:L + n])),
                             torch.from_numpy(np.ascontiguousarray(sc[:, :, L:L + n])).cuda(), n, i32_device([L] * B))
        L += n
    torch.cuda.synchronize()
    assert paged.flags() == 0 and flat.flags() == 0
    gpp, Q = P // 64, S // 64
    for name, per in (("k.codes", 2048), ("v.codes", 2048), ("k.scale", 512), ("v.scale", 512),
                      ("k.codes2", 2048), ("v.codes2", 2048), ("k.scale2", 1024), ("v.scale2", 1024),
                      ("k.zero2", 256), ("v.zero2", 256), ("dsq_mask", 8)):
        pg = host_bytes(paged.buf(name)).view(np.uint8).reshape(pool, H, gpp, per)
        fl = host_bytes(flat.buf(name)).view(np.uint8).reshape(B, H, Q, per)
        for b in range(B):
            g = np.arange(T // 64)
            got = pg[table[b, g // gpp], :, g % gpp].transpose(1, 0, 2)
            assert np.array_equal(got, fl[b, :, :T // 64]), (name, b)
    for name in ("k.codes16", "v.codes16", "k.oscale"):
        assert np.array_equal(host_bytes(paged.buf(name)), host_bytes(flat.buf(name))), name
    n0 = T & ~63
    deq = {}
    for b in range(B):
        for h in range(H):
            kh = np.zeros((T, 128), np.float32)
            vh = np.zeros((T, 128), np.float32)
            kh[:n0], vh[:n0] = oracle.dsq_dequant(oracle.dsq_quant(k[b, h, :n0], v[b, h, :n0], sc[b, h, :n0]))
            kh[n0:] = k[b, h, n0:].view(np.float16).astype(np.float32)
            vh[n0:] = v[b, h, n0:].view(np.float16).astype(np.float32)
            deq[b, h] = kh, vh
    for lens in ([T, T], [T, n0 - 64]):
        refs = np.stack([oracle.attention(q[b], np.stack([deq[b, h][0][:Lb] for h in range(H)]),
                                          np.stack([deq[b, h][1][:Lb] for h in range(H)]), SM)
                         for b, Lb in enumerate(lens)])
        for ns in (0, 1, 3):
            out_p = decode(paged, q, H * G, lens, T, ns)
            out_f = decode(flat, q, H * G, lens, T, ns)
            assert np.array_equal(out_p.view(np.uint32), out_f.view(np.uint32)), (lens, ns)
            err = float(rel_err_rows(out_p, refs).max())
            print("paged dsq P%d G%d ns%d lens%s: max rel err %.3e" % (P, G, ns, lens, err), flush=True)
            assert err <= ATTN_BAR and err <= ATTN_TIGHT


@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("P", [64, 256])
@pytest.mark.parametrize("G", [1, 4, 16])
def test_paged_channel_k(bits, P, G):
    """K per channel over 64-token blocks with its codes and block scales in pages (a block never
    straddles a page), the fp16 tail per sequence: streamed appends into a paged and a contiguous
    cache give the same blocks (gathered through the block table), tails and V rows byte for byte,
    decode equals the contiguous decode bit for bit and meets the attention bar against the oracle."""
    B, H, S = 2, 2, 512
    steps = [300, 1, 70, 29]  # 400 tokens: blocks completed in bulk, by one token and across appends
    T = sum(steps)
    print("case paged channel-K bits=%d P=%d G=%d" % (bits, P, G), flush=True)
    w = synth.scaled(synth.WORKLOADS[3], batch=B, kv_heads=H, q_heads=H * G, seq=T, tokens=T)
    k, v, q = w.kv(0), w.kv(1), w.q()
    per_seq, used = S // P, -(-T // P)
    pool = B * used + 3
    ids = np.random.default_rng(500 + P + bits).permutation(pool)[:B * used].reshape(B, used)
    table = np.full((B, per_seq), -1, np.int32)
    table[:, :used] = ids
    kw = dict(k_bits=bits, k_axis=K.KVQ_AXIS_CHANNEL, k_group=64, v_group=64, zero_fill=True)
    paged = K.QuantKVCache(B, H, S, K.KVQ_MODE_UNIFORM, page_tokens=P, num_pages=pool,
                           block_table=i32_device(table.reshape(-1)), **kw)
    flat = K.QuantKVCache(B, H, S, K.KVQ_MODE_UNIFORM, **kw)
    L = 0
    for n in steps:
        for cache in (paged, flat):
            K.kvq_quant_append(cache.desc, to_device(np.ascontiguousarray(k[:, :, L:L + n])),
                               to_device(np.ascontiguousarray(v[:, :, L:L + n])), n, i32_device([L] * B))
        L += n
    torch.cuda.synchronize()
    assert paged.flags() == 0 and flat.flags() == 0
    RB, nq = 128 * bits // 8, T // 64 * 64
    t = np.arange(T)
    for name, per, rows in (("k.codes", RB, nq), ("v.codes", RB, T), ("v.scale", 8, T), ("v.zero", 2, T)):
        pg = host_bytes(paged.buf(name)).view(np.uint8).reshape(pool, H, P, per)
        fl = host_bytes(flat.buf(name)).view(np.uint8).reshape(B, H, S, per)
        for b in range(B):
            got = pg[table[b, t[:rows] // P], :, t[:rows] % P].transpose(1, 0, 2)
            assert np.array_equal(got, fl[b, :, :rows]), (name, b)
    for name, per in (("k.scale", 512), ("k.zero", 128)):  # per 64-token block
        pg = host_bytes(paged.buf(name)).view(np.uint8).reshape(pool, H, P // 64, per)
        fl = host_bytes(flat.buf(name)).view(np.uint8).reshape(B, H, S // 64, per)
        for b in range(B):
            blk = np.arange(nq // 64)
            got = pg[table[b, blk * 64 // P], :, blk % (P // 64)].transpose(1, 0, 2)
            assert np.array_equal(got, fl[b, :, :nq // 64]), (name, b)
    assert np.array_equal(host_bytes(paged.buf("k.codes16")), host_bytes(flat.buf("k.codes16")))
    kc, ks, kz = oracle.quant_channel_blocks(k[:, :, :nq], 64, bits)
    kh = np.concatenate([oracle.dequant_channel_blocks(kc, ks, kz, 64),
                         k[:, :, nq:T].view(np.float16).astype(np.float32)], axis=2)
    vc, vs, vz = oracle.quant_rows(v, 64, bits)
    vh = oracle.dequant_rows(vc, vs, vz, 64)
    for lens in ([T, T], [T, nq - 64]):
        refs = np.stack([oracle.attention(q[b], kh[b][:, :Lb], vh[b][:, :Lb], SM) for b, Lb in enumerate(lens)])
        for ns in (0, 1, 3):
            out_p = decode(paged, q, H * G, lens, T, ns)
            out_f = decode(flat, q, H * G, lens, T, ns)
            assert np.array_equal(out_p.view(np.uint32), out_f.view(np.uint32)), (lens, ns)
            err = float(rel_err_rows(out_p, refs).max())
            print("paged channel b%d P%d G%d ns%d lens%s: max rel err %.3e" % (bits, P, G, ns, lens, err),
                  flush=True)
            assert err <= ATTN_BAR and err <= ATTN_TIGHT


# chunk-mixed class pools: (buffer, bytes per row) of each class, groups of 32 channels
MIX_CLASS_BUFS = {0: (("codes16", 256),), 1: (("codes", 64), ("scale", 16), ("zero", 4)),
                  2: (("codes2", 32), ("scale2", 16), ("zero2", 4))}


def mixed_tables(rng, seg, B, S, P, CT):
    """Per-class block tables [3][B][S / P] mapping the pages each class of each sequence uses (by
    the final seg, plus the FP16 page of the waiting chunk), drawn at random from that class's pool."""
    per_seq = S // P
    tables = np.full((3, B, per_seq), -1, np.int32)
    need = []
    for c in range(3):
        lp = []
        for b in range(B):
            pages = set(range(-(-int(seg[b, c]) * CT // P)))
            if c == 0:
                pages.add((S - CT) // P)  # the waiting chunk: the FP16 class's last chunk
            lp.append(sorted(pages))
        need.append(lp)
    pool = max(sum(len(x) for x in lp) for lp in need) + 3
    for c in range(3):
        ids = iter(rng.permutation(pool))
        for b in range(B):
            for lpg in need[c][b]:
                tables[c, b, lpg] = next(ids)
    return tables, pool


def gather_class_rows(cache, name, field, per, pool, H, P, table_cb, rows):
    """Rows 0 .. rows-1 of one sequence's class pool, [H][rows][per] bytes, through its table."""
    pg = host_bytes(cache.buf(name + "." + field)).view(np.uint8)[:pool * H * P * per].reshape(pool, H, P, per)
    r = np.arange(rows)
    return pg[table_cb[r // P], :, r % P].transpose(1, 0, 2)


@pytest.mark.parametrize("P,CT", [(64, 16), (64, 32), (128, 32)])
@pytest.mark.parametrize("G", [1, 4, 16])
def test_paged_chunk_mixed(P, CT, G):
    """Cocktail class pools in pages, one block table per class: the bulk path (reorder, then
    quantize) and streamed appends (the waiting chunk in the FP16 class's last page) into paged and
    contiguous caches give the same class rows (gathered through each class's table) byte for byte;
    decode equals the contiguous decode bit for bit and meets the attention bar against the oracle."""
    B, H, S, group = 2, 2, 512, 32
    C = S // CT
    print("case paged mixed P=%d CT=%d G=%d" % (P, CT, G), flush=True)
    w = synth.scaled(synth.WORKLOADS[4], batch=B, kv_heads=H, q_heads=H * G, seq=S, tokens=S, emb_dim=64)
    k, v, q = w.kv(0), w.kv(1), w.q()
    rng = np.random.default_rng(300 + P + CT)
    bits = rng.choice(np.array([16, 4, 2], np.uint8), size=(B, C), p=[0.2, 0.35, 0.45])
    perm_o, seg_o = oracle.reorder(bits)
    tables, pool = mixed_tables(rng, seg_o, B, S, P, CT)
    kw = dict(k_group=group, chunk_tokens=CT, zero_fill=True)

    def pair():
        paged = K.QuantKVCache(B, H, S, K.KVQ_MODE_CHUNK_MIXED, page_tokens=P, num_pages=pool,
                               block_table=i32_device(tables.reshape(-1)), **kw)
        return paged, K.QuantKVCache(B, H, S, K.KVQ_MODE_CHUNK_MIXED, **kw)

    def compare(paged, flat, seg, L):
        n = L // CT
        for name in ("k", "v"):
            for c in range(3):
                for field, per in MIX_CLASS_BUFS[c]:
                    fl = host_bytes(flat.buf(name + "." + field)).view(np.uint8)[:B * H * S * per]
                    fl = fl.reshape(B, H, S, per)
                    for b in range(B):
                        rows = int(seg[b, c]) * CT
                        got = gather_class_rows(paged, name, field, per, pool, H, P, tables[c, b], S)
                        assert np.array_equal(got[:, :rows], fl[b, :, :rows]), (name, field, b, L)
                        if c == 0 and L > n * CT:  # the waiting tokens
                            w0 = S - CT
                            assert np.array_equal(got[:, w0:w0 + L - n * CT], fl[b, :, w0:w0 + L - n * CT]), \
                                (name, b, L)

    def decode_both(paged, flat, lens, ns):
        out_p = decode_mixed(paged, q, H * G, lens, ns)
        out_f = decode_mixed(flat, q, H * G, lens, ns)
        assert paged.flags() == 0 and flat.flags() == 0
        assert np.array_equal(out_p.view(np.uint32), out_f.view(np.uint32)), (lens, ns)
        return out_p

    # bulk: reorder, then quantize the whole sequence
    paged, flat = pair()
    for cache in (paged, flat):
        K.kvq_reorder_chunks(cache.desc, torch.from_numpy(bits).cuda(), C)
        K.kvq_quant_append(cache.desc, to_device(k), to_device(v), S, i32_device([0] * B))
    torch.cuda.synchronize()
    assert paged.flags() == 0 and flat.flags() == 0
    compare(paged, flat, seg_o, S)
    kh = {}
    for name, x in (("k", k), ("v", v)):
        ref = np.zeros((B, H, S, 128), np.float32)
        for b in range(B):
            for c in range(C):
                rows = x[b, :, c * CT:(c + 1) * CT]
                if bits[b, c] == 16:
                    ref[b, :, c * CT:(c + 1) * CT] = rows.view(np.float16).astype(np.float32)
                else:
                    oc, os_, oz = oracle.quant_rows(rows, group, 4 if bits[b, c] == 4 else 2)
                    ref[b, :, c * CT:(c + 1) * CT] = oracle.dequant_rows(oc, os_, oz, group)
        kh[name] = ref
    refs = np.stack([oracle.attention(q[b], kh["k"][b], kh["v"][b], SM) for b in range(B)])
    for ns in (0, 1, 5):
        out = decode_both(paged, flat, None, ns)
        err = float(rel_err_rows(out, refs).max())
        print("paged mixed bulk P%d CT%d G%d ns%d: max rel err %.3e" % (P, CT, G, ns, err), flush=True)
        assert err <= ATTN_BAR and err <= ATTN_TIGHT

    # streaming: chunks join their class pools as appends complete them
    paged, flat = pair()
    L = 0
    for step in (45, 1, 30, 100, 1, 70, 265):
        done0 = L // CT
        n_new = -(-step // CT) + 1
        nb = np.full((B, n_new), 16, np.uint8)
        m = (L + step) // CT - done0
        nb[:, :m] = bits[:, done0:done0 + m]
        for cache in (paged, flat):
            K.kvq_append_chunks(cache.desc, to_device(np.ascontiguousarray(k[:, :, L:L + step])),
                                to_device(np.ascontiguousarray(v[:, :, L:L + step])), step, i32_device([L] * B),
                                torch.from_numpy(nb).cuda(), n_new)
        L += step
        torch.cuda.synchronize()
        assert paged.flags() == 0 and flat.flags() == 0
        seg = host_bytes(flat.buf("seg")).reshape(B, 4)
        assert np.array_equal(host_bytes(paged.buf("seg")).reshape(B, 4), seg)
        compare(paged, flat, seg, L)
        if step in (1, 70, 265):
            for ns in (0, 3):
                decode_both(paged, flat, [L] * B, ns)
    assert L == S


def decode_mixed(cache, q, Hq, lens, ns):
    B = q.shape[0]
    S = cache.desc.max_seq
    out = torch.full((B, Hq, 128), float("nan"), dtype=torch.float32, device="cuda")
    ws, n = cache.workspace(Hq, S, ns)
    K.kvq_decode_attn(cache.desc, to_device(q), Hq, None if lens is None else i32_device(lens), S, SM, out, ws, n,
                      ns)
    torch.cuda.synchronize()
    return out.cpu().numpy()
