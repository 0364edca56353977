"""HIP path vs the fp64 oracle, element by element, through the C ABI."""
import math

import numpy as np
import pytest

import oracle
from causal_gqa_prefill_amd import inputs
from causal_gqa_prefill_amd.configs import CONFIGS

from gpu_util import compare, from_dev_bf16, run_gpu, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from causal_gqa_prefill_amd import binding
    binding.library()  # raises if the HIP library is missing: no fallback


def _check_case(B, L, n_q, n_kv, d, causal, scale, seed, rows=None, name=None):
    name = name or f"B={B} L={L} n_q={n_q} n_kv={n_kv} d={d} causal={causal} scale={scale:.4g}"
    say(f"case {name}")
    qb, kb, vb = inputs.make_qkv(B, L, n_q, n_kv, d, seed)
    o, l = run_gpu(qb, kb, vb, scale, causal)
    ref_o, ref_l, _ = oracle.attention_rows(qb, kb, vb, scale, causal, rows=rows)
    o = o.reshape(-1, d)
    l = l.reshape(-1)
    if rows is not None:
        o, l = o[rows], l[rows]
    compare(name, o, l, ref_o, ref_l)


# ---------------------------------------------------------------------------
# the five workloads: every row for configs 1-3, 4096 seeded rows for 4-5
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("cfg", CONFIGS, ids=[f"config{c.index}" for c in CONFIGS])
def test_config_parity(cfg):
    say(f"config {cfg.index}: {cfg.describe()}")
    qb, kb, vb = inputs.make_config_qkv(cfg)
    o, l = run_gpu(qb, kb, vb, cfg.scale, cfg.causal)
    o = o.reshape(-1, cfg.d_h)
    l = l.reshape(-1)
    if cfg.sampled_rows:
        rows = inputs.sample_rows(cfg.B, cfg.n_q, cfg.L, cfg.sampled_rows, cfg.seed)
        ref_o, ref_l, _ = oracle.attention_rows(qb, kb, vb, cfg.scale, cfg.causal, rows=rows)
        compare(f"config{cfg.index} sampled", o[rows], l[rows], ref_o, ref_l)
    else:
        # every row, one head-chunk at a time so progress shows
        total = cfg.B * cfg.n_q * cfg.L
        chunk = max(cfg.L, total // 8)
        for r0 in range(0, total, chunk):
            rows = np.arange(r0, min(total, r0 + chunk), dtype=np.int64)
            ref_o, ref_l, _ = oracle.attention_rows(qb, kb, vb, cfg.scale, cfg.causal, rows=rows)
            compare(f"config{cfg.index} rows {r0}..{rows[-1]}", o[rows], l[rows], ref_o, ref_l)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(l))


# ---------------------------------------------------------------------------
# the persistent schedule: far more work items than CUs, so every
# workgroup walks several items back to back and the K/V ring runs across
# item boundaries (items of 1 to 11 tiles, next-item tiles requested by the
# last tile steps or after them, short items whose successor's first tiles
# all come after the loop); every row against the oracle
# ---------------------------------------------------------------------------
MANY_ITEMS = [
    # B, L, n_q, n_kv, d, causal: items = B * n_kv * (g / HWG) * ceil(L / BR)
    (160, 260, 8, 1, 128, 1),    # 1440 items of 1..5 tiles (32-row q-blocks)
    (300, 64, 1, 1, 128, 1),     # 300 one-tile items (256-row q-blocks, MHA)
    (64, 700, 2, 1, 64, 1),      # 384 items of 1..11 tiles, d_h = 64
    (96, 300, 4, 2, 128, 0),     # 576 non-causal items of 5 tiles each (last step loads the
                                 # staging slot: the barrier before the output staging)
    (40, 130, 12, 4, 128, 1),    # g = 3 (one head per item): 480 items of 3 tiles
]


@pytest.mark.parametrize("B,L,n_q,n_kv,d,causal", MANY_ITEMS)
def test_many_items_per_workgroup(B, L, n_q, n_kv, d, causal):
    scale = float(np.float32(1.0 / np.sqrt(d)))
    _check_case(B, L, n_q, n_kv, d, causal, scale, seed=4000 + B + L,
                name=f"many items B={B} L={L} n_q={n_q} n_kv={n_kv} d={d} causal={causal}")


# Stream blocks (on a 256-CU grid): short sequences put every q-block of a
# head on one XCD in the same round (1, 2 and 4 heads per XCD and round,
# several rounds); very long ones give each XCD runs of adjacent q-blocks of
# one or two (batch, kv-head) streams, cut into super-groups of 10 q-blocks
# for g = 6 (the last one partial here).  One seeded row of every 32-row
# block of every head is checked, so every work item is.
STREAM_BLOCKS = [
    # B, L, n_q, n_kv, d, causal
    (8, 2048, 32, 8, 128, 1),    # GQA-4, 32 q-blocks of 64 rows: 1 head per XCD, 8 rounds
    (16, 1024, 32, 8, 64, 1),    # 16 q-blocks: 2 heads per XCD, 8 rounds, d_h = 64
    (8, 2048, 16, 16, 128, 1),   # MHA, 8 q-blocks of 256 rows: 4 heads per XCD, 8 rounds
    (4, 2048, 16, 16, 128, 0),   # non-causal: 4 heads per XCD, 2 rounds
    (1, 82560, 24, 4, 128, 1),   # GQA-6, 645 q-blocks: 64 super-groups of 10 and one of 5
]


@pytest.mark.parametrize("B,L,n_q,n_kv,d,causal", STREAM_BLOCKS)
def test_stream_block_item_order(B, L, n_q, n_kv, d, causal):
    scale = float(np.float32(1.0 / np.sqrt(d)))
    rng = np.random.default_rng(4500 + B + L)
    blocks = np.arange(0, B * n_q * L, 32, dtype=np.int64)
    rows = blocks + rng.integers(0, 32, size=blocks.size)
    _check_case(B, L, n_q, n_kv, d, causal, scale, seed=4500 + B + L, rows=rows,
                name=f"stream blocks B={B} L={L} n_q={n_q} n_kv={n_kv} d={d} causal={causal}")


# ---------------------------------------------------------------------------
# edge shapes: ragged L, every GQA ratio class, both head sizes, B > 1,
# non-causal, scales other than 1/sqrt(d)
# ---------------------------------------------------------------------------
EDGE = [
    # B, L, n_q, n_kv, d, causal, scale
    (1, 1, 4, 4, 64, 1, None),
    (1, 2, 8, 2, 128, 1, None),
    (1, 15, 6, 1, 128, 1, None),
    (1, 63, 4, 1, 64, 1, None),
    (1, 64, 8, 8, 128, 1, None),
    (1, 65, 16, 2, 128, 1, None),
    (3, 127, 4, 2, 64, 1, None),
    (1, 129, 12, 2, 128, 1, None),
    (2, 257, 3, 1, 128, 1, None),
    (1, 1000, 8, 1, 128, 1, None),
    (1, 4097, 6, 6, 64, 1, None),
    (1, 1, 2, 1, 128, 0, None),
    (1, 65, 8, 2, 64, 0, None),
    (2, 300, 4, 4, 128, 0, None),
    (1, 777, 16, 4, 128, 0, 0.3),
    (1, 200, 4, 2, 128, 1, 0.5),
    (1, 200, 4, 2, 64, 1, 0.0),
    (1, 200, 4, 2, 128, 1, -0.0883883),
    (1, 130, 5, 5, 128, 1, None),
    (1, 96, 24, 3, 64, 1, None),
]


@pytest.mark.parametrize("B,L,n_q,n_kv,d,causal,scale", EDGE)
def test_edge_shapes(B, L, n_q, n_kv, d, causal, scale):
    if scale is None:
        scale = float(np.float32(1.0 / math.sqrt(d)))
    _check_case(B, L, n_q, n_kv, d, causal, scale, seed=2000 + L + 7 * n_q + d)


# ---------------------------------------------------------------------------
# closed forms on the GPU
# ---------------------------------------------------------------------------
def test_constant_v_gpu():
    B, L, n_q, n_kv, d = 1, 300, 8, 2, 128
    qb, kb, _ = inputs.make_qkv(B, L, n_q, n_kv, d, seed=31)
    c = np.zeros((B, n_kv, L, d), dtype=np.float32)
    c[:, 0] = 1.5
    c[:, 1] = -0.75
    vb = inputs.bf16_bits(c)
    o, l = run_gpu(qb, kb, vb, 0.088, True)
    want = np.where(np.arange(n_q) // 4 == 0, 1.5, -0.75)[None, :, None, None]
    assert np.max(np.abs(o - want)) <= 1e-2


def test_zero_query_gpu():
    B, L, n_q, n_kv, d = 1, 500, 4, 1, 64
    _, kb, vb = inputs.make_qkv(B, L, n_q, n_kv, d, seed=32)
    qb = np.zeros((B, n_q, L, d), dtype=np.uint16)
    o, l = run_gpu(qb, kb, vb, 0.125, True)
    vv = inputs.bf16_to_f32(vb)[0, 0].astype(np.float64)
    means = np.cumsum(vv, axis=0) / np.arange(1, L + 1)[:, None]
    assert np.max(np.abs(o[0] - means[None])) <= 1e-2
    assert np.max(np.abs(l[0] - np.log(np.arange(1, L + 1))[None])) <= 1e-3


def test_first_row_is_v0_gpu():
    B, L, n_q, n_kv, d = 2, 130, 4, 2, 128
    qb, kb, vb = inputs.make_qkv(B, L, n_q, n_kv, d, seed=33)
    o, _ = run_gpu(qb, kb, vb, 0.088, True)
    vv = inputs.bf16_to_f32(vb).astype(np.float64)
    for h in range(n_q):
        assert np.array_equal(o[:, h, 0], vv[:, h // 2, 0])  # P = 1 exactly


def test_gqa_equals_repeated_kv_gpu():
    B, L, n_q, n_kv, d = 1, 333, 8, 2, 128
    qb, kb, vb = inputs.make_qkv(B, L, n_q, n_kv, d, seed=34)
    og, lg = run_gpu(qb, kb, vb, 0.088, True)
    kr = np.ascontiguousarray(np.repeat(kb, 4, axis=1))
    vr = np.ascontiguousarray(np.repeat(vb, 4, axis=1))
    om, lm = run_gpu(qb, kr, vr, 0.088, True)
    assert np.max(np.abs(og - om)) <= 1e-2 and np.max(np.abs(lg - lm)) <= 1e-4


def test_large_scores_gpu():
    # Q x 20: scores beyond 150 must not overflow the softmax
    B, L, n_q, n_kv, d = 1, 512, 4, 2, 128
    qb, kb, vb = inputs.make_qkv(B, L, n_q, n_kv, d, seed=35)
    qb = inputs.bf16_bits(inputs.bf16_to_f32(qb) * np.float32(20.0))
    scale = float(np.float32(1 / math.sqrt(d)))
    o, l = run_gpu(qb, kb, vb, scale, True)
    ref_o, ref_l, _ = oracle.attention_rows(qb, kb, vb, scale, True)
    compare("large scores", o.reshape(-1, d), l.reshape(-1), ref_o, ref_l)


# ---------------------------------------------------------------------------
# robustness: determinism, streams, argument errors
# ---------------------------------------------------------------------------
def test_bitwise_deterministic():
    import torch
    from causal_gqa_prefill_amd import attn_prefill
    qb, kb, vb = inputs.make_qkv(1, 1000, 8, 2, 128, seed=36)
    q, k, v = to_dev(qb), to_dev(kb), to_dev(vb)
    outs = [attn_prefill(q, k, v) for _ in range(3)]
    torch.cuda.synchronize()
    for o, l in outs[1:]:
        assert torch.equal(o.view(torch.int16), outs[0][0].view(torch.int16))
        assert torch.equal(l, outs[0][1])


def test_non_default_stream():
    import torch
    qb, kb, vb = inputs.make_qkv(1, 700, 4, 1, 128, seed=37)
    s = torch.cuda.Stream()
    o, l = run_gpu(qb, kb, vb, 0.088, True, stream=s)
    ref_o, ref_l, _ = oracle.attention_rows(qb, kb, vb, 0.088, True)
    compare("side stream", o.reshape(-1, 128), l.reshape(-1), ref_o, ref_l)


def test_concurrent_calls_on_two_streams_from_two_threads():
    """Two calls in flight at once (two host threads, two streams, persistent
    grids competing for the same CUs, each schedule ending in a dynamic tail
    with a counter pair of its own) give the same bits as the calls run one
    after the other."""
    import threading
    import torch
    from causal_gqa_prefill_amd import attn_prefill_into
    # 4096 work items each on 256 CUs: 16 rounds, the last 5 of them handed
    # out through the counters
    shapes = [(1, 16384, 64, 8, 128, 1, 51), (16, 2048, 32, 32, 64, 1, 52)]
    runs = []
    for (B, L, n_q, n_kv, d, causal, seed) in shapes:
        qb, kb, vb = inputs.make_qkv(B, L, n_q, n_kv, d, seed)
        q, k, v = to_dev(qb), to_dev(kb), to_dev(vb)
        runs.append((q, k, v, causal))
    # one after the other
    ref = []
    for (q, k, v, causal) in runs:
        out = torch.empty_like(q)
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
        attn_prefill_into(q, k, v, out, lse, causal=bool(causal))
        torch.cuda.synchronize()
        ref.append((out.clone(), lse.clone()))
    # both in flight: each thread launches 5 calls on its own stream
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [(torch.full_like(q, float("nan")),
             torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device=q.device))
            for (q, k, v, causal) in runs]
    torch.cuda.synchronize()
    errors = []

    def work(i):
        try:
            q, k, v, causal = runs[i]
            for _ in range(5):
                attn_prefill_into(q, k, v, outs[i][0], outs[i][1], causal=bool(causal),
                                  stream=streams[i])
        except Exception as e:  # reported after the join
            errors.append(e)

    threads = [threading.Thread(target=work, args=(i,)) for i in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for i in range(2):
        same_o = torch.equal(outs[i][0].view(torch.int16), ref[i][0].view(torch.int16))
        same_l = torch.equal(outs[i][1].view(torch.int32), ref[i][1].view(torch.int32))
        say(f"  concurrent call {i}: output bits equal {same_o}, lse bits equal {same_l}")
        assert same_o and same_l


# shapes whose schedules end in a dynamic tail on 256 CUs (at least 16
# rounds; items, rounds): GQA-8 at 16K (4096, 16), MHA at 2K with 16
# sequences (4096, 16), non-causal GQA-8 (4096, 16), a ragged GQA-6 sequence
# with 64-wide heads (5778, 23: a partial last round)
DYN_TAIL = [
    (1, 16384, 64, 8, 128, 1),
    (16, 2048, 32, 32, 64, 1),
    (4, 4096, 64, 8, 64, 0),
    (1, 41000, 36, 6, 64, 1),
]


@pytest.mark.parametrize("B,L,n_q,n_kv,d,causal", DYN_TAIL)
def test_dynamic_tail_computes_every_item_once(B, L, n_q, n_kv, d, causal):
    """Outputs poisoned with NaN, two calls in a row: every row of both is
    written (an item the counter skipped would leave NaN; a counter pair not
    set back to zero would make the second call skip its whole tail), both
    calls give the same bits, and one seeded row of every 32-row block
    matches the oracle."""
    import torch
    from causal_gqa_prefill_amd import attn_prefill_into
    say(f"case dynamic tail B={B} L={L} n_q={n_q} n_kv={n_kv} d={d} causal={causal}")
    scale = float(np.float32(1.0 / math.sqrt(d)))
    qb, kb, vb = inputs.make_qkv(B, L, n_q, n_kv, d, seed=7000 + L + n_q)
    q, k, v = to_dev(qb), to_dev(kb), to_dev(vb)
    res = []
    for _ in range(2):
        out = torch.full_like(q, float("nan"))
        lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device=q.device)
        attn_prefill_into(q, k, v, out, lse, scale=scale, causal=bool(causal))
        torch.cuda.synchronize()
        assert bool(torch.all(torch.isfinite(out.float()))), "an output row was not written"
        assert bool(torch.all(torch.isfinite(lse))), "an lse entry was not written"
        res.append((out, lse))
    assert torch.equal(res[0][0].view(torch.int16), res[1][0].view(torch.int16))
    assert torch.equal(res[0][1].view(torch.int32), res[1][1].view(torch.int32))
    o = from_dev_bf16(res[0][0]).reshape(-1, d)
    l = res[0][1].cpu().numpy().astype(np.float64).reshape(-1)
    rng = np.random.default_rng(L)
    blocks = np.arange(0, B * n_q * L, 32, dtype=np.int64)
    rows = blocks + (rng.random(blocks.size) * np.minimum(32, B * n_q * L - blocks)).astype(np.int64)
    ref_o, ref_l, _ = oracle.attention_rows(qb, kb, vb, scale, causal, rows=rows)
    compare(f"dynamic tail L={L}", o[rows], l[rows], ref_o, ref_l)


def test_graph_capture_takes_the_static_schedule():
    """A call captured into a graph runs without a counter (the static
    schedule); each replay, with eager calls (which do use counters) between
    the replays, gives the eager call's bits."""
    import torch
    from causal_gqa_prefill_amd import attn_prefill_into
    B, L, n_q, n_kv, d = 1, 16384, 64, 8, 128   # 16 rounds: a dynamic tail when eager
    qb, kb, vb = inputs.make_qkv(B, L, n_q, n_kv, d, seed=7100)
    q, k, v = to_dev(qb), to_dev(kb), to_dev(vb)
    ref_o = torch.empty_like(q)
    ref_l = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    attn_prefill_into(q, k, v, ref_o, ref_l)
    torch.cuda.synchronize()
    out = torch.full_like(q, float("nan"))
    lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device=q.device)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # one eager call on the capture stream first
        attn_prefill_into(q, k, v, out, lse)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        attn_prefill_into(q, k, v, out, lse)
    for rep in range(3):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        same = (torch.equal(out.view(torch.int16), ref_o.view(torch.int16)) and
                torch.equal(lse.view(torch.int32), ref_l.view(torch.int32)))
        say(f"  replay {rep}: bits equal to the eager call {same}")
        assert same
        eo = torch.empty_like(q)
        el = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
        attn_prefill_into(q, k, v, eo, el)   # an eager call between replays
        torch.cuda.synchronize()
        assert torch.equal(eo.view(torch.int16), ref_o.view(torch.int16))


def test_argument_errors_raise():
    import torch
    from causal_gqa_prefill_amd import AttnPrefillError, attn_prefill
    q = torch.zeros((1, 6, 64, 128), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((1, 4, 64, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(AttnPrefillError):
        attn_prefill(q, k, k.clone())  # 6 % 4 != 0
    q = torch.zeros((1, 4, 64, 96), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(AttnPrefillError):
        attn_prefill(q, q.clone(), q.clone())  # d_h = 96
    with pytest.raises(TypeError):
        attn_prefill(q.float(), q.float(), q.float())
