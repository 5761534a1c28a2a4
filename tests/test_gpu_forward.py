"""GPU parity of the forward path (route, permute, grouped FFN, combine, bias
update, whole layer) against the oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import as_f64, check_close, check_permute, check_route, dev, host, say
from workloads import CONFIGS, make_inputs, scaled

pytestmark = pytest.mark.gpu

L = None


def setup_module():
    global L
    from mixture_experts_layer_free_amd import _lib
    L = _lib
    L.lib()
    assert torch.cuda.is_available()


def _kind(cfg):
    return "bf16" if cfg.dtype == "bf16" else "f32"


def _route_case(cfg, inp, score=None, bias=True, offset=True):
    score = score or cfg.score
    b = inp["bias"] if bias else None
    o = inp["logit_offset"] if offset else None
    x = dev(inp["x"])
    idx, gate, logits = L.moe_route(x, dev(inp["w_router"]), cfg.k, score, dev(o), dev(b))
    torch.cuda.synchronize()
    ref = oracle.route(inp["x"], inp["w_router"], cfg.k, score, b, o)
    return check_route(host(idx), host(gate), host(logits), ref, cfg.k), idx, x


# ---------------------------------------------------------------------------- route

@pytest.mark.parametrize("score", oracle.SCORE_FNS)
def test_route_tiny(score):
    cfg = CONFIGS["tiny"]
    say(f"[route tiny {score}]")
    inp = make_inputs(cfg)
    inp["logit_offset"] = np.random.default_rng(5).uniform(-0.3, 0.3, cfg.E).astype(np.float32)
    for k in (1, 2, 5, 8):
        excl, _, _ = _route_case(scaled(cfg, k=k), inp, score)
        assert excl == 0


@pytest.mark.parametrize("T,d,E,k", [(300, 256, 16, 4), (77, 64, 1, 1), (129, 128, 96, 16), (64, 2048, 1024, 16),
                                     (33, 64, 16, 16), (150, 200, 12, 3), (150, 200, 40, 5), (2100, 1032, 8, 2),
                                     (40, 8, 17, 2),
                                     # >= 256 tiles of 64 x 64: the LDS-shared router, ragged T, E and d
                                     (16383, 200, 100, 5), (4100, 72, 300, 8)])
def test_route_shapes(T, d, E, k):
    say(f"[route shape T={T} d={d} E={E} k={k}]")
    cfg = scaled(CONFIGS["fine"], T=T, d=d, E=E, k=k, f=64, bias="uniform")
    inp = make_inputs(cfg, experts=False)
    for score in oracle.SCORE_FNS:
        _route_case(cfg, inp, score)


def test_route_ties_go_to_lower_index():
    say("[route ties]")
    T, d, E = 64, 64, 12
    r = np.random.default_rng(0)
    x = r.standard_normal((T, d)).astype(np.float32)
    w = (r.standard_normal((E, d)) * 0.1).astype(np.float32)
    w[2] = w[7] = w[11] = 1.0          # three identical, strong router rows
    bias = np.zeros(E, np.float32)
    idx, gate, logits = L.moe_route(dev(x), dev(w), 2, "softmax", None, dev(bias))
    idx = host(idx)
    ref = oracle.route(x, w, 2, "softmax", bias)
    assert np.array_equal(idx, ref["idx"])
    strong = x.sum(axis=1) > 1.0
    assert np.all(idx[strong] == np.array([2, 7]))


@pytest.mark.parametrize("E", [64, 40, 17, 100])
def test_route_all_keys_equal(E):
    """Zero input rows give every expert the same key: the choice is experts
    0..k-1 in index order with equal gates (the tie rule read into the
    lesson's Build it step 1: lower index first), both on the one-key-per-lane
    path (E <= 64) and on the argmax rounds (E > 64); the other rows follow
    the oracle."""
    say(f"[route all keys equal E={E}]")
    T, d, k = 96, 64, 8
    r = np.random.default_rng(E)
    x = r.standard_normal((T, d)).astype(np.float32)
    x[::2] = 0.0
    w = (r.standard_normal((E, d)) * 0.1).astype(np.float32)
    for score in oracle.SCORE_FNS:
        idx, gate, logits = L.moe_route(dev(x), dev(w), k, score, None, None)
        idx, gate = host(idx), host(gate)
        assert np.all(idx[::2] == np.arange(k)), score
        assert np.allclose(gate[::2], 1.0 / k, rtol=0, atol=1e-7), score
        ref = oracle.route(x, w, k, score)
        check_route(idx, gate, host(logits), ref, k)


def test_route_fp32_not_bf16_winner():
    """fp32-distinct, bf16-equal router rows: the GPU router picks the true
    winner, which a bf16 router would not."""
    say("[route bf16 counterexample]")
    d, E = 8, 4
    x = np.zeros((4, d), np.float32)
    x[:, 0] = 1.0
    w = np.zeros((E, d), np.float32)
    w[0, 0] = 1.0
    w[1, 0] = np.float32(1.0 + 2.0 ** -9)
    w[2, 0] = 0.5
    w[3, 0] = -1.0
    idx, _, logits = L.moe_route(dev(x), dev(w), 1, "softmax")
    assert np.all(host(idx)[:, 0] == 1)
    assert oracle.bf16_round(float(w[1, 0])) == oracle.bf16_round(float(w[0, 0]))


@pytest.mark.parametrize("name", ["coarse", "fine", "dsv3", "train"])
def test_route_full_size(name):
    cfg = CONFIGS[name]
    say(f"[route full {name} T={cfg.T} d={cfg.d} E={cfg.E} k={cfg.k}]")
    inp = make_inputs(cfg, experts=False)
    excl, idx, x = _route_case(cfg, inp)
    assert excl <= 10


@pytest.mark.parametrize("T,E,k,salt", [(1000, 64, 8, 0), (333, 1024, 16, 7), (77, 3, 3, 1), (4096, 256, 8, 2)])
def test_route_hash(T, E, k, salt):
    """Hash router: bit-exact expert choice (integer hashing), gates exactly 1/k."""
    say(f"[route hash T={T} E={E} k={k} salt={salt}]")
    ids = np.random.default_rng(T).integers(-2 ** 31, 2 ** 31 - 1, T).astype(np.int32)
    idx, gate = L.moe_route_hash(dev(ids), E, k, salt)
    torch.cuda.synchronize()
    ref = oracle.hash_route(ids, E, k, salt)
    assert np.array_equal(host(idx), ref["idx"])
    assert np.all(host(gate) == np.float32(1.0 / k))


@pytest.mark.parametrize("score", oracle.SCORE_FNS)
def test_route_replay(score):
    """Routing replay: the gates of moe_route's own choice are reproduced bit for
    bit; a foreign choice gets the oracle's gates for that choice."""
    say(f"[route replay {score}]")
    cfg = scaled(CONFIGS["fine"], T=300, d=256, E=40, k=6, f=64, score=score, bias="uniform")
    inp = make_inputs(cfg)
    x, w, off = dev(inp["x"]), dev(inp["w_router"]), dev(inp["logit_offset"])
    idx, gate, logits = L.moe_route(x, w, cfg.k, score, off, dev(inp["bias"]))
    g2, l2 = L.moe_route_replay(x, w, idx, score, off)
    torch.cuda.synchronize()
    assert np.array_equal(host(g2), host(gate)) and np.array_equal(host(l2), host(logits))
    rng = np.random.default_rng(3)
    ridx = np.stack([rng.permutation(cfg.E)[:cfg.k] for _ in range(cfg.T)])
    g3, _ = L.moe_route_replay(x, w, dev(ridx.astype(np.int32)), score, off)
    torch.cuda.synchronize()
    ref = oracle.forward(inp["x"], inp["w_router"], inp["w_gate_up"], inp["w_down"], cfg.k, score, True,
                         logit_offset=inp["logit_offset"], idx=ridx)
    check_close(host(g3), ref["gates"], "f32", "replayed gates")


@pytest.mark.parametrize("score", oracle.SCORE_FNS)
def test_route_fewer_experts_at_serving(score):
    """k is a per-call argument: serving with k' < k picks the first k' of the k
    experts and renormalises their gates."""
    say(f"[route runtime k {score}]")
    cfg = scaled(CONFIGS["fine"], T=500, d=128, E=64, k=8, f=64, score=score, bias="uniform")
    inp = make_inputs(cfg, experts=False)
    x, w, off, b = dev(inp["x"]), dev(inp["w_router"]), dev(inp["logit_offset"]), dev(inp["bias"])
    i8, g8, _ = L.moe_route(x, w, 8, score, off, b)
    for k in (1, 3, 5):
        ik, gk, lk = L.moe_route(x, w, k, score, off, b)
        torch.cuda.synchronize()
        check_route(host(ik), host(gk), host(lk), oracle.route(inp["x"], inp["w_router"], k, score, inp["bias"],
                                                               inp["logit_offset"]), k)
        assert np.array_equal(host(ik), host(i8)[:, :k])      # same keys, same first k rounds
        pre = host(g8)[:, :k].astype(np.float64)
        np.testing.assert_allclose(host(gk), pre / pre.sum(1, keepdims=True), rtol=2e-6, atol=1e-7)


@pytest.mark.parametrize("T,E,k,score", [(300, 40, 6, "softmax"), (16384, 64, 8, "sqrt_softplus"),
                                         (4096, 256, 8, "sigmoid"), (64, 1024, 16, "softmax"), (4096, 8, 2, "softmax"),
                                         (513, 17, 3, "sigmoid")])
def test_aux_loss(T, E, k, score):
    """Auxiliary load-balancing loss and the mean router probabilities against
    the oracle's own fp64 logits; the counts are the GPU's integer counts,
    which equal the oracle's wherever no token is a near-tie (fixed-order
    reductions: also bit-reproducible run to run)."""
    say(f"[aux loss T={T} E={E} k={k} {score}]")
    cfg = scaled(CONFIGS["fine"], T=T, d=64, E=E, k=k, f=64, score=score, bias="uniform")
    inp = make_inputs(cfg, experts=False)
    x = dev(inp["x"])
    idx, gate, logits = L.moe_route(x, dev(inp["w_router"]), k, score, dev(inp["logit_offset"]), dev(inp["bias"]))
    counts = L.moe_permute(idx, x, E)[0]
    p_mean = torch.empty(E, dtype=torch.float32, device="cuda")
    loss = L.moe_aux_loss(logits, counts, k, score, 0.01, p_mean_out=p_mean)
    loss2 = L.moe_aux_loss(logits, counts, k, score, 0.01)
    torch.cuda.synchronize()
    ref = oracle.route(inp["x"], inp["w_router"], k, score, inp["bias"], inp["logit_offset"])
    lg = ref["logits"]
    if np.all(ref["margin"] >= 1e-6):
        assert np.array_equal(host(counts), oracle.permute(ref["idx"], E)[0])
    want = oracle.aux_loss(lg, host(counts), k, score, 0.01)
    assert abs(float(host(loss)[0]) - want) <= 1e-5 * abs(want), (float(host(loss)[0]), want)
    check_close(host(p_mean), oracle.aux_probs(lg, score).mean(axis=0), "f32", "P")
    assert host(loss)[0] == host(loss2)[0]


# ---------------------------------------------------------------------------- permute

def _permute_case(idx_np, x_np, E):
    idx = dev(idx_np.astype(np.int32))
    x = dev(x_np)
    counts, offsets, row_of, token_of, x_perm = L.moe_permute(idx, x, E)
    torch.cuda.synchronize()
    check_permute(idx_np, E, host(counts), host(offsets), host(row_of), host(token_of), host(x_perm), x_np)


@pytest.mark.parametrize("T,E,k,d", [(1, 4, 2, 8), (255, 8, 2, 64), (257, 64, 8, 128), (1000, 37, 3, 32),
                                     (4096, 1024, 16, 16), (513, 1, 1, 24)])
def test_permute_random(T, E, k, d):
    say(f"[permute T={T} E={E} k={k} d={d}]")
    rng = np.random.default_rng(T + E)
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)])
    x = rng.standard_normal((T, d)).astype(np.float32)
    _permute_case(idx, x, E)
    xb = (rng.integers(0, 65535, (T, d * 2))).astype(np.uint16)  # bf16 bit patterns, even d for 16-byte rows
    _permute_case(idx, xb, E)


def test_permute_skew_extremes():
    say("[permute skew]")
    T, E, d = 3000, 16, 64
    x = np.random.default_rng(1).standard_normal((T, d)).astype(np.float32)
    _permute_case(np.full((T, 1), 5), x, E)                        # everything on expert 5
    _permute_case(np.tile(np.array([[15, 0]]), (T, 1)), x, E)      # two experts, rest empty
    _permute_case(np.tile(np.arange(E)[::-1], (T, 1)), x, E)       # k = E


@pytest.mark.parametrize("T,E,k,d,skew", [(300, 8, 2, 64, 0.0), (1000, 37, 3, 32, 0.5), (2049, 64, 8, 128, 0.2),
                                          (700, 16, 16, 16, 0.0), (513, 1, 1, 24, 0.0)])
def test_permute_capacity(T, E, k, d, skew):
    """Expert capacity: kept rows first (offsets), dropped rows after them, row_of = ~row
    for a dropped assignment; bit-exact against the oracle for several caps."""
    say(f"[permute capacity T={T} E={E} k={k} d={d} skew={skew}]")
    rng = np.random.default_rng(T + 7 * E)
    p = np.exp(-skew * np.arange(E))
    p /= p.sum()
    idx = np.stack([rng.choice(E, k, replace=False, p=p) for _ in range(T)])
    x = (rng.integers(0, 65535, (T, d))).astype(np.uint16)
    A = T * k
    for cap in (0, 1, max(1, A // E // 2), A // E, 2 * A // E, A, -1):
        counts, offsets, row_of, token_of, x_perm = L.moe_permute_capacity(dev(idx.astype(np.int32)), dev(x), E, cap)
        torch.cuda.synchronize()
        check_permute(idx, E, host(counts), host(offsets), host(row_of), host(token_of), host(x_perm), x,
                      capacity=cap)


def test_permute_capacity_full_size():
    """The 64-expert forward shape with its Zipf-skewed load at capacity factor 1.0."""
    from mixture_experts_layer_free_amd.layer import expert_capacity
    cfg = CONFIGS["fine"]
    say("[permute capacity full fine]")
    inp = make_inputs(cfg, experts=False)
    ref = oracle.route(inp["x"], inp["w_router"], cfg.k, cfg.score, inp["bias"], inp["logit_offset"])
    idx = ref["idx"]
    cap = expert_capacity(1.0, cfg.T, cfg.k, cfg.E)
    counts, offsets, row_of, token_of, x_perm = L.moe_permute_capacity(dev(idx.astype(np.int32)), dev(inp["x"]),
                                                                       cfg.E, cap)
    torch.cuda.synchronize()
    assert int(host(offsets)[-1]) < cfg.T * cfg.k          # the skew makes some experts overflow
    check_permute(idx, cfg.E, host(counts), host(offsets), host(row_of), host(token_of), host(x_perm), inp["x"],
                  capacity=cap)


@pytest.mark.parametrize("name", ["coarse", "fine", "dsv3", "train"])
def test_permute_full_size(name):
    cfg = CONFIGS[name]
    say(f"[permute full {name}]")
    inp = make_inputs(cfg, experts=False)
    x = dev(inp["x"])
    idx, _, _ = L.moe_route(x, dev(inp["w_router"]), cfg.k, cfg.score, dev(inp["logit_offset"]), dev(inp["bias"]))
    counts, offsets, row_of, token_of, x_perm = L.moe_permute(idx, x, cfg.E)
    torch.cuda.synchronize()
    check_permute(host(idx), cfg.E, host(counts), host(offsets), host(row_of), host(token_of), host(x_perm), inp["x"])
    c = host(counts)
    say(f"  load max/mean {c.max() / c.mean():.2f} min/mean {c.min() / c.mean():.2f}")


# ---------------------------------------------------------------------------- grouped FFN

def _ffn_case(cfg, offsets_np, x_rows_np, wgu_np, wd_np, rows_to_check=None, save_gu=True):
    G = len(offsets_np) - 1
    gu, h, y = L.moe_grouped_ffn(dev(x_rows_np), dev(offsets_np.astype(np.int32)), dev(wgu_np), dev(wd_np),
                                 save_gu=save_gu)
    torch.cuda.synchronize()
    bf = cfg.dtype == "bf16"
    kind = _kind(cfg)
    f = wd_np.shape[2]
    rows = np.arange(x_rows_np.shape[0]) if rows_to_check is None else np.asarray(rows_to_check)
    grp = np.searchsorted(offsets_np, rows, side="right") - 1
    ref = {"G": [], "U": [], "H": [], "Y": []}
    for g in np.unique(grp):
        sel = rows[grp == g]
        o = oracle.expert_ffn(x_rows_np[sel], wgu_np[g], wd_np[g], bf)
        for key in ref:
            ref[key].append((sel, o[key]))
    def gather(key):
        out = np.zeros((len(rows), ref[key][0][1].shape[1]))
        pos = {r: i for i, r in enumerate(rows)}
        for sel, v in ref[key]:
            out[[pos[r] for r in sel]] = v
        return out
    check_close(host(y)[rows], gather("Y"), kind, "Y")
    check_close(host(h)[rows], gather("H"), kind, "H")
    if save_gu:
        g_ = host(gu)[rows]
        check_close(g_[:, :f], gather("G"), kind, "G")
        check_close(g_[:, f:], gather("U"), kind, "U")


def test_ffn_tiny_f32():
    cfg = CONFIGS["tiny"]
    say("[ffn tiny f32]")
    inp = make_inputs(cfg)
    offsets = np.array([0, 10, 10, 30, 31, 64, 64, 100, 128])
    x = np.random.default_rng(0).standard_normal((128, cfg.d)).astype(np.float32)
    _ffn_case(cfg, offsets, x, inp["w_gate_up"], inp["w_down"])


@pytest.mark.parametrize("d,f,seg", [# f not a multiple of 128: 128x128 tiles
                                     (128, 64, [0, 1, 129, 129, 300, 557]), (256, 192, [0, 0, 0, 1000]),
                                     # f a multiple of 128: 256x256 tiles; groups and ragged ends of at
                                     # most 128 rows run as 128x256 half tiles
                                     (192, 128, [0, 128, 256, 384]), (128, 128, [0, 300, 650, 1000]),
                                     (256, 256, [0, 600, 1300, 1301, 2600]), (384, 384, [0, 0, 2048, 2049, 2049])])
def test_ffn_bf16_tiles_and_tails(d, f, seg):
    say(f"[ffn bf16 d={d} f={f} seg={seg}]")
    G = len(seg) - 1
    cfg = scaled(CONFIGS["fine"], T=seg[-1], d=d, E=G, f=f, k=1)
    inp = make_inputs(cfg)
    _ffn_case(cfg, np.array(seg), inp["x"], inp["w_gate_up"], inp["w_down"])


@pytest.mark.parametrize("f", [64, 128])
def test_ffn_bf16_many_groups(f):
    """300 groups of 0..299 rows: 128x128 tiles (f = 64), and 256x256 tiles
    with most groups on 128x256 half tiles (f = 128)."""
    say(f"[ffn bf16 300 groups f={f}]")
    rng = np.random.default_rng(3)
    G, d = 300, 128
    n = rng.integers(0, 300, G)
    n[::7] = 0
    offsets = np.concatenate([[0], np.cumsum(n)])
    cfg = scaled(CONFIGS["dsv3"], T=int(offsets[-1]), d=d, E=G, f=f, k=1, shared=0)
    inp = make_inputs(cfg)
    check = np.unique(np.concatenate([offsets[:-1][n > 0], offsets[1:][n > 0] - 1, rng.integers(0, offsets[-1], 200)]))
    _ffn_case(cfg, offsets, inp["x"], inp["w_gate_up"], inp["w_down"], rows_to_check=check)


@pytest.mark.parametrize("T,d,E,k,f", [(300, 128, 8, 2, 64), (1500, 256, 4, 2, 256), (700, 192, 24, 3, 128),
                                       (64, 32, 8, 2, 64)])
def test_ffn_gather_equals_permuted_rows(T, d, E, k, f):
    """The fused permute: moe_grouped_ffn_gather on x through token_of gives
    bit for bit what moe_grouped_ffn gives on the copied X_perm, and both match
    the oracle's expert FFN on sampled rows (fp32 for the d = 32 case)."""
    say(f"[ffn gather T={T} d={d} E={E} k={k} f={f}]")
    base = CONFIGS["tiny"] if d == 32 else CONFIGS["fine"]
    cfg = scaled(base, T=T, d=d, E=E, k=k, f=f, bias="uniform", zipf_s=None)
    inp = make_inputs(cfg)
    x = dev(inp["x"])
    idx, _, _ = L.moe_route(x, dev(inp["w_router"]), cfg.k, cfg.score, sel_bias=dev(inp["bias"]))
    counts, offsets, row_of, token_of, x_perm = L.moe_permute(idx, x, cfg.E)
    c2, o2, r2, t2, none = L.moe_permute(idx, x, cfg.E, copy=False)
    torch.cuda.synchronize()
    assert none is None
    for u, v in ((counts, c2), (offsets, o2), (row_of, r2), (token_of, t2)):
        assert torch.equal(u, v)
    wgu, wd = dev(inp["w_gate_up"]), dev(inp["w_down"])
    g1, h1, y1 = L.moe_grouped_ffn(x_perm, offsets, wgu, wd, save_gu=True)
    g2, h2, y2 = L.moe_grouped_ffn_gather(x, token_of, offsets, wgu, wd, save_gu=True)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(h1, h2) and torch.equal(g1, g2)
    A = T * k
    rng = np.random.default_rng(2)
    rows = np.unique(np.concatenate([[0, A - 1], rng.integers(0, A, 48)]))
    off = host(offsets).astype(np.int64)
    grp = np.searchsorted(off, rows, side="right") - 1
    xp = host(x_perm)
    y = host(y2)
    ref = np.zeros((len(rows), d))
    for g in np.unique(grp):
        sel = grp == g
        ref[sel] = oracle.expert_ffn(xp[rows[sel]], inp["w_gate_up"][g], inp["w_down"][g], cfg.dtype == "bf16")["Y"]
    check_close(y[rows], ref, _kind(cfg), "Y (gathered)")


def test_ffn_gather_out_of_range_token_reads_zero():
    """A token index outside [0, T) reads as a zero row (bf16 and fp32),
    including indices whose byte offset is a multiple of 2^32 plus a valid
    row's offset (they must not wrap onto a row of x)."""
    for base in ("fine", "tiny"):
        d = 128 if base == "fine" else 32
        cfg = scaled(CONFIGS[base], T=200, d=d, E=2, k=1, f=64)
        inp = make_inputs(cfg)
        tok = np.arange(200, dtype=np.int32)
        wrap = (1 << 32) // (d * 2)                    # rows per 2^32 bytes of bf16 x
        bad = [3, 150, 151, 152, 153]
        tok[bad] = [-5, 1 << 20, wrap, wrap + 7, -(1 << 31)]
        offsets = np.array([0, 100, 200], np.int32)
        _, h, y = L.moe_grouped_ffn_gather(dev(inp["x"]), dev(tok), dev(offsets), dev(inp["w_gate_up"]),
                                           dev(inp["w_down"]))
        torch.cuda.synchronize()
        yh = host(y)
        assert np.all(yh[bad] == 0) and np.all(host(h).astype(np.float64)[bad] == 0)
        assert np.count_nonzero(yh[4]) > 0


@pytest.mark.parametrize("name", ["coarse", "fine", "dsv3"])
def test_ffn_full_size_every_expert(name):
    """The grouped FFN at full size in the layer's configuration (x gathered
    through token_of): the first and the last row of every expert against
    the oracle's expert FFN, so every expert's weights are checked."""
    cfg = CONFIGS[name]
    say(f"[ffn full size {name}: every expert's first and last row]")
    inp = make_inputs(cfg)
    x = dev(inp["x"])
    idx, _, _ = L.moe_route(x, dev(inp["w_router"]), cfg.k, cfg.score, dev(inp["logit_offset"]), dev(inp["bias"]))
    _, offsets, _, token_of, _ = L.moe_permute(idx, x, cfg.E, copy=False)
    wgu, wd = dev(inp["w_gate_up"]), dev(inp["w_down"])
    _, h, y = L.moe_grouped_ffn_gather(x, token_of, offsets, wgu, wd)
    torch.cuda.synchronize()
    off, tok = host(offsets).astype(np.int64), host(token_of)
    del wgu, wd, h
    rows, exps = [], []
    for e in range(cfg.E):
        ends = sorted({int(off[e]), int(off[e + 1] - 1)}) if off[e + 1] > off[e] else []
        rows += ends
        exps += [e] * len(ends)
    rows, exps = np.array(rows), np.array(exps)
    say(f"  {len(set(exps.tolist()))} experts with rows, {len(rows)} rows compared")
    yh = host(y)[rows]
    ref = np.empty_like(yh, dtype=np.float64)
    for e in np.unique(exps):
        sel = exps == e
        ref[sel] = oracle.expert_ffn(inp["x"][tok[rows[sel]]], inp["w_gate_up"][e], inp["w_down"][e], True)["Y"]
    check_close(yh, ref, "bf16", "Y (first and last row of every expert)")


def test_ffn_ep8_shard():
    """One expert-parallel rank's share of the 256-expert shape: a 32768-token
    global batch routed and permuted on the GPU, the rank's 32 experts (about
    1024 rows each) through the grouped FFN in the configuration the bench
    times; every group's first and last row and a random sample against the
    oracle's expert FFN."""
    from workloads import ep_shard, expert_weight_range
    cfg, e0, e1 = ep_shard("dsv3_ep8")
    say(f"[ffn ep8 shard: experts {e0}..{e1 - 1} of {cfg.T} tokens]")
    inp = make_inputs(cfg, experts=False)
    x = dev(inp["x"])
    idx, _, _ = L.moe_route(x, dev(inp["w_router"]), cfg.k, cfg.score, sel_bias=dev(inp["bias"]))
    _, offsets, _, _, x_perm = L.moe_permute(idx, x, cfg.E)
    off = host(offsets)[e0:e1 + 1].astype(np.int64)
    n = off[1:] - off[:-1]
    say(f"  rows {off[-1] - off[0]}, per expert min {n.min()} max {n.max()}")
    assert n.min() > 0
    xs_np = host(x_perm[int(off[0]):int(off[-1])])
    del x, x_perm
    wgu, wd = expert_weight_range(cfg, e0, e1)
    g_off = off - off[0]
    rng = np.random.default_rng(5)
    check = np.unique(np.concatenate([g_off[:-1], g_off[1:] - 1, rng.integers(0, g_off[-1], 64)]))
    _ffn_case(cfg, g_off, xs_np, wgu, wd, rows_to_check=check, save_gu=False)


@pytest.mark.parametrize("case", ["256 experts of ~100 rows, gathered", "8 ragged experts, d = 512, f = 384",
                                  "empty and skewed experts, d = 192", "one expert, permuted rows"])
def test_ffn_packed_weights_bit_identical(case):
    """moe_grouped_ffn_packed on the tile-order copies of
    moe_pack_expert_weights gives bit for bit what the unpacked call gives
    (half tiles, ragged and empty experts, down-projection rows padded past
    d, gathered and already-permuted rows), and matches the oracle's expert
    FFN on sampled rows."""
    from workloads import f32_to_bf16_bits
    say(f"[ffn packed weights: {case}]")
    rng = np.random.default_rng(len(case))
    if case.startswith("256"):
        E, d, f, T = 256, 256, 256, 3000
        counts = rng.integers(60, 160, E)
    elif case.startswith("8"):
        E, d, f, T = 8, 512, 384, 900
        counts = np.array([300, 1, 0, 777, 256, 255, 129, 40])
    elif case.startswith("empty"):
        E, d, f, T = 16, 192, 128, 1200
        counts = np.zeros(E, np.int64)
        counts[[1, 5, 6]] = [1000, 3, 700]
    else:
        E, d, f, T = 1, 128, 256, 640
        counts = np.array([640])
    rows = int(counts.sum())
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    bits = lambda *shape, sd: f32_to_bf16_bits((rng.standard_normal(shape) * sd).astype(np.float32))
    x = bits(T, d, sd=1.0)
    wgu, wd = bits(E, 2 * f, d, sd=0.05), bits(E, d, f, sd=0.05)
    gathered = case != "one expert, permuted rows"
    tok = rng.integers(0, T, rows).astype(np.int32) if gathered else None
    xd, offd, wgud, wdd = dev(x), dev(offsets), dev(wgu), dev(wd)
    if gathered:
        g0, h0, y0 = L.moe_grouped_ffn_gather(xd, dev(tok), offd, wgud, wdd, save_gu=True)
    else:
        g0, h0, y0 = L.moe_grouped_ffn(xd, offd, wgud, wdd, save_gu=True)
    pgu, pd = L.moe_pack_expert_weights(wgud, wdd)
    g1, h1, y1 = L.moe_grouped_ffn_packed(xd, dev(tok) if gathered else None, offd, pgu, pd, f, save_gu=True)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1) and torch.equal(h0, h1) and torch.equal(g0, g1)
    sample = np.unique(np.concatenate([offsets[:-1][counts > 0], offsets[1:][counts > 0] - 1,
                                       rng.integers(0, rows, 32)]))
    grp = np.searchsorted(offsets, sample, side="right") - 1
    ref = np.zeros((len(sample), d))
    xin = x[tok] if gathered else x
    for e in np.unique(grp):
        sel = grp == e
        ref[sel] = oracle.expert_ffn(xin[sample[sel]], wgu[e], wd[e], True)["Y"]
    check_close(host(y1)[sample], ref, "bf16", f"Y ({len(sample)} rows)")



def _last_round_split(counts, NB, rows, smax):
    """Column parts per tile of a row-grouped 256 x 256 GEMM's last round, as
    the kernel decides it: the persistent grid (one workgroup per CU at
    most, a multiple of 8, sized by the upper bound on tiles) and the tiles
    left for its last round, cut in 2 or 4 while they fill at most the grid."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    total = int(sum(-(-int(n) // 256) for n in counts)) * NB
    upper = (-(-rows // 256) + len(counts)) * NB
    grid = max(8, min(cus & ~7, (upper + 7) & ~7))
    rem, s = total % grid, 1
    while rem > 0 and s < smax and rem * s * 2 <= grid:
        s *= 2
    return s


@pytest.mark.parametrize("mode", ["rows given", "gathered", "packed weights"])
def test_ffn_last_round_column_parts_bit_identical(mode):
    """Tiles of a GEMM's under-filled last round run as 2 or 4 column parts;
    each part computes its outputs exactly as the whole tile does.  Two
    calls on the same experts 0 and 1: in the first they make up the whole
    (last) round and both expert GEMMs cut their tiles in four; in the
    second a large expert 2 fills the grid past half, nothing is cut, and
    expert 0's ragged tile runs as a 128-row half tile.  Rows of experts 0
    and 1 must come out bit for bit the same, and match the oracle."""
    from workloads import f32_to_bf16_bits
    say(f"[ffn last-round column parts: {mode}]")
    rng = np.random.default_rng(11)
    E, d, f = 8, 256, 256
    bits = lambda *shape, sd: f32_to_bf16_bits((rng.standard_normal(shape) * sd).astype(np.float32))
    wgu, wd = bits(E, 2 * f, d, sd=0.05), bits(E, d, f, sd=0.05)
    runs = []
    for extra in (0, 4096):
        counts = np.array([300, 200, extra, 0, 0, 0, 0, 0])
        rows = int(counts.sum())
        split_up = _last_round_split(counts, f // 128, rows, 4)
        split_down = _last_round_split(counts, -(-d // 256), rows, 4)
        assert (split_up, split_down) == ((4, 4) if extra == 0 else (1, 1)), (split_up, split_down)
        runs.append(counts)
    x = bits(4596, d, sd=1.0)
    tok = rng.permutation(4596).astype(np.int32)
    xd, wgud, wdd = dev(x), dev(wgu), dev(wd)
    packed = L.moe_pack_expert_weights(wgud, wdd) if mode == "packed weights" else None
    outs = []
    for counts in runs:
        rows = int(counts.sum())
        offd = dev(np.concatenate([[0], np.cumsum(counts)]).astype(np.int32))
        if mode == "rows given":
            outs.append(L.moe_grouped_ffn(dev(x[:rows]), offd, wgud, wdd, save_gu=True))
        elif mode == "gathered":
            outs.append(L.moe_grouped_ffn_gather(xd, dev(tok[:rows]), offd, wgud, wdd, save_gu=True))
        else:
            outs.append(L.moe_grouped_ffn_packed(xd, dev(tok[:rows]), offd, packed[0], packed[1], f, save_gu=True))
    torch.cuda.synchronize()
    for a, b, what in zip(outs[0], outs[1], ("G|U", "H", "Y")):
        assert torch.equal(a[:500], b[:500]), what
    xin = x[:500] if mode == "rows given" else x[tok[:500]]
    for e, (r0, r1) in enumerate([(0, 300), (300, 500)]):
        o = oracle.expert_ffn(xin[r0:r1], wgu[e], wd[e], True)
        check_close(host(outs[0][2])[r0:r1], o["Y"], "bf16", f"Y expert {e}")
        check_close(host(outs[0][1])[r0:r1], o["H"], "bf16", f"H expert {e}")

def test_forward_packed_weights():
    """A forward-only layer with packed expert weights (routed and shared)
    gives the same output, bit for bit, as with the weights as given, and
    the oracle's."""
    say("[forward packed weights]")
    from mixture_experts_layer_free_amd.layer import MoELayer, Shape
    cfg = scaled(CONFIGS["dsv3"], T=700, d=256, E=24, k=3, f=128, f_shared=256, bias_update=False)
    inp = make_inputs(cfg)
    outs = []
    for packed in (False, True):
        sh = Shape(cfg.T, cfg.d, cfg.E, cfg.k, cfg.f, torch.bfloat16, cfg.score, cfg.shared, cfg.f_shared,
                   packed_weights=packed)
        layer = MoELayer(sh, dev(inp["w_router"]), dev(inp["w_gate_up"]), dev(inp["w_down"]), dev(inp["bias"]),
                         dev(inp["logit_offset"]), dev(inp["w_gate_up_shared"]), dev(inp["w_down_shared"]))
        assert (layer.packed is not None) == packed and (layer.packed_sh is not None) == packed
        outs.append(host(layer.forward(dev(inp["x"]))).copy())
    torch.cuda.synchronize()
    assert np.array_equal(outs[0], outs[1])
    ref = oracle.forward(inp["x"], inp["w_router"], inp["w_gate_up"], inp["w_down"], cfg.k, cfg.score, True,
                         sel_bias=inp["bias"], logit_offset=inp["logit_offset"],
                         w_gate_up_shared=inp["w_gate_up_shared"], w_down_shared=inp["w_down_shared"])
    keep = ref["margin"] >= 1e-6
    check_close(outs[1][keep], ref["out"][keep], "bf16", "out (packed weights)")


@pytest.mark.parametrize("packed,fp32", [(False, False), (True, False), (False, True)])
def test_forward_ffn_stage_events(packed, fp32):
    """The grouped FFN timing hook: the routed call records both events (the
    output unchanged, bit for bit), and only that call (the shared expert's
    call after it and a later forward leave them as they were)."""
    say(f"[forward ffn stage events packed={packed} fp32={fp32}]")
    from mixture_experts_layer_free_amd.layer import MoELayer, Shape
    cfg = scaled(CONFIGS["dsv3"], T=700, d=256, E=24, k=3, f=128, f_shared=256, bias_update=False)
    inp = make_inputs(cfg)
    dt = torch.float32 if fp32 else torch.bfloat16
    sh = Shape(cfg.T, cfg.d, cfg.E, cfg.k, cfg.f, dt, cfg.score, cfg.shared, cfg.f_shared, packed_weights=packed)
    cast = (lambda a: dev(a).float()) if fp32 else dev
    layer = MoELayer(sh, dev(inp["w_router"]), cast(inp["w_gate_up"]), cast(inp["w_down"]), dev(inp["bias"]),
                     dev(inp["logit_offset"]), cast(inp["w_gate_up_shared"]), cast(inp["w_down_shared"]))
    x = cast(inp["x"])
    plain = host(layer.forward(x)).copy()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(1 + len(L.FFN_STAGES))]
    for e in evs:
        e.record()
    torch.cuda.synchronize()
    timed = host(layer.forward(x, ffn_events=evs)).copy()
    torch.cuda.synchronize()
    assert np.array_equal(plain, timed)
    t_up, t_down = evs[0].elapsed_time(evs[1]), evs[1].elapsed_time(evs[2])
    assert t_up > 0 and t_down > 0, (t_up, t_down)
    layer.forward(x)
    torch.cuda.synchronize()
    assert (evs[0].elapsed_time(evs[1]), evs[1].elapsed_time(evs[2])) == (t_up, t_down)


# ---------------------------------------------------------------------------- combine / bias

@pytest.mark.parametrize("k,shared,bf16", [(2, False, False), (8, True, False), (16, False, True), (1, True, True)])
def test_combine(k, shared, bf16):
    say(f"[combine k={k} shared={shared} bf16={bf16}]")
    rng = np.random.default_rng(k)
    T, d = 333, 96
    A = T * k
    y = rng.standard_normal((A, d)).astype(np.float32)
    row_of = rng.permutation(A).reshape(T, k).astype(np.int32)
    g = rng.uniform(0, 1, (T, k)).astype(np.float32)
    sh = rng.standard_normal((T, d)).astype(np.float32) if shared else None
    out = L.moe_combine(dev(y), dev(row_of), dev(g), dev(sh), out_dtype=torch.bfloat16 if bf16 else torch.float32)
    ref = oracle.combine(y, row_of, g, sh)
    got = host(out)
    if bf16:
        # a bf16 output carries at most half a bf16 ulp (<= 2^-8 |value|) of
        # rounding on top of the fp32 sum's own error
        err = np.abs(as_f64(got) - ref)
        assert np.all(err <= 2.0 ** -8 * np.abs(ref) + 1e-5), float((err - 2.0 ** -8 * np.abs(ref)).max())
    else:
        check_close(got, ref, "f32", "out")


def test_bias_update_bit_exact():
    say("[bias update]")
    rng = np.random.default_rng(0)
    for E, T, k in ((8, 64, 2), (64, 8192, 8), (256, 4096, 8), (7, 5, 3), (1024, 333, 16)):
        b = rng.uniform(-0.05, 0.05, E).astype(np.float32)
        counts = rng.multinomial(T * k, np.ones(E) / E).astype(np.int32)
        counts[:3] = T * k // E          # some exactly on target when divisible
        tb = dev(b.copy())
        L.moe_bias_update(tb, dev(counts), T, k, 1e-3)
        assert np.array_equal(host(tb), oracle.bias_update(b, counts, T, k, 1e-3))


def test_bias_trajectory_over_steps():
    """The loss-free controller's feedback loop (lesson, Load balancing item 3
    and Build it step 2): five steps of route -> permute -> bias update on the
    GPU, each step's bias steering the next selection.  Every step: the
    routing against the oracle fed the GPU's current bias (near-ties
    excluded), the counts of the GPU's choice bit-exact, and the updated bias
    bit-exact."""
    say("[bias trajectory]")
    cfg = scaled(CONFIGS["fine"], T=2048, d=256, E=64, k=8, f=64)
    inp = make_inputs(cfg, experts=False)
    w, o = dev(inp["w_router"]), inp["logit_offset"]
    bias = np.zeros(cfg.E, np.float32)
    tb = dev(bias.copy())
    for step in range(5):
        x_np = make_inputs(scaled(cfg, seed=1000 + step), experts=False)["x"]
        x = dev(x_np)
        idx, gate, logits = L.moe_route(x, w, cfg.k, cfg.score, dev(o), tb)
        ref = oracle.route(x_np, inp["w_router"], cfg.k, cfg.score, bias, o)
        check_route(host(idx), host(gate), host(logits), ref, cfg.k)
        counts = L.moe_permute(idx, x, cfg.E, copy=False)[0]
        c = host(counts)
        assert np.array_equal(c, oracle.permute(host(idx), cfg.E)[0])
        L.moe_bias_update(tb, counts, cfg.T, cfg.k, cfg.gamma)
        bias = oracle.bias_update(bias, c, cfg.T, cfg.k, cfg.gamma)
        assert np.array_equal(host(tb), bias), step
    assert np.count_nonzero(bias) > cfg.E // 2   # the controller moved most experts


# ---------------------------------------------------------------------------- whole layer

def _layer(cfg, inp, train=False):
    from mixture_experts_layer_free_amd.layer import MoELayer, Shape
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    s = Shape(cfg.T, cfg.d, cfg.E, cfg.k, cfg.f, dt, cfg.score, cfg.shared, cfg.f_shared, cfg.bias_update, cfg.gamma,
              train)
    return MoELayer(s, dev(inp["w_router"]), dev(inp["w_gate_up"]), dev(inp["w_down"]), dev(inp["bias"].copy()),
                    dev(inp["logit_offset"]), dev(inp.get("w_gate_up_shared")), dev(inp.get("w_down_shared")))


def _forward_check(cfg, inp, sample=None):
    layer = _layer(cfg, inp)
    x = dev(inp["x"])
    out = host(layer.forward(x))
    torch.cuda.synchronize()
    T = cfg.T
    tok = np.arange(T) if sample is None else np.asarray(sample)
    ref = oracle.forward(np.asarray(inp["x"])[tok], inp["w_router"], inp["w_gate_up"], inp["w_down"], cfg.k, cfg.score,
                         cfg.dtype == "bf16", sel_bias=inp["bias"], logit_offset=inp["logit_offset"],
                         w_gate_up_shared=inp.get("w_gate_up_shared"), w_down_shared=inp.get("w_down_shared"))
    keep = ref["margin"] >= 1e-6
    say(f"  tokens compared {int(keep.sum())} of {len(tok)}")
    check_close(out[tok][keep], ref["out"][keep], _kind(cfg), "out")
    if cfg.bias_update:
        b = oracle.bias_update(inp["bias"], host(layer.counts), T, cfg.k, cfg.gamma)
        assert np.array_equal(host(layer.sel_bias), b)
    return layer


@pytest.mark.parametrize("name", ["tiny", "tiny_dense"])
@pytest.mark.parametrize("score", oracle.SCORE_FNS)
def test_forward_tiny(name, score):
    say(f"[forward {name} {score}]")
    cfg = scaled(CONFIGS[name], score=score)
    _forward_check(cfg, make_inputs(cfg))


@pytest.mark.parametrize("score", oracle.SCORE_FNS)
def test_forward_bf16_small(score):
    say(f"[forward bf16 small {score}]")
    cfg = scaled(CONFIGS["dsv3"], T=700, d=256, E=24, k=3, f=128, f_shared=192, score=score, bias_update=True)
    _forward_check(cfg, make_inputs(cfg))


@pytest.mark.parametrize("name,n_sample", [("coarse", 512), ("fine", 1024), ("dsv3", 256)])
def test_forward_full_size(name, n_sample):
    """Full-size layer forward, sampled tokens against the oracle (the whole
    layer: routing, every chosen expert and, for the 256+1 expert shape, the
    shared expert; that shape holds 22.6 GB of expert weights, which its
    oracle converts one expert at a time)."""
    cfg = CONFIGS[name]
    say(f"[forward full {name}]")
    inp = make_inputs(cfg)
    say("  inputs generated")
    rng = np.random.default_rng(0)
    _forward_check(cfg, inp, sample=np.sort(rng.choice(cfg.T, n_sample, replace=False)))


@pytest.mark.parametrize("name,score,cap", [("tiny", "softmax", 5), ("tiny", "sigmoid", 0), ("tiny", "sqrt_softplus", 9),
                                            ("bf16", "sigmoid", 60), ("bf16", "softmax", 1)])
def test_forward_capacity(name, score, cap):
    """Layer forward with an expert capacity against the oracle fed the GPU's
    routing: dropped slots add nothing, gates are not renormalised."""
    say(f"[forward capacity {name} {score} cap={cap}]")
    if name == "tiny":
        cfg = scaled(CONFIGS["tiny"], score=score)
    else:
        cfg = scaled(CONFIGS["dsv3"], T=700, d=256, E=24, k=3, f=128, f_shared=192, score=score)
    inp = make_inputs(cfg)
    from mixture_experts_layer_free_amd.layer import MoELayer, Shape
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    sh = Shape(cfg.T, cfg.d, cfg.E, cfg.k, cfg.f, dt, cfg.score, cfg.shared, cfg.f_shared, False, cfg.gamma, False,
               capacity=cap)
    layer = MoELayer(sh, dev(inp["w_router"]), dev(inp["w_gate_up"]), dev(inp["w_down"]), dev(inp["bias"]),
                     dev(inp["logit_offset"]), dev(inp.get("w_gate_up_shared")), dev(inp.get("w_down_shared")))
    out = host(layer.forward(dev(inp["x"])))
    torch.cuda.synchronize()
    idx = host(layer.idx).astype(np.int64)
    ref = oracle.forward(inp["x"], inp["w_router"], inp["w_gate_up"], inp["w_down"], cfg.k, cfg.score,
                         cfg.dtype == "bf16", sel_bias=inp["bias"], logit_offset=inp["logit_offset"],
                         w_gate_up_shared=inp.get("w_gate_up_shared"), w_down_shared=inp.get("w_down_shared"),
                         idx=idx, capacity=cap)
    assert np.array_equal(host(layer.row_of), ref["row_of"]) and np.array_equal(host(layer.counts), ref["counts"])
    assert (ref["row_of"] < 0).any()
    check_close(out, ref["out"], _kind(cfg), "out")


@pytest.mark.parametrize("name", ["tiny", "bf16"])
def test_forward_hash_router(name):
    """Layer forward with the hash router (token ids in, gates 1/k) against the oracle."""
    say(f"[forward hash {name}]")
    if name == "tiny":
        cfg = CONFIGS["tiny"]
    else:
        cfg = scaled(CONFIGS["dsv3"], T=700, d=256, E=24, k=3, f=128, f_shared=192)
    inp = make_inputs(cfg)
    ids = np.random.default_rng(9).integers(0, 32000, cfg.T).astype(np.int32)
    from mixture_experts_layer_free_amd.layer import MoELayer, Shape
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    sh = Shape(cfg.T, cfg.d, cfg.E, cfg.k, cfg.f, dt, cfg.score, cfg.shared, cfg.f_shared, router="hash", salt=5)
    layer = MoELayer(sh, None, dev(inp["w_gate_up"]), dev(inp["w_down"]),
                     w_gate_up_shared=dev(inp.get("w_gate_up_shared")), w_down_shared=dev(inp.get("w_down_shared")))
    out = host(layer.forward(dev(inp["x"]), token_ids=dev(ids)))
    torch.cuda.synchronize()
    idx = oracle.hash_route(ids, cfg.E, cfg.k, 5)["idx"]
    assert np.array_equal(host(layer.idx), idx)
    ref = oracle.forward(inp["x"], None, inp["w_gate_up"], inp["w_down"], cfg.k, "uniform", cfg.dtype == "bf16",
                         w_gate_up_shared=inp.get("w_gate_up_shared"), w_down_shared=inp.get("w_down_shared"), idx=idx)
    check_close(out, ref["out"], _kind(cfg), "out")


@pytest.mark.parametrize("name", ["tiny", "bf16"])
def test_forward_fused_permute(name):
    """The layer with the permute fused into the expert GEMM (no X_perm) gives
    the same output as with the copy, and the oracle's."""
    from mixture_experts_layer_free_amd.layer import MoELayer, Shape
    cfg = CONFIGS["tiny"] if name == "tiny" else scaled(CONFIGS["fine"], T=900, d=256, E=24, k=3, f=128)
    say(f"[forward fused permute {name}]")
    inp = make_inputs(cfg)
    dt = torch.float32 if cfg.dtype == "f32" else torch.bfloat16
    outs = []
    for fuse in (False, True):
        sh = Shape(cfg.T, cfg.d, cfg.E, cfg.k, cfg.f, dt, cfg.score, fuse_permute=fuse)
        layer = MoELayer(sh, dev(inp["w_router"]), dev(inp["w_gate_up"]), dev(inp["w_down"]), dev(inp["bias"]),
                         dev(inp["logit_offset"]))
        assert (layer.x_perm is None) == fuse
        outs.append(host(layer.forward(dev(inp["x"]))).copy())
    torch.cuda.synchronize()
    assert np.array_equal(outs[0], outs[1])
    ref = oracle.forward(inp["x"], inp["w_router"], inp["w_gate_up"], inp["w_down"], cfg.k, cfg.score,
                         cfg.dtype == "bf16", sel_bias=inp["bias"], logit_offset=inp["logit_offset"])
    keep = ref["margin"] >= 1e-6
    check_close(outs[1][keep], ref["out"][keep], _kind(cfg), "out (fused permute)")


def test_forward_deterministic():
    say("[forward determinism]")
    cfg = scaled(CONFIGS["fine"], T=1000, d=256, E=32, k=4, f=128)
    inp = make_inputs(cfg)
    a = _layer(cfg, inp)
    b = _layer(cfg, inp)
    x = dev(inp["x"])
    oa = host(a.forward(x)).copy()
    ob = host(b.forward(x))
    assert np.array_equal(oa, ob)
    assert np.array_equal(host(a.token_of), host(b.token_of))
    assert np.array_equal(host(a.y_perm), host(b.y_perm))
