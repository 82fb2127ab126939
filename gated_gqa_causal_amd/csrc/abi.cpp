// abi.cpp -- the C ABI of libgatedattn.so: argument validation, the context
// and its workspace, kernel dispatch on the caller's stream, and event timing.
//
// Boundary conventions follow the attention-tile page ("cuda: widen the
// attention query tile on sm_89 and sm_120", review sections
// "Dispatch/guard" and the device-ownership finding: pre-validate, return the
// error, never fall back; decisions keyed by the current device) and the QSA
// kernel page ("What changed": geometry validated before sizing any buffer,
// a short cos/sin table refused, an empty launch a no-op).

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <new>
#include <vector>

#include "gatedattn.h"
#include "kernels.h"
#include "schedule.h"
#ifdef ATTN_TEST_HOOKS
#include "test_hooks.h"
#endif

struct attn_ctx {
    int device = -1;
    int num_cus = 0;               // compute units of the device
    attn_geometry geom{};
    int tpad = 0;                  // max_tokens rounded up to 64
    int mask_words = 0;            // 32-key words per mask row at max_tokens
    uint16_t *kp = nullptr;        // prepared keys, [Hkv][tpad/32] tiles of 32 x 256
    uint16_t *vt = nullptr;        // transposed values, [Hkv][tpad/32] tiles of 256 x 32
    uint32_t *mask_bits = nullptr; // [mask_words][tpad]: key word major
    uint8_t *tile_vis = nullptr;   // [ceil(max_tokens/64)][mask_words]
    float *row_stats = nullptr;    // [max_tokens][Hq][2]: softmax max and sum (weights calls)
    // packed batches: the per-call sequence tables (device), staged through a
    // pinned host buffer whose previous copy `batch_copied` must have landed
    // before it is rewritten
    int *batch_tab = nullptr;
    int *batch_host = nullptr;
    size_t batch_cap = 0;          // ints in each
    hipEvent_t batch_copied = nullptr;
    bool batch_pending = false;
    // the attention kernel's work table (schedule.h's sched_plan or
    // sched_plan_halves) of the last launch shape, staged like the batch
    // tables; kept while the shape repeats
    int *sched_tab = nullptr;
    int *sched_host = nullptr;
    size_t sched_cap = 0;          // ints in each
    hipEvent_t sched_copied = nullptr;
    bool sched_pending = false;
    bool sched_valid = false;      // sched_key holds the last shape planned
    bool sched_use = false;        // and the table is in sched_tab (else the snake)
    int sched_P = 0;               // the table's workgroups (the launch grid)
    int sched_key[7] = {0, 0, 0, 0, 0, 0, 0};
    // timing
    int timing = 0;                // bit (1 << ATTN_KERNEL_*) per timed kernel
    std::vector<hipEvent_t> pool;
    size_t pool_used = 0;
    struct Rec {
        int kernel;
        hipEvent_t a, b;
    };
    std::vector<Rec> recs;
};

namespace {

constexpr int kKinds = 6;   // 0 gated, 1 prefix, 2 masked, 3 bidirectional, 4 append to a K/V cache,
                            // 5 append to an fp8 K/V cache

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_geometry(const attn_geometry *g)
{
    if (!g)
        return ATTN_ERR_NULL_ARG;
    if (g->head_dim != ATTN_HEAD_DIM || g->rotary_dim != ATTN_ROTARY_DIM)
        return ATTN_ERR_GEOMETRY;
    if (g->n_kv_heads < 1 || g->n_q_heads < 1 || g->n_q_heads % g->n_kv_heads != 0)
        return ATTN_ERR_GEOMETRY;
    const int G = g->n_q_heads / g->n_kv_heads;
    if (G < 1 || G > ATTN_MAX_GROUP || g->n_kv_heads > 1024)
        return ATTN_ERR_GEOMETRY;
    if (!(g->rms_eps > 0.0f) || !std::isfinite(g->rms_eps))
        return ATTN_ERR_GEOMETRY;
    if (g->max_tokens < 1 || g->max_tokens > ATTN_MAX_TOKENS)
        return ATTN_ERR_RANGE;
    return ATTN_OK;
}

struct Timer {
    attn_ctx *ctx;
    hipStream_t stream;
    int kernel;
    hipEvent_t a = nullptr, b = nullptr;
    Timer(attn_ctx *c, hipStream_t s, int k) : ctx(c), stream(s), kernel(k)
    {
        if ((ctx->timing >> kernel & 1) && ctx->pool_used + 2 <= ctx->pool.size()) {
            a = ctx->pool[ctx->pool_used++];
            b = ctx->pool[ctx->pool_used++];
            (void)hipEventRecord(a, stream);
        }
    }
    void stop()
    {
        if (a) {
            (void)hipEventRecord(b, stream);
            ctx->recs.push_back({kernel, a, b});
        }
    }
};

int current_device_matches(const attn_ctx *ctx)
{
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess || cur != ctx->device)
        return ATTN_ERR_DEVICE;
    return ATTN_OK;
}

// Prepared keys / transposed values of Hkv x tpad keys at kp_ws / vt_ws.
void fill_kv_params_ws(ga::KvPrologueParams &kp, const attn_geometry &g, uint16_t *kp_ws, uint16_t *vt_ws,
                       int tpad, const attn_inputs *in, int T)
{
    kp.k = static_cast<const uint16_t *>(in->k);
    kp.v = static_cast<const uint16_t *>(in->v);
    kp.wk = static_cast<const uint16_t *>(in->k_norm_w);
    kp.cos_tab = in->cos_tab;
    kp.sin_tab = in->sin_tab;
    kp.kp = kp_ws;
    kp.vt = vt_ws;
    kp.T = T;
    kp.Hkv = g.n_kv_heads;
    kp.Tpad = tpad;
    kp.tile0 = 0;
    kp.k_row0 = 0;
    kp.eps = g.rms_eps;
    kp.tile_seg = nullptr;
    kp.seg = nullptr;
    kp.k8 = kp.v8 = nullptr;
    kp.k8s = kp.v8s = nullptr;
}

void fill_kv_params(ga::KvPrologueParams &kp, const attn_ctx *ctx, const attn_inputs *in, int T)
{
    fill_kv_params_ws(kp, ctx->geom, ctx->kp, ctx->vt, ctx->tpad, in, T);
}

// Bytes of a caller-owned K/V cache for a geometry: prepared keys and
// transposed values, max_tokens rounded up to 64, in the workspace's layout.
size_t kv_cache_bytes(const attn_geometry &g)
{
    const size_t tpad = ((size_t)g.max_tokens + 63) / 64 * 64;
    return 2 * (size_t)g.n_kv_heads * tpad * ATTN_HEAD_DIM * 2;
}

// Bytes of a caller-owned fp8 K/V cache: e4m3 key rows and value rows
// [Hkv][tpad][256] each, then fp32 scales [Hkv][tpad] for keys and values.
size_t kv_cache_fp8_bytes(const attn_geometry &g)
{
    const size_t tpad = ((size_t)g.max_tokens + 63) / 64 * 64;
    return 2 * (size_t)g.n_kv_heads * tpad * ATTN_HEAD_DIM + 2 * (size_t)g.n_kv_heads * tpad * 4;
}

void fill_attn_params_ws(ga::AttnParams &ap, const attn_geometry &g, const uint16_t *kp_ws, const uint16_t *vt_ws,
                         int tpad, int num_cus, const attn_inputs *in, int T, int q_base, void *out)
{
    ap.qg = static_cast<const uint16_t *>(in->qg);
    ap.kp = kp_ws;
    ap.vt = vt_ws;
    ap.wq = static_cast<const uint16_t *>(in->q_norm_w);
    ap.cos_tab = in->cos_tab;
    ap.sin_tab = in->sin_tab;
    ap.bits = nullptr;
    ap.tilevis = nullptr;
    ap.out = static_cast<uint16_t *>(out);
    ap.S = T - q_base;
    ap.T = T;
    ap.q_base = q_base;
    ap.Hq = g.n_q_heads;
    ap.Hkv = g.n_kv_heads;
    ap.G = g.n_q_heads / g.n_kv_heads;
    ap.n_hg = (ap.G + ga::kHeadsPerBlock - 1) / ga::kHeadsPerBlock;
    ap.nrb = (ap.S + ga::kRowsPerBlock - 1) / ga::kRowsPerBlock;
    ap.Tpad = tpad;
    ap.W = (T + 31) / 32;
    ap.bstride = (ap.S + ga::kRowsPerBlock - 1) / ga::kRowsPerBlock * ga::kRowsPerBlock;
    ap.eps = g.rms_eps;
    // One workgroup per compute unit at most; each walks its share of the
    // work items (see the attention kernel).
    ap.n_wg = (int)std::min<int64_t>((int64_t)ap.nrb * ap.Hkv * ap.n_hg, num_cus);
    ap.pairs = nullptr;
    ap.seg = nullptr;
    ap.ckp = ap.cvt = nullptr;
    ap.ml = nullptr;
    ap.sched = nullptr;
}

void fill_attn_params(ga::AttnParams &ap, const attn_ctx *ctx, const attn_inputs *in, int T, int q_base,
                      void *out)
{
    fill_attn_params_ws(ap, ctx->geom, ctx->kp, ctx->vt, ctx->tpad, ctx->num_cus, in, T, q_base, out);
    ap.bits = ctx->mask_bits;
    ap.tilevis = ctx->tile_vis;
}

// Scratch bytes the allocation-free pass over S tokens needs.
size_t noalloc_bytes(const attn_geometry &g, int S)
{
    const size_t tpad = ((size_t)S + 63) / 64 * 64;
    return 2 * (size_t)g.n_kv_heads * tpad * ATTN_HEAD_DIM * 2;
}

// Packed batch bookkeeping: ints of the per-call table for a workspace of
// `tpad` keys: seg {len, first row, first tile, 0} per sequence, the sequence
// of every prepared tile, and the (sequence, row block) pairs heaviest first.
size_t batch_table_ints(int tpad) { return 4 * (size_t)ATTN_MAX_SEQS + tpad / 32 + 2 * ((size_t)tpad / 64 + ATTN_MAX_SEQS); }

struct BatchPlan {
    int64_t total = 0, tiles = 0;
    int max_len = 0, pairs = 0;
};

// Checks the lengths (and, with `tab`, writes the table): every length in
// [0, max_tokens], their sum <= max_tokens, and their 32-key tiles within the
// workspace (each sequence starts on a tile boundary).  pos0: the position of
// every sequence's first key (0, or a shared prefix's length).
int plan_batch(const attn_geometry &g, int32_t n_seqs, const int32_t *lens, BatchPlan *plan, int *tab,
               int pos0 = 0)
{
    if (n_seqs < 0 || n_seqs > ATTN_MAX_SEQS)
        return ATTN_ERR_RANGE;
    if (n_seqs > 0 && !lens)
        return ATTN_ERR_NULL_ARG;
    const int64_t tpad = ((int64_t)g.max_tokens + 63) / 64 * 64;
    BatchPlan pl;
    for (int i = 0; i < n_seqs; ++i) {
        if (lens[i] < 0 || lens[i] > g.max_tokens)
            return ATTN_ERR_RANGE;
        pl.total += lens[i];
        pl.tiles += (lens[i] + 31) / 32;
        pl.max_len = std::max(pl.max_len, (int)lens[i]);
    }
    if (pl.total > g.max_tokens || pl.tiles * 32 > tpad)
        return ATTN_ERR_RANGE;
    struct Pair {
        int nt, seq, rb;
    };
    std::vector<Pair> pairs;
    if (tab) {
        int *seg = tab, *tile_seg = tab + 4 * n_seqs;
        int row = 0, tile = 0;
        for (int i = 0; i < n_seqs; ++i) {
            const int L = lens[i], nt = (L + 31) / 32;
            seg[4 * i] = L;
            seg[4 * i + 1] = row;
            seg[4 * i + 2] = tile;
            seg[4 * i + 3] = pos0;
            for (int t = 0; t < nt; ++t)
                tile_seg[tile + t] = i;
            for (int rb = 0; rb * 64 < L; ++rb)
                pairs.push_back({(pos0 + std::min(rb * 64 + 63, L - 1)) / 32 + 1, i, rb});
            row += L;
            tile += nt;
        }
        // Heaviest walks first (ties: sequence, then row block), as the single
        // pass numbers its row blocks.
        std::sort(pairs.begin(), pairs.end(), [](const Pair &a, const Pair &b) {
            return a.nt != b.nt ? a.nt > b.nt : a.seq != b.seq ? a.seq < b.seq : a.rb < b.rb;
        });
        int *pr = tile_seg + pl.tiles;
        for (size_t k = 0; k < pairs.size(); ++k) {
            pr[2 * k] = pairs[k].seq;
            pr[2 * k + 1] = pairs[k].rb;
        }
        pl.pairs = (int)pairs.size();
    }
    if (plan)
        *plan = pl;
    return ATTN_OK;
}

// kind 4: `mask` is the caller's K/V cache; the prologue writes keys
// q_base..T-1 into it (k and v hold only those rows) and attention reads it.
// A work item's query prologue and epilogue, in key tiles of the walk (cycle
// counts of the kernel: about 35 K cycles per item, 2.6 K per key tile).
constexpr int kSchedOverheadTiles = 14;

// The attention kernel's work table for ap's launch (a causal or masked pass,
// row block rbi walking the key tiles up to its last row's position): planned
// on the host once per launch shape (schedule.h's sched_plan, and
// sched_plan_halves with items split into 32-row halves over every compute
// unit) and copied to the device when its busiest workgroup is at least 1%
// lighter than the snake order's, which the kernel follows otherwise.  The
// staging buffer is rewritten only after its previous copy has landed.
int attach_schedule(attn_ctx *ctx, ga::AttnParams &ap, hipStream_t s, bool masked)
{
    const int key[7] = {ap.n_wg, ap.nrb, ap.Hkv, ap.n_hg, ap.T, ap.q_base, masked ? 1 : 0};
    if (!ctx->sched_valid || !std::equal(key, key + 7, ctx->sched_key)) {
        std::vector<int> tiles((size_t)ap.nrb), rows((size_t)ap.nrb);
        for (int rbi = 0; rbi < ap.nrb; ++rbi) {
            const int r0 = ga::kRowsPerBlock * (ap.nrb - 1 - rbi);
            const int p0 = ap.q_base + r0;
            tiles[rbi] = std::min(p0 + ga::kRowsPerBlock - 1, ap.T - 1) / ga::kKeysPerTile + 1;
            rows[rbi] = std::min(ga::kRowsPerBlock, ap.S - r0);
        }
        std::vector<int> table, halves;
        long busiest_snake = 0, busiest_table = 0, busiest_halves = 0;
        int P = ap.n_wg;
        // The table only for a real gain (its busiest workgroup at least 1%
        // lighter than the snake's); then items split into 32-row halves and
        // dealt over every compute unit where that makes the busiest workgroup
        // at least 1/8 lighter still (few items per workgroup, the heaviest far
        // above the mean).  A split item costs about 1.28 whole ones in all, and
        // on the power-limited chip that extra work slows every compute unit:
        // measured, plans 6-8% lighter in this model ran 1-6% slower, plans
        // 16-28% lighter 5-6% faster.
        bool use = ga::sched_plan(ap.n_wg, ap.nrb, ap.Hkv, ap.n_hg, tiles.data(), kSchedOverheadTiles, table,
                                  &busiest_snake, &busiest_table) &&
                   100 * busiest_table <= 99 * busiest_snake;
        const long busiest = use ? busiest_table : busiest_snake;
        if (ga::sched_plan_halves(ctx->num_cus, ap.nrb, ap.Hkv, ap.n_hg, tiles.data(), rows.data(),
                                  kSchedOverheadTiles, halves, &busiest_halves) &&
            8 * busiest_halves <= 7 * busiest) {
            table.swap(halves);
            use = true;
            P = ctx->num_cus;
        }
        ctx->sched_valid = false;
        if (use) {
            if (table.size() > ctx->sched_cap)
                return ATTN_ERR_RANGE;
            if (ctx->sched_pending && hipEventSynchronize(ctx->sched_copied) != hipSuccess)
                return ATTN_ERR_LAUNCH;
            ctx->sched_pending = false;
            std::memcpy(ctx->sched_host, table.data(), table.size() * sizeof(int));
            if (hipMemcpyAsync(ctx->sched_tab, ctx->sched_host, table.size() * sizeof(int), hipMemcpyHostToDevice,
                               s) != hipSuccess ||
                hipEventRecord(ctx->sched_copied, s) != hipSuccess)
                return ATTN_ERR_LAUNCH;
            ctx->sched_pending = true;
        }
        std::copy(key, key + 7, ctx->sched_key);
        ctx->sched_valid = true;
        ctx->sched_use = use;
        ctx->sched_P = P;
    }
    ap.sched = ctx->sched_use ? ctx->sched_tab : nullptr;
    if (ctx->sched_use)
        ap.n_wg = ctx->sched_P;
    return ATTN_OK;
}

int run(attn_ctx *ctx, const attn_inputs *in, int32_t T, int32_t q_base, int kind, const uint8_t *mask,
        void *out, void *stream, void *weights = nullptr)
{
    if (!ctx)
        return ATTN_ERR_NULL_ARG;
    int rc = attn_validate(&ctx->geom, in, T, q_base, kind, mask, out);
    if (rc != ATTN_OK)
        return rc;
    if (T - q_base == 0)
        return ATTN_OK;
    rc = current_device_matches(ctx);
    if (rc != ATTN_OK)
        return rc;
    hipStream_t s = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();   // clear a stale error so the launch status below is ours

    uint16_t *cache_k = nullptr, *cache_v = nullptr;
    if (kind == 4) {
        cache_k = reinterpret_cast<uint16_t *>(const_cast<uint8_t *>(mask));
        cache_v = cache_k + (size_t)ctx->geom.n_kv_heads * ctx->tpad * ATTN_HEAD_DIM;
    }
    ga::KvPrologueParams kvp;
    fill_kv_params(kvp, ctx, in, T);
    if (kind == 4) {
        kvp.kp = cache_k;
        kvp.vt = cache_v;
    }
    if (kind == 4 || kind == 5) {
        kvp.tile0 = q_base / ga::kKeysPerTile;
        kvp.k_row0 = q_base;
    }
    ga::KvWidenParams wp{};
    if (kind == 5) {
        // fp8 rows of the new keys into the cache, then every row 0..T-1
        // widened into the workspace's tiles for the attention kernel.
        const size_t rows = (size_t)ctx->geom.n_kv_heads * ctx->tpad;
        uint8_t *c8 = const_cast<uint8_t *>(mask);
        kvp.k8 = c8;
        kvp.v8 = c8 + rows * ATTN_HEAD_DIM;
        kvp.k8s = reinterpret_cast<float *>(c8 + 2 * rows * ATTN_HEAD_DIM);
        kvp.v8s = kvp.k8s + rows;
        wp.k8 = kvp.k8;
        wp.v8 = kvp.v8;
        wp.k8s = kvp.k8s;
        wp.v8s = kvp.v8s;
        wp.kp = ctx->kp;
        wp.vt = ctx->vt;
        wp.T = T;
        wp.Tpad = ctx->tpad;
    }
    {
        Timer tm(ctx, s, ATTN_KERNEL_KV_PROLOGUE);
        const int tiles = (T + ga::kKeysPerTile - 1) / ga::kKeysPerTile - kvp.tile0;
        if ((kind == 5 ? ga::launch_kv_prologue_fp8(kvp, tiles, s) : ga::launch_kv_prologue(kvp, tiles, s)) !=
            hipSuccess)
            return ATTN_ERR_LAUNCH;
        if (kind == 5 && ga::launch_kv_widen(wp, (T + ga::kKeysPerTile - 1) / ga::kKeysPerTile,
                                             ctx->geom.n_kv_heads, s) != hipSuccess)
            return ATTN_ERR_LAUNCH;
        tm.stop();
    }
    ga::AttnParams ap;
    fill_attn_params(ap, ctx, in, T, q_base, out);
    if (kind == 4) {
        ap.kp = cache_k;
        ap.vt = cache_v;
    }
    if (kind == 2) {
        ga::MaskPackParams mp;
        mp.mask = mask;
        mp.bits = ctx->mask_bits;
        mp.tilevis = ctx->tile_vis;
        mp.S = T;
        mp.W = ap.W;
        mp.bstride = ap.bstride;
        mp.vec16 = (T % 16 == 0) && aligned16(mask);
        Timer tm(ctx, s, ATTN_KERNEL_MASK_PACK);
        if (ga::launch_mask_pack(mp, ap.nrb, s) != hipSuccess)
            return ATTN_ERR_LAUNCH;
        tm.stop();
    }
    const ga::AttnMode mode = kind == 2 ? ga::AttnMode::Masked
                              : kind == 3 ? ga::AttnMode::Bidirectional : ga::AttnMode::Causal;
    if (weights)
        ap.ml = ctx->row_stats;
    if (mode != ga::AttnMode::Bidirectional) {
        const int rc = attach_schedule(ctx, ap, s, mode == ga::AttnMode::Masked);
        if (rc != ATTN_OK)
            return rc;
    }
    {
        Timer tm(ctx, s, ATTN_KERNEL_ATTENTION);
        if (ga::launch_attention(ap, mode, s) != hipSuccess)
            return ATTN_ERR_LAUNCH;
        tm.stop();
    }
    if (weights) {
        Timer tm(ctx, s, ATTN_KERNEL_WEIGHTS);
        if (ga::launch_attn_weights(ap, mode, static_cast<uint16_t *>(weights), ctx->num_cus, s) != hipSuccess)
            return ATTN_ERR_LAUNCH;
        tm.stop();
    }
    return ATTN_OK;
}

// A packed batch (validated): sequences of lens[i] rows back to back, each at
// positions pos0 .. pos0 + len - 1.  With pos0 > 0 they are branches of one
// shared prefix whose prepared keys 0..pos0-1 the caller's cache holds; each
// branch's own keys go to the workspace, the cache is only read.
int run_batch(attn_ctx *ctx, const attn_inputs *in, int32_t n_seqs, const int32_t *lens, int32_t pos0,
              const void *kv_cache, void *out, void *stream)
{
    BatchPlan pl;
    (void)plan_batch(ctx->geom, n_seqs, lens, &pl, nullptr);
    if (pl.total == 0)
        return ATTN_OK;
    int rc = current_device_matches(ctx);
    if (rc != ATTN_OK)
        return rc;
    hipStream_t s = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    // The staging buffer is reused: the previous call's copy must have landed.
    if (ctx->batch_pending && hipEventSynchronize(ctx->batch_copied) != hipSuccess)
        return ATTN_ERR_LAUNCH;
    ctx->batch_pending = false;
    (void)plan_batch(ctx->geom, n_seqs, lens, &pl, ctx->batch_host, pos0);
    const size_t n_int = 4 * (size_t)n_seqs + (size_t)pl.tiles + 2 * (size_t)pl.pairs;
    if (n_int > ctx->batch_cap)
        return ATTN_ERR_RANGE;
    if (hipMemcpyAsync(ctx->batch_tab, ctx->batch_host, n_int * sizeof(int), hipMemcpyHostToDevice, s) !=
            hipSuccess ||
        hipEventRecord(ctx->batch_copied, s) != hipSuccess)
        return ATTN_ERR_LAUNCH;
    ctx->batch_pending = true;
    const int *seg = ctx->batch_tab, *tile_seg = seg + 4 * n_seqs, *pairs = tile_seg + pl.tiles;

    ga::KvPrologueParams kvp;
    fill_kv_params(kvp, ctx, in, pos0 + pl.max_len);
    kvp.tile_seg = tile_seg;
    kvp.seg = seg;
    {
        Timer tm(ctx, s, ATTN_KERNEL_KV_PROLOGUE);
        if (ga::launch_kv_prologue(kvp, (int)pl.tiles, s) != hipSuccess)
            return ATTN_ERR_LAUNCH;
        tm.stop();
    }
    ga::AttnParams ap;
    fill_attn_params(ap, ctx, in, pos0 + pl.max_len, pos0, out);
    ap.pairs = pairs;
    ap.seg = seg;
    ap.nrb = pl.pairs;
    ap.n_wg = (int)std::min<int64_t>((int64_t)ap.nrb * ap.Hkv * ap.n_hg, ctx->num_cus);
    ga::AttnMode mode = ga::AttnMode::Causal;
    if (pos0 > 0) {
        const uint16_t *ck = static_cast<const uint16_t *>(kv_cache);
        ap.ckp = ck;
        ap.cvt = ck + (size_t)ctx->geom.n_kv_heads * ctx->tpad * ATTN_HEAD_DIM;
        mode = ga::AttnMode::SharedPrefix;
    }
    {
        Timer tm(ctx, s, ATTN_KERNEL_ATTENTION);
        if (ga::launch_attention(ap, mode, s) != hipSuccess)
            return ATTN_ERR_LAUNCH;
        tm.stop();
    }
    return ATTN_OK;
}

}  // namespace

extern "C" {

int attn_abi_version(void) { return ATTN_ABI_VERSION; }

const char *attn_status_string(int status)
{
    switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_NULL_ARG: return "null argument";
    case ATTN_ERR_GEOMETRY: return "unsupported geometry";
    case ATTN_ERR_RANGE: return "argument out of range";
    case ATTN_ERR_ALIGN: return "misaligned q_base or pointer";
    case ATTN_ERR_DEVICE: return "device unavailable or not the context's device";
    case ATTN_ERR_NOMEM: return "workspace allocation failed";
    case ATTN_ERR_LAUNCH: return "kernel launch failed";
    default: return "unknown status";
    }
}

int attn_validate(const attn_geometry *geom, const attn_inputs *in, int32_t T, int32_t q_base,
                  int32_t kind, const void *mask, const void *out)
{
    int rc = check_geometry(geom);
    if (rc != ATTN_OK)
        return rc;
    if (kind < 0 || kind >= kKinds)
        return ATTN_ERR_RANGE;
    if (T < 0 || T > geom->max_tokens)
        return ATTN_ERR_RANGE;
    if (q_base < 0 || q_base > T)
        return ATTN_ERR_RANGE;
    if (kind != 1 && kind != 4 && kind != 5 && q_base != 0)
        return ATTN_ERR_RANGE;
    if (q_base % ATTN_QBASE_ALIGN != 0)
        return ATTN_ERR_ALIGN;
    if (T - q_base == 0)
        return ATTN_OK;             // empty launch: no-op, pointers unused
    if (!in || !out)
        return ATTN_ERR_NULL_ARG;
    if (!in->qg || !in->k || !in->v || !in->q_norm_w || !in->k_norm_w || !in->cos_tab || !in->sin_tab)
        return ATTN_ERR_NULL_ARG;
    if ((kind == 2 || kind == 4 || kind == 5) && !mask)
        return ATTN_ERR_NULL_ARG;
    if (in->n_pos < T)
        return ATTN_ERR_RANGE;
    if (!aligned16(in->qg) || !aligned16(in->k) || !aligned16(in->v) || !aligned16(in->q_norm_w) ||
        !aligned16(in->k_norm_w) || !aligned16(in->cos_tab) || !aligned16(in->sin_tab) || !aligned16(out))
        return ATTN_ERR_ALIGN;
    if ((kind == 4 || kind == 5) && !aligned16(mask))
        return ATTN_ERR_ALIGN;
    return ATTN_OK;
}

int attn_ctx_create(const attn_geometry *geom, int device, attn_ctx **out)
{
    if (!out)
        return ATTN_ERR_NULL_ARG;
    *out = nullptr;
    int rc = check_geometry(geom);
    if (rc != ATTN_OK)
        return rc;
    int ndev = 0;
    if (hipGetDeviceCount(&ndev) != hipSuccess || device < 0 || device >= ndev) {
        (void)hipGetLastError();
        return ATTN_ERR_DEVICE;
    }
    if (hipSetDevice(device) != hipSuccess)
        return ATTN_ERR_DEVICE;
    attn_ctx *ctx = new (std::nothrow) attn_ctx;
    if (!ctx)
        return ATTN_ERR_NOMEM;
    ctx->device = device;
    ctx->geom = *geom;
    if (hipDeviceGetAttribute(&ctx->num_cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess ||
        ctx->num_cus <= 0) {
        (void)hipGetLastError();
        delete ctx;
        return ATTN_ERR_DEVICE;
    }
    ctx->tpad = (geom->max_tokens + 63) / 64 * 64;
    ctx->mask_words = (geom->max_tokens + 31) / 32;
    const size_t kv_elems = (size_t)geom->n_kv_heads * ctx->tpad * ATTN_HEAD_DIM;
    const size_t nrb = (size_t)(geom->max_tokens + 63) / 64;
    bool ok = hipMalloc(&ctx->kp, kv_elems * 2) == hipSuccess &&
              hipMalloc(&ctx->vt, kv_elems * 2) == hipSuccess &&
              hipMalloc(&ctx->mask_bits, (size_t)ctx->tpad * ctx->mask_words * 4) == hipSuccess &&
              hipMalloc(&ctx->tile_vis, nrb * ctx->mask_words) == hipSuccess &&
              hipMalloc(&ctx->row_stats, (size_t)geom->max_tokens * geom->n_q_heads * 2 * sizeof(float)) ==
                  hipSuccess;
    ctx->batch_cap = batch_table_ints(ctx->tpad);
    ok = ok && hipMalloc(&ctx->batch_tab, ctx->batch_cap * sizeof(int)) == hipSuccess &&
         hipHostMalloc(&ctx->batch_host, ctx->batch_cap * sizeof(int), hipHostMallocDefault) == hipSuccess &&
         hipEventCreateWithFlags(&ctx->batch_copied, hipEventDisableTiming) == hipSuccess;
    const int n_hg = (geom->n_q_heads / geom->n_kv_heads + ga::kHeadsPerBlock - 1) / ga::kHeadsPerBlock;
    // offsets for the workgroups, then the entries: every item once, or both
    // halves of a split one
    ctx->sched_cap = (size_t)ctx->num_cus + 1 + 2 * std::max<size_t>(nrb * geom->n_kv_heads * n_hg, ctx->num_cus);
    ok = ok && hipMalloc(&ctx->sched_tab, ctx->sched_cap * sizeof(int)) == hipSuccess &&
         hipHostMalloc(&ctx->sched_host, ctx->sched_cap * sizeof(int), hipHostMallocDefault) == hipSuccess &&
         hipEventCreateWithFlags(&ctx->sched_copied, hipEventDisableTiming) == hipSuccess;
    if (!ok) {
        (void)hipGetLastError();
        attn_ctx_destroy(ctx);
        return ATTN_ERR_NOMEM;
    }
    *out = ctx;
    return ATTN_OK;
}

void attn_ctx_destroy(attn_ctx *ctx)
{
    if (!ctx)
        return;
    int prev = -1;
    (void)hipGetDevice(&prev);
    if (prev != ctx->device)
        (void)hipSetDevice(ctx->device);
    (void)hipFree(ctx->kp);
    (void)hipFree(ctx->vt);
    (void)hipFree(ctx->mask_bits);
    (void)hipFree(ctx->tile_vis);
    (void)hipFree(ctx->row_stats);
    (void)hipFree(ctx->batch_tab);
    if (ctx->batch_host)
        (void)hipHostFree(ctx->batch_host);
    if (ctx->batch_copied)
        (void)hipEventDestroy(ctx->batch_copied);
    (void)hipFree(ctx->sched_tab);
    if (ctx->sched_host)
        (void)hipHostFree(ctx->sched_host);
    if (ctx->sched_copied)
        (void)hipEventDestroy(ctx->sched_copied);
    for (hipEvent_t e : ctx->pool)
        (void)hipEventDestroy(e);
    if (prev >= 0 && prev != ctx->device)
        (void)hipSetDevice(prev);
    delete ctx;
}

int attn_prefill_gated(attn_ctx *ctx, const attn_inputs *in, int32_t S, void *out, void *stream)
{
    return run(ctx, in, S, 0, 0, nullptr, out, stream);
}

int attn_prefill_gated_noalloc(const attn_geometry *geom, const attn_inputs *in, int32_t S, void *out,
                               void *stream)
{
    static_assert(ga::kNoallocScratchBytes == ATTN_NOALLOC_SCRATCH_BYTES, "scratch size");
    int rc = attn_validate(geom, in, S, 0, 0, nullptr, out);
    if (rc != ATTN_OK)
        return rc;
    if (S == 0)
        return ATTN_OK;
    if (noalloc_bytes(*geom, S) > ga::kNoallocScratchBytes)
        return ATTN_ERR_RANGE;
    int device = -1, num_cus = 0;
    if (hipGetDevice(&device) != hipSuccess ||
        hipDeviceGetAttribute(&num_cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess ||
        num_cus <= 0) {
        (void)hipGetLastError();
        return ATTN_ERR_DEVICE;
    }
    uint16_t *scr = nullptr;
    if (ga::noalloc_scratch(device, &scr) != hipSuccess) {
        (void)hipGetLastError();
        return ATTN_ERR_DEVICE;
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    // The scratch holds this call's prepared keys, then its transposed values;
    // every tile the attention reads is written by this call's prologue first.
    const int tpad = (S + 63) / 64 * 64;
    uint16_t *kp_ws = scr, *vt_ws = scr + (size_t)geom->n_kv_heads * tpad * ATTN_HEAD_DIM;
    ga::KvPrologueParams kvp;
    fill_kv_params_ws(kvp, *geom, kp_ws, vt_ws, tpad, in, S);
    if (ga::launch_kv_prologue(kvp, (S + ga::kKeysPerTile - 1) / ga::kKeysPerTile, s) != hipSuccess)
        return ATTN_ERR_LAUNCH;
    ga::AttnParams ap;
    fill_attn_params_ws(ap, *geom, kp_ws, vt_ws, tpad, num_cus, in, S, 0, out);
    if (ga::launch_attention(ap, ga::AttnMode::Causal, s) != hipSuccess)
        return ATTN_ERR_LAUNCH;
    return ATTN_OK;
}

int attn_prefill_prefix(attn_ctx *ctx, const attn_inputs *in, int32_t T, int32_t q_base, void *out,
                        void *stream)
{
    return run(ctx, in, T, q_base, 1, nullptr, out, stream);
}

int attn_prefill_masked(attn_ctx *ctx, const attn_inputs *in, int32_t S, const uint8_t *mask, void *out,
                        void *stream)
{
    return run(ctx, in, S, 0, 2, mask, out, stream);
}

int attn_validate_weights(const attn_geometry *geom, const attn_inputs *in, int32_t T, int32_t q_base,
                          int32_t kind, const void *mask, const void *out, const void *weights)
{
    if (!geom)
        return ATTN_ERR_NULL_ARG;
    if (kind < 0 || kind > 3)
        return ATTN_ERR_RANGE;   // the cache kinds have no weights variant
    int rc = attn_validate(geom, in, T, q_base, kind, mask, out);
    if (rc != ATTN_OK || T - q_base == 0)
        return rc;
    if (!weights)
        return ATTN_ERR_NULL_ARG;
    if (!aligned16(weights))
        return ATTN_ERR_ALIGN;
    return ATTN_OK;
}

int attn_prefill_weights(attn_ctx *ctx, const attn_inputs *in, int32_t T, int32_t q_base, int32_t kind,
                         const uint8_t *mask, void *out, void *weights, void *stream)
{
    if (!ctx)
        return ATTN_ERR_NULL_ARG;
    int rc = attn_validate_weights(&ctx->geom, in, T, q_base, kind, mask, out, weights);
    if (rc != ATTN_OK)
        return rc;
    return run(ctx, in, T, q_base, kind, kind == 2 ? mask : nullptr, out, stream, weights);
}

int attn_kv_cache_bytes(const attn_geometry *geom, size_t *bytes)
{
    if (!bytes)
        return ATTN_ERR_NULL_ARG;
    *bytes = 0;
    const int rc = check_geometry(geom);
    if (rc != ATTN_OK)
        return rc;
    *bytes = kv_cache_bytes(*geom);
    return ATTN_OK;
}

int attn_prefill_append(attn_ctx *ctx, const attn_inputs *in, int32_t T, int32_t q_base, void *kv_cache,
                        void *out, void *stream)
{
    return run(ctx, in, T, q_base, 4, static_cast<const uint8_t *>(kv_cache), out, stream);
}

int attn_kv_cache_fp8_bytes(const attn_geometry *geom, size_t *bytes)
{
    if (!bytes)
        return ATTN_ERR_NULL_ARG;
    *bytes = 0;
    const int rc = check_geometry(geom);
    if (rc != ATTN_OK)
        return rc;
    *bytes = kv_cache_fp8_bytes(*geom);
    return ATTN_OK;
}

int attn_prefill_append_fp8(attn_ctx *ctx, const attn_inputs *in, int32_t T, int32_t q_base, void *kv_cache8,
                            void *out, void *stream)
{
    return run(ctx, in, T, q_base, 5, static_cast<const uint8_t *>(kv_cache8), out, stream);
}

int attn_prefill_bidirectional(attn_ctx *ctx, const attn_inputs *in, int32_t S, void *out, void *stream)
{
    return run(ctx, in, S, 0, 3, nullptr, out, stream);
}

int attn_validate_batch(const attn_geometry *geom, const attn_inputs *in, int32_t n_seqs, const int32_t *seq_lens,
                        const void *out)
{
    int rc = check_geometry(geom);
    if (rc != ATTN_OK)
        return rc;
    BatchPlan pl;
    rc = plan_batch(*geom, n_seqs, seq_lens, &pl, nullptr);
    if (rc != ATTN_OK)
        return rc;
    if (pl.total == 0)
        return ATTN_OK;             // nothing to do: pointers unused
    if (!in || !out)
        return ATTN_ERR_NULL_ARG;
    if (!in->qg || !in->k || !in->v || !in->q_norm_w || !in->k_norm_w || !in->cos_tab || !in->sin_tab)
        return ATTN_ERR_NULL_ARG;
    if (in->n_pos < pl.max_len)
        return ATTN_ERR_RANGE;
    if (!aligned16(in->qg) || !aligned16(in->k) || !aligned16(in->v) || !aligned16(in->q_norm_w) ||
        !aligned16(in->k_norm_w) || !aligned16(in->cos_tab) || !aligned16(in->sin_tab) || !aligned16(out))
        return ATTN_ERR_ALIGN;
    return ATTN_OK;
}

int attn_prefill_gated_batch(attn_ctx *ctx, const attn_inputs *in, int32_t n_seqs, const int32_t *seq_lens,
                             void *out, void *stream)
{
    if (!ctx)
        return ATTN_ERR_NULL_ARG;
    int rc = attn_validate_batch(&ctx->geom, in, n_seqs, seq_lens, out);
    if (rc != ATTN_OK)
        return rc;
    return run_batch(ctx, in, n_seqs, seq_lens, 0, nullptr, out, stream);
}

int attn_validate_shared_batch(const attn_geometry *geom, const attn_inputs *in, int32_t prefix_len,
                               const void *kv_cache, int32_t n_branches, const int32_t *branch_lens, const void *out)
{
    int rc = check_geometry(geom);
    if (rc != ATTN_OK)
        return rc;
    if (prefix_len < 0 || prefix_len > geom->max_tokens)
        return ATTN_ERR_RANGE;
    if (prefix_len % ATTN_QBASE_ALIGN != 0)
        return ATTN_ERR_ALIGN;
    BatchPlan pl;
    rc = plan_batch(*geom, n_branches, branch_lens, &pl, nullptr);
    if (rc != ATTN_OK)
        return rc;
    if ((int64_t)prefix_len + pl.max_len > geom->max_tokens)
        return ATTN_ERR_RANGE;      // a branch's positions past the geometry
    if (pl.total == 0)
        return ATTN_OK;             // nothing to do: pointers unused
    if (!in || !out)
        return ATTN_ERR_NULL_ARG;
    if (!in->qg || !in->k || !in->v || !in->q_norm_w || !in->k_norm_w || !in->cos_tab || !in->sin_tab)
        return ATTN_ERR_NULL_ARG;
    if (prefix_len > 0 && !kv_cache)
        return ATTN_ERR_NULL_ARG;
    if (in->n_pos < (int64_t)prefix_len + pl.max_len)
        return ATTN_ERR_RANGE;
    if (!aligned16(in->qg) || !aligned16(in->k) || !aligned16(in->v) || !aligned16(in->q_norm_w) ||
        !aligned16(in->k_norm_w) || !aligned16(in->cos_tab) || !aligned16(in->sin_tab) || !aligned16(out))
        return ATTN_ERR_ALIGN;
    if (kv_cache && !aligned16(kv_cache))
        return ATTN_ERR_ALIGN;
    return ATTN_OK;
}

int attn_prefill_shared_batch(attn_ctx *ctx, const attn_inputs *in, int32_t prefix_len, const void *kv_cache,
                              int32_t n_branches, const int32_t *branch_lens, void *out, void *stream)
{
    if (!ctx)
        return ATTN_ERR_NULL_ARG;
    int rc = attn_validate_shared_batch(&ctx->geom, in, prefix_len, kv_cache, n_branches, branch_lens, out);
    if (rc != ATTN_OK)
        return rc;
    return run_batch(ctx, in, n_branches, branch_lens, prefix_len, kv_cache, out, stream);
}

#ifdef ATTN_TEST_HOOKS
int attn_debug_prepare(attn_ctx *ctx, const attn_inputs *in, int32_t T, int32_t q_base, void *qp_out,
                       void *kp_out, void *stream)
{
    if (!ctx)
        return ATTN_ERR_NULL_ARG;
    if (T - q_base != 0 && !qp_out && !kp_out)
        return ATTN_ERR_NULL_ARG;
    int rc = attn_validate(&ctx->geom, in, T, q_base, 1, nullptr, qp_out ? qp_out : kp_out);
    if (rc != ATTN_OK)
        return rc;
    if ((qp_out && !aligned16(qp_out)) || (kp_out && !aligned16(kp_out)))
        return ATTN_ERR_ALIGN;
    if (T - q_base == 0)
        return ATTN_OK;
    rc = current_device_matches(ctx);
    if (rc != ATTN_OK)
        return rc;
    hipStream_t s = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    if (kp_out) {
        ga::KvPrologueParams kvp;
        fill_kv_params(kvp, ctx, in, T);
        if (ga::launch_kv_prologue(kvp, (T + ga::kKeysPerTile - 1) / ga::kKeysPerTile, s) != hipSuccess)
            return ATTN_ERR_LAUNCH;
        if (ga::launch_kp_unpack(ctx->kp, ctx->tpad, T, ctx->geom.n_kv_heads, static_cast<uint16_t *>(kp_out),
                                 s) != hipSuccess)
            return ATTN_ERR_LAUNCH;
    }
    if (qp_out) {
        ga::AttnParams ap;
        fill_attn_params(ap, ctx, in, T, q_base, nullptr);
        if (ga::launch_q_prologue_debug(ap, static_cast<uint16_t *>(qp_out), s) != hipSuccess)
            return ATTN_ERR_LAUNCH;
    }
    return ATTN_OK;
}

int attn_debug_fp8_encode(const float *x, const float *sc, float *q, uint8_t *codes, int64_t n, void *stream)
{
    if (n < 0 || n > ((int64_t)1 << 30))
        return ATTN_ERR_RANGE;
    if (n == 0)
        return ATTN_OK;
    if (!x || !sc || !q || !codes)
        return ATTN_ERR_NULL_ARG;
    (void)hipGetLastError();
    if (ga::launch_fp8_encode_debug(x, sc, q, codes, n, static_cast<hipStream_t>(stream)) != hipSuccess)
        return ATTN_ERR_LAUNCH;
    return ATTN_OK;
}
#endif  // ATTN_TEST_HOOKS

int attn_ctx_set_timing_mask(attn_ctx *ctx, int kernel_mask)
{
    if (!ctx)
        return ATTN_ERR_NULL_ARG;
    if (kernel_mask & ~ATTN_TIMING_ALL)
        return ATTN_ERR_RANGE;
    if (current_device_matches(ctx) != ATTN_OK)
        return ATTN_ERR_DEVICE;
    if (kernel_mask && ctx->pool.empty()) {
        // Timing-only events: no system-scope fence when they are recorded,
        // so recording one neither writes back and invalidates the caches
        // around the timed kernel nor slows the work that follows it.
        for (int i = 0; i < 8192; ++i) {
            hipEvent_t e;
            if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess)
                return ATTN_ERR_NOMEM;
            ctx->pool.push_back(e);
        }
    }
    ctx->timing = kernel_mask;
    ctx->pool_used = 0;
    ctx->recs.clear();
    return ATTN_OK;
}

int attn_ctx_set_timing(attn_ctx *ctx, int enable)
{
    return attn_ctx_set_timing_mask(ctx, enable ? ATTN_TIMING_ALL : 0);
}

int attn_ctx_read_timing(attn_ctx *ctx, int kernel, double *total_ms, int32_t *launches)
{
    if (!ctx || !total_ms || !launches)
        return ATTN_ERR_NULL_ARG;
    if (kernel < 0 || kernel > ATTN_KERNEL_WEIGHTS)
        return ATTN_ERR_RANGE;
    if (current_device_matches(ctx) != ATTN_OK)
        return ATTN_ERR_DEVICE;
    double sum = 0.0;
    int n = 0;
    std::vector<attn_ctx::Rec> keep;
    for (const auto &r : ctx->recs) {
        if (r.kernel != kernel) {
            keep.push_back(r);
            continue;
        }
        if (hipEventSynchronize(r.b) != hipSuccess)
            return ATTN_ERR_LAUNCH;
        float ms = 0.0f;
        if (hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess)
            return ATTN_ERR_LAUNCH;
        sum += ms;
        ++n;
    }
    ctx->recs.swap(keep);
    if (ctx->recs.empty())
        ctx->pool_used = 0;
    *total_ms = sum;
    *launches = n;
    return ATTN_OK;
}

int attn_mfma_clock_probe(int32_t iters, void *stream, double *mhz, double *tflops)
{
    if (!mhz || !tflops)
        return ATTN_ERR_NULL_ARG;
    if (iters < 1 || iters > 10000000)
        return ATTN_ERR_RANGE;
    int device = 0, cus = 0;
    if (hipGetDevice(&device) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess || cus <= 0)
        return ATTN_ERR_DEVICE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    long long *rec = nullptr;
    float *sink = nullptr;
    if (hipMalloc(&rec, sizeof(long long) * 2 * cus) != hipSuccess)
        return ATTN_ERR_NOMEM;
    if (hipMalloc(&sink, sizeof(float) * 256 * cus) != hipSuccess) {
        (void)hipFree(rec);
        return ATTN_ERR_NOMEM;
    }
    std::vector<long long> h(2 * (size_t)cus);
    int rc = ATTN_OK;
    if (ga::launch_mfma_clock_probe(iters, cus, rec, sink, s) != hipSuccess || hipStreamSynchronize(s) != hipSuccess ||
        hipMemcpy(h.data(), rec, sizeof(long long) * 2 * cus, hipMemcpyDeviceToHost) != hipSuccess)
        rc = ATTN_ERR_LAUNCH;
    (void)hipFree(rec);
    (void)hipFree(sink);
    if (rc != ATTN_OK)
        return rc;
    double cyc = 0.0, ticks = 0.0;
    for (int i = 0; i < cus; ++i) {
        cyc += (double)h[2 * i];
        ticks += (double)h[2 * i + 1];
    }
    cyc /= cus;
    ticks /= cus;
    if (ticks <= 0.0)
        return ATTN_ERR_LAUNCH;
    const double seconds = ticks / 100.0e6;
    *mhz = cyc / seconds / 1.0e6;
    *tflops = (double)cus * 4.0 * iters * 16.0 * 32768.0 / seconds / 1.0e12;
    return ATTN_OK;
}

}  // extern "C"
