// zero_api.cpp -- the C ABI of the per-rank ZeRO shard step in all its forms
// (fused ZeRO-1, composed, ZeRO-2 streaming, CPU-offloaded, and their
// dynamic-loss-scale variants): argument checks, host-side scalar
// derivation, element layouts, the workspace plans and the launch sequences.
// Every GPU kernel is in zero_kernels.hip; the host optimizer of the
// CPU-offloaded step is in zero_host_adamw.cpp.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <limits>
#include <map>
#include <memory>
#include <mutex>
#include <utility>
#include <vector>

#include "zero_host.h"
#include "zero_internal.h"
#include "zero_step.h"

using namespace zero;

namespace {

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

bool is_fin(double x) { return std::isfinite(x); }

// The kernels multiply by grad_scale rounded to binary32 once, so that
// rounding must be a finite normal binary32 value: a scale that rounds to 0
// would zero every gradient, one that rounds to +inf would flag every step.
bool scale_ok(double s)
{
    if (!is_fin(s) || !(s > 0.0)) return false;
    const float f = static_cast<float>(s);
    return std::isfinite(f) && f >= std::numeric_limits<float>::min();
}

// The other ranks' sum of squares: NaN and +inf pass into the norm (a rank
// saw a non-finite gradient); a negative value is no sum of squares.
bool external_ok(double x) { return !(x < 0.0); }

bool hparams_ok(const zero_adamw_hparams* hp)
{
    if (hp == nullptr) return false;
    if (!is_fin(hp->lr) || hp->lr < 0.0) return false;
    if (!(hp->beta1 >= 0.0 && hp->beta1 < 1.0)) return false;
    if (!(hp->beta2 >= 0.0 && hp->beta2 < 1.0)) return false;
    if (!is_fin(hp->eps) || hp->eps < 0.0) return false;
    if (!is_fin(hp->weight_decay)) return false;
    if (hp->step < 1) return false;
    if (std::isnan(hp->max_grad_norm)) return false;
    if (!scale_ok(hp->grad_scale)) return false;
    if (hp->reserved != 0) return false;
    return true;
}

// The binary64 scalars of one step.
AdamScalars derive(const zero_adamw_hparams* hp)
{
    const double t = static_cast<double>(hp->step);
    AdamScalars c;
    c.b1 = hp->beta1;
    c.omb1 = 1.0 - hp->beta1;
    c.b2 = hp->beta2;
    c.omb2 = 1.0 - hp->beta2;
    c.decay = 1.0 - hp->lr * hp->weight_decay;
    c.lr = hp->lr;
    c.bc1 = 1.0 - std::pow(hp->beta1, t);
    c.bc2 = 1.0 - std::pow(hp->beta2, t);
    c.eps = hp->eps;
    return c;
}

bool loss_scale_config_ok(const zero_loss_scale_config* c)
{
    return c != nullptr && c->initial_scale_power >= -126 && c->initial_scale_power <= 127 && c->window >= 1 &&
           c->hysteresis >= 1 && std::isfinite(c->min_scale) && c->min_scale > 0.0f;
}

bool two_pass_of(const zero_adamw_hparams* hp) { return hp->max_grad_norm > 0.0 || hp->skip_on_nonfinite != 0; }

// Vector mode needs one head length h in [0, 8) at which every bf16 pointer
// (2-byte elements) and every fp32 pointer (4-byte elements) is 16-byte
// aligned; otherwise the shard is visited element by element.
Layout make_layout(int64_t n, const std::vector<uintptr_t>& b16, const std::vector<uintptr_t>& f32)
{
    Layout L{n, -1, 0, 0};
    if (n <= 0) return L;
    for (int h = 0; h < kVec; ++h) {
        bool ok = true;
        for (uintptr_t p : b16)
            if ((p + 2u * h) % 16u != 0) { ok = false; break; }
        if (ok)
            for (uintptr_t p : f32)
                if ((p + 4u * h) % 16u != 0) { ok = false; break; }
        if (!ok) continue;
        if (h > n) break;
        L.head = h;
        L.nvec = (n - h) / kVec;
        L.tail = static_cast<int32_t>(n - h - kVec * L.nvec);
        return L;
    }
    return L;
}

int grid_for(int64_t tiles, int resident)
{
    if (tiles <= 0) return 1;
    return static_cast<int>(tiles < resident ? tiles : resident);
}

int hip_status(hipError_t e) { return e == hipSuccess ? ZERO_OK : ZERO_ERR_HIP; }

int64_t tiles_of(const std::vector<Layout>& layouts, int geom)
{
    const int64_t tv = static_cast<int64_t>(kGeoms[geom].nt) * kGeoms[geom].u;
    int64_t tiles = 0;
    for (const Layout& L : layouts) tiles += layout_tiles(L, tv);
    return tiles;
}

// Geometry of the pass that folds the replicas: long per-replica bursts in
// workgroup lockstep -- for a single pass 512 threads x 16 vectors (128 KiB of
// one replica per workgroup, registers to spare for the binary64 update) when
// the replica reads dominate (M > 16), else 256 x 16, whose two workgroups
// per CU overlap one's state update with the other's fold; for a first pass
// that only folds (two-pass step, bucket reduce, offloaded fold), 512 x 16
// from four tiles per CU on, below that 1024 x 8 (more waves per tile) --
// unless the bucket is too small to reach half the compute units.
int pick_geom_fold(const std::vector<Layout>& layouts, int M, bool two_pass, int cus)
{
    int first;
    if (!two_pass)
        first = M > 16 ? 5 : 6;
    else
        first = tiles_of(layouts, 5) >= 4 * static_cast<int64_t>(cus) ? 5 : 4;
    if (2 * tiles_of(layouts, first) >= static_cast<int64_t>(cus)) return first;
    for (int g = 3; g > 0; --g)
        if (2 * tiles_of(layouts, g) >= static_cast<int64_t>(cus)) return g;
    return 0;
}

// Geometry of the update pass of a two-pass step (no replica streams):
// small tiles, like any read-modify-write stream.
int pick_geom_update(const std::vector<Layout>& layouts, int cus)
{
    (void)layouts;
    (void)cus;
    return 0;
}

// ------------------------------------------------------------------ plans

bool kind_folds(PlanKind k) { return k != PlanKind::AccStep; }
// the fp32 gradient of the fold pass is kept in the workspace
bool kind_keeps_g(PlanKind k) { return k == PlanKind::StepTwoPass || k == PlanKind::Fold; }
bool kind_updates_after(PlanKind k) { return k == PlanKind::StepTwoPass || k == PlanKind::AccStep; }

PlanOffsets plan_offsets(const std::vector<int64_t>& ns, int32_t M, PlanKind kind)
{
    PlanOffsets o{};
    const size_t T = ns.size();
    int64_t tiles = 0;  // bound over every geometry (the smallest tile is kTileElems)
    size_t gbytes = 0;
    for (int64_t n : ns) {
        tiles += tiles_bound(n);
        if (kind_keeps_g(kind) && n > 0) gbytes += align_up((static_cast<size_t>(n) + 3) * 4, kAlign);
    }
    const size_t ntiles = static_cast<size_t>(tiles);
    const bool folds = kind_folds(kind);
    o.desc = kAlign;
    o.ptrs = align_up(o.desc + sizeof(TensorDesc) * T, kAlign);
    o.map0 = align_up(o.ptrs + (folds ? sizeof(void*) * T * static_cast<size_t>(M) : 0), kAlign);
    o.map1 = align_up(o.map0 + (folds ? sizeof(TileRef) * ntiles : 0), kAlign);
    o.parts = align_up(o.map1 + (kind_updates_after(kind) ? sizeof(TileRef) * ntiles : 0), kAlign);
    o.gbuf = align_up(o.parts + (folds ? sizeof(Partial) * ntiles : 0), kAlign);
    o.total = o.gbuf + gbytes;
    return o;
}

uint64_t fnv1a(const uint8_t* p, size_t n, uint64_t h)
{
    for (size_t i = 0; i < n; ++i) {
        h ^= p[i];
        h *= 1099511628211ull;
    }
    return h;
}

std::mutex g_plan_mu;
std::map<std::pair<int, uintptr_t>, uint64_t> g_plan_cache;  // (device, ws) -> signature held there

void forget_ws(const void* ws)
{
    std::lock_guard<std::mutex> lk(g_plan_mu);
    for (auto it = g_plan_cache.begin(); it != g_plan_cache.end();) {
        if (it->first.second == reinterpret_cast<uintptr_t>(ws)) it = g_plan_cache.erase(it);
        else ++it;
    }
}

// One tensor of a plan: the M replica pointers of the passes that fold them,
// the state and output of the passes that update, and the caller's fp32
// gradient buffer of the bucket and accumulated-step plans.
struct PlanTensor {
    int64_t n = 0;
    const void* const* grads = nullptr;
    float* master = nullptr;
    float* m = nullptr;
    float* v = nullptr;
    void* out = nullptr;
    float* acc = nullptr;
};

struct Plan {
    std::vector<float*> gbuf;  // per tensor: the fp32 gradient the fold pass writes (null unless kept)
    std::vector<Layout> layouts;        // per tensor: the element layout the kernels follow
    std::vector<int64_t> fold_begin;    // per tensor: its first tile in the fold pass's map
    std::vector<int64_t> fold_tiles;    // per tensor: its tiles in the fold pass
    PlanOffsets off;
    int geom[2];
    int64_t tiles[2];
    uint64_t sig;
    PlanHeader* hdr;
    TensorDesc* desc;
    TileRef* map0;
    TileRef* map1;
    Partial* parts;
    unsigned* counter;
};

// Builds the plan of `kind` for these tensors in `ws` (tables, tile maps,
// header with its signature), uploading it unless the workspace already
// holds it. Returns a status.
int make_plan(const std::vector<PlanTensor>& ts, int32_t M, PlanKind kind, void* ws, size_t ws_bytes,
              hipStream_t stream, Plan* plan)
{
    if (ws == nullptr || reinterpret_cast<uintptr_t>(ws) % kAlign != 0) return ZERO_ERR_INVALID_ARGUMENT;
    const int32_t T = static_cast<int32_t>(ts.size());
    std::vector<int64_t> ns;
    for (const PlanTensor& x : ts) ns.push_back(x.n);
    const bool folds = kind_folds(kind), updates = kind_updates_after(kind);
    const PlanOffsets off = plan_offsets(ns, M, kind);
    if (ws_bytes < off.total) return ZERO_ERR_WORKSPACE_TOO_SMALL;

    // ---- header, tensor table, rank-pointer table (host image)
    uint8_t* wsb = static_cast<uint8_t*>(ws);
    std::vector<uint8_t> blob(off.map0, 0);
    PlanHeader* hdr = reinterpret_cast<PlanHeader*>(blob.data());
    TensorDesc* desc = reinterpret_cast<TensorDesc*>(blob.data() + off.desc);
    const uint16_t** ptrs = reinterpret_cast<const uint16_t**>(blob.data() + off.ptrs);
    std::vector<Layout> layouts(static_cast<size_t>(T));
    for (int32_t t = 0; t < T; ++t) {
        const PlanTensor& x = ts[t];
        if (x.n == 0) {
            layouts[t] = Layout{0, -1, 0, 0};
            continue;
        }
        std::vector<uintptr_t> b16, f32;
        if (folds)
            for (int32_t r = 0; r < M; ++r) b16.push_back(reinterpret_cast<uintptr_t>(x.grads[r]));
        if (x.out) b16.push_back(reinterpret_cast<uintptr_t>(x.out));
        for (const float* p : {x.acc, x.master, x.m, x.v})
            if (p) f32.push_back(reinterpret_cast<uintptr_t>(p));
        layouts[t] = make_layout(x.n, b16, f32);
    }
    const int cus = compute_units();
    // the single-pass plans (the fused step, a bucket's fused final pass) take
    // the single-pass fold geometry; every other fold pass only folds
    const bool fold_only = !(kind == PlanKind::Step || kind == PlanKind::BucketStep);
    const int geom[2] = {folds ? pick_geom_fold(layouts, M, fold_only, cus) : 0,
                         updates ? pick_geom_update(layouts, cus) : 0};
    const int64_t tile_vecs[2] = {static_cast<int64_t>(kGeoms[geom[0]].nt) * kGeoms[geom[0]].u,
                                  static_cast<int64_t>(kGeoms[geom[1]].nt) * kGeoms[geom[1]].u};
    int64_t tiles[2] = {0, 0};
    size_t gpos = off.gbuf;
    for (int32_t t = 0; t < T; ++t) {
        const PlanTensor& x = ts[t];
        TensorDesc& d = desc[t];
        d.grads = folds ? reinterpret_cast<const uint16_t* const*>(wsb + off.ptrs + sizeof(void*) * static_cast<size_t>(t) * M)
                        : nullptr;
        d.n = x.n;
        for (int p = 0; p < 2; ++p) d.tile_begin[p] = tiles[p];
        if (x.n == 0) {
            d.nvec = -1;
            continue;
        }
        if (folds)
            for (int32_t r = 0; r < M; ++r)
                ptrs[static_cast<size_t>(t) * M + r] = static_cast<const uint16_t*>(x.grads[r]);
        const Layout& L = layouts[t];
        d.master = x.master;
        d.exp_avg = x.m;
        d.exp_avg_sq = x.v;
        d.out = static_cast<uint16_t*>(x.out);
        d.nvec = L.nvec;
        d.head = L.head;
        d.tail = L.tail;
        d.ntiles[0] = folds ? layout_tiles(L, tile_vecs[0]) : 0;
        d.ntiles[1] = updates ? layout_tiles(L, tile_vecs[1]) : 0;
        if (kind_keeps_g(kind)) {
            // aligned with the other pointers at element `head`
            const size_t shift = L.nvec >= 0 ? 4u * ((4u - static_cast<unsigned>(L.head) % 4u) % 4u) : 0u;
            d.gbuf = reinterpret_cast<float*>(wsb + gpos + shift);
            gpos += align_up((static_cast<size_t>(x.n) + 3) * 4, kAlign);
        } else {
            d.gbuf = x.acc;
        }
        for (int p = 0; p < 2; ++p) tiles[p] += d.ntiles[p];
    }
    // one workgroup per tile: a pass launches at most 2^31 - 1 of them
    if (tiles[0] > 0x7FFFFFFF || tiles[1] > 0x7FFFFFFF) return ZERO_ERR_INVALID_ARGUMENT;
    hdr->tiles[0] = tiles[0];
    hdr->tiles[1] = tiles[1];
    hdr->T = T;
    hdr->M = M;
    hdr->geom[0] = geom[0];
    hdr->geom[1] = geom[1];
    hdr->two_pass = kind == PlanKind::StepTwoPass ? 1 : 0;
    hdr->kind = static_cast<int32_t>(kind);
    uint64_t sig = fnv1a(blob.data(), blob.size(), 1469598103934665603ull);
    const uintptr_t wsaddr = reinterpret_cast<uintptr_t>(ws);
    sig = fnv1a(reinterpret_cast<const uint8_t*>(&wsaddr), sizeof(wsaddr), sig);
    if (sig == 0) sig = 1;
    hdr->signature = sig;

    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return ZERO_ERR_HIP;
    const auto key = std::make_pair(dev, wsaddr);
    bool cached;
    {
        std::lock_guard<std::mutex> lk(g_plan_mu);
        auto it = g_plan_cache.find(key);
        cached = it != g_plan_cache.end() && it->second == sig;
    }
    plan->gbuf.assign(static_cast<size_t>(T), nullptr);
    plan->layouts = layouts;
    plan->fold_begin.assign(static_cast<size_t>(T), 0);
    plan->fold_tiles.assign(static_cast<size_t>(T), 0);
    for (int32_t t = 0; t < T; ++t) {
        plan->gbuf[t] = desc[t].gbuf;
        plan->fold_begin[t] = desc[t].tile_begin[0];
        plan->fold_tiles[t] = desc[t].ntiles[0];
    }
    plan->off = off;
    plan->geom[0] = geom[0];
    plan->geom[1] = geom[1];
    plan->tiles[0] = tiles[0];
    plan->tiles[1] = tiles[1];
    plan->sig = sig;
    plan->hdr = reinterpret_cast<PlanHeader*>(wsb);
    plan->desc = reinterpret_cast<TensorDesc*>(wsb + off.desc);
    plan->map0 = folds ? reinterpret_cast<TileRef*>(wsb + off.map0) : nullptr;
    plan->map1 = updates ? reinterpret_cast<TileRef*>(wsb + off.map1) : nullptr;
    plan->parts = folds ? reinterpret_cast<Partial*>(wsb + off.parts) : nullptr;
    plan->counter = reinterpret_cast<unsigned*>(wsb + kCounterOffset);
    if (!cached) {
        // tables first, tile maps next, header (with the signature) last
        WriteChunk c;
        const size_t bytes_per = sizeof(c.data);
        for (size_t pos = off.desc; pos < blob.size(); pos += bytes_per) {
            const size_t len = (blob.size() - pos) < bytes_per ? (blob.size() - pos) : bytes_per;
            c.offset = pos;
            c.words = static_cast<uint32_t>(len / 4);
            c.pad = 0;
            std::memcpy(c.data, blob.data() + pos, len);
            if (launch_plan_write(wsb, c, stream) != hipSuccess) return ZERO_ERR_HIP;
        }
        if (launch_plan_tiles(plan->desc, T, plan->map0, plan->map1, stream) != hipSuccess) return ZERO_ERR_HIP;
        c.offset = 0;
        c.words = static_cast<uint32_t>(off.desc / 4);
        c.pad = 0;
        std::memcpy(c.data, blob.data(), off.desc);
        if (launch_plan_write(wsb, c, stream) != hipSuccess) return ZERO_ERR_HIP;
        std::lock_guard<std::mutex> lk(g_plan_mu);
        g_plan_cache[key] = sig;
    }
    return ZERO_OK;
}

std::vector<int64_t> sizes_of(const zero_tensor* ts, int32_t T)
{
    std::vector<int64_t> ns;
    for (int32_t t = 0; t < T; ++t) ns.push_back(ts[t].n);
    return ns;
}

// The fused step; `ls` (with its config `lscfg`) non-null for the AMP form:
// always two-pass, always skipping on a non-finite gradient, the multiplier
// read from the device state, which the fold's last workgroup then moves.
// The arguments of a fused step, checked on the host (nothing launched):
// fills the plan's tensor list and the total element count.
int step_args(const zero_tensor* tensors, int32_t T, int32_t M, const zero_adamw_hparams* hp, double external_sumsq,
              const zero_result* res_dev, std::vector<PlanTensor>* pts, int64_t* total_n)
{
    if (T < 0 || M < 1 || M > ZERO_MAX_RANKS || !hparams_ok(hp) || res_dev == nullptr ||
        !external_ok(external_sumsq))
        return ZERO_ERR_INVALID_ARGUMENT;
    if (T > 0 && tensors == nullptr) return ZERO_ERR_INVALID_ARGUMENT;
    *total_n = 0;
    pts->assign(static_cast<size_t>(T), PlanTensor{});
    for (int32_t t = 0; t < T; ++t) {
        const zero_tensor& x = tensors[t];
        if (x.n < 0) return ZERO_ERR_INVALID_ARGUMENT;
        (*pts)[t].n = x.n;
        if (x.n == 0) continue;
        if (!x.grads || !x.master || !x.exp_avg || !x.exp_avg_sq || !x.param_out) return ZERO_ERR_INVALID_ARGUMENT;
        for (int32_t r = 0; r < M; ++r)
            if (x.grads[r] == nullptr) return ZERO_ERR_INVALID_ARGUMENT;
        (*pts)[t] = PlanTensor{x.n, x.grads, x.master, x.exp_avg, x.exp_avg_sq, x.param_out, nullptr};
        *total_n += x.n;
    }
    return ZERO_OK;
}

int step_impl(const zero_tensor* tensors, int32_t T, int32_t M, const zero_adamw_hparams* hp, double external_sumsq,
              void* ws, size_t ws_bytes, zero_result* res_dev, hipStream_t stream,
              const zero_loss_scale_config* lscfg, zero_loss_scale* ls)
{
    // ---- arguments
    int64_t total_n = 0;
    std::vector<PlanTensor> pts;
    const int arg = step_args(tensors, T, M, hp, external_sumsq, res_dev, &pts, &total_n);
    if (arg != ZERO_OK) return arg;
    const bool amp = ls != nullptr;
    const bool two_pass = amp || two_pass_of(hp);
    const int skip = amp || hp->skip_on_nonfinite != 0;
    if (total_n == 0) {
        hipError_t e = launch_finalize(nullptr, 0, external_sumsq, hp->max_grad_norm, skip, res_dev, stream);
        if (e == hipSuccess && amp) e = launch_loss_scale_update(*lscfg, res_dev, ls, stream);
        return hip_status(e);
    }
    Plan plan;
    const int st = make_plan(pts, M, two_pass ? PlanKind::StepTwoPass : PlanKind::Step, ws, ws_bytes, stream, &plan);
    if (st != ZERO_OK) return st;

    // ---- the step
    const AdamScalars c = derive(hp);
    const float gscale = static_cast<float>(hp->grad_scale);
    const Mode first_mode = two_pass ? Mode::PassA : Mode::Full;
    FinalizeArgs fin{};
    fin.res = res_dev;
    fin.counter = plan.counter;
    fin.external = external_sumsq;
    fin.max_norm = hp->max_grad_norm;
    fin.skip = skip;
    fin.ls = ls;
    fin.scale_from = ls;
    fin.stream = stream_state_stores(total_n);
    if (amp) fin.lscfg = *lscfg;
    hipError_t e = launch_fused(first_mode, plan.geom[0], plan.hdr, plan.desc, plan.map0, plan.tiles[0], plan.sig, M,
                                gscale, c, plan.parts, fin, nullptr, stream);
    if (e != hipSuccess) return ZERO_ERR_HIP;
    if (two_pass) {
        // the stored gradient is already scaled
        FinalizeArgs none{};
        none.stream = stream_state_stores(total_n);
        e = launch_fused(Mode::PassB, plan.geom[1], plan.hdr, plan.desc, plan.map1, plan.tiles[1], plan.sig, M, 1.0f,
                         c, plan.parts, none, res_dev, stream);
        if (e != hipSuccess) return ZERO_ERR_HIP;
    }
    return ZERO_OK;
}

}  // namespace

extern "C" {

const char* zero_status_string(int status)
{
    switch (status) {
    case ZERO_OK: return "ok";
    case ZERO_ERR_INVALID_ARGUMENT: return "invalid argument";
    case ZERO_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case ZERO_ERR_HIP: return "HIP runtime error";
    case ZERO_ERR_STALE_WORKSPACE: return "workspace no longer holds the plan of this call";
    case ZERO_ERR_BUCKET_PARTIALS: return "a bucket partial was not written by a final bucket reduce of this step";
    case ZERO_ERR_SCRATCH_TOO_SMALL:
        return "the call needs more workspace than the library's static scratch holds (ZERO_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown status";
    }
}

int zero_shard_reduce(const void* const* grads, int32_t M, int64_t n, double grad_scale, float* g_out,
                      hipStream_t stream)
{
    if (n < 0 || M < 1 || M > ZERO_MAX_RANKS) return ZERO_ERR_INVALID_ARGUMENT;
    if (!scale_ok(grad_scale)) return ZERO_ERR_INVALID_ARGUMENT;
    if (n == 0) return ZERO_OK;
    if (grads == nullptr || g_out == nullptr) return ZERO_ERR_INVALID_ARGUMENT;
    std::vector<uintptr_t> b16;
    b16.reserve(M);
    for (int32_t r = 0; r < M; ++r) {
        if (grads[r] == nullptr) return ZERO_ERR_INVALID_ARGUMENT;
        b16.push_back(reinterpret_cast<uintptr_t>(grads[r]));
    }
    const Layout L = make_layout(n, b16, {reinterpret_cast<uintptr_t>(g_out)});
    const float scale = static_cast<float>(grad_scale);
    const int64_t tiles = layout_tiles(L);
    for (int32_t r0 = 0; r0 < M; r0 += kInlineRanks) {
        const int Mc = (M - r0) < kInlineRanks ? (M - r0) : kInlineRanks;
        RankPtrs p{};
        for (int j = 0; j < Mc; ++j) p.p[j] = static_cast<const uint16_t*>(grads[r0 + j]);
        const bool first = r0 == 0, last = r0 + Mc == M;
        const int grid = grid_for(tiles, resident_grid_reduce(Mc, first));
        const hipError_t e = launch_reduce(p, Mc, first, last, scale, L, g_out, grid, stream);
        if (e != hipSuccess) return ZERO_ERR_HIP;
    }
    return ZERO_OK;
}

size_t zero_grad_check_norm_workspace_bytes(int64_t n)
{
    return n > 0 ? sizeof(Partial) * static_cast<size_t>(kMaxPartials) : 0;
}

int zero_grad_check_norm(const float* g, int64_t n, const zero_adamw_hparams* hp, double external_sumsq, void* ws,
                         size_t ws_bytes, zero_result* res_dev, hipStream_t stream)
{
    if (n < 0 || res_dev == nullptr || !external_ok(external_sumsq)) return ZERO_ERR_INVALID_ARGUMENT;
    if (hp != nullptr && !hparams_ok(hp)) return ZERO_ERR_INVALID_ARGUMENT;
    const double max_norm = hp ? hp->max_grad_norm : 0.0;
    const int skip = hp ? (hp->skip_on_nonfinite != 0) : 0;
    if (n == 0)
        return hip_status(launch_finalize(nullptr, 0, external_sumsq, max_norm, skip, res_dev, stream));
    if (g == nullptr || ws == nullptr) return ZERO_ERR_INVALID_ARGUMENT;
    if (reinterpret_cast<uintptr_t>(ws) % 16u != 0) return ZERO_ERR_INVALID_ARGUMENT;
    if (ws_bytes < zero_grad_check_norm_workspace_bytes(n)) return ZERO_ERR_WORKSPACE_TOO_SMALL;
    forget_ws(ws);  // a zero_step plan cached in this workspace is overwritten
    const Layout L = make_layout(n, {}, {reinterpret_cast<uintptr_t>(g)});
    const int grid = grid_for(layout_tiles(L), resident_grid_check());
    Partial* parts = static_cast<Partial*>(ws);
    hipError_t e = launch_check(g, L, parts, grid, stream);
    if (e != hipSuccess) return ZERO_ERR_HIP;
    return hip_status(launch_finalize(parts, grid, external_sumsq, max_norm, skip, res_dev, stream));
}

int zero_adamw_step(float* master, float* exp_avg, float* exp_avg_sq, const float* g, void* param_out, int64_t n,
                    const zero_adamw_hparams* hp, const zero_result* res_dev, hipStream_t stream)
{
    if (n < 0 || !hparams_ok(hp)) return ZERO_ERR_INVALID_ARGUMENT;
    if (n == 0) return ZERO_OK;
    if (!master || !exp_avg || !exp_avg_sq || !g || !param_out) return ZERO_ERR_INVALID_ARGUMENT;
    const Layout L = make_layout(n, {reinterpret_cast<uintptr_t>(param_out)},
                                 {reinterpret_cast<uintptr_t>(master), reinterpret_cast<uintptr_t>(exp_avg),
                                  reinterpret_cast<uintptr_t>(exp_avg_sq), reinterpret_cast<uintptr_t>(g)});
    const int grid = grid_for(layout_tiles(L), resident_grid_adamw());
    return hip_status(launch_adamw(master, exp_avg, exp_avg_sq, g, static_cast<uint16_t*>(param_out), L,
                                   derive(hp), res_dev, grid, stream));
}

size_t zero_step_workspace_bytes(const zero_tensor* tensors, int32_t T, int32_t M, const zero_adamw_hparams* hp)
{
    if (T < 0 || M < 1 || M > ZERO_MAX_RANKS || !hparams_ok(hp)) return 0;
    if (T > 0 && tensors == nullptr) return 0;
    for (int32_t t = 0; t < T; ++t)
        if (tensors[t].n < 0) return 0;
    return plan_offsets(sizes_of(tensors, T), M, two_pass_of(hp) ? PlanKind::StepTwoPass : PlanKind::Step).total;
}

int zero_step(const zero_tensor* tensors, int32_t T, int32_t M, const zero_adamw_hparams* hp, double external_sumsq,
              void* ws, size_t ws_bytes, zero_result* res_dev, hipStream_t stream)
{
    return step_impl(tensors, T, M, hp, external_sumsq, ws, ws_bytes, res_dev, stream, nullptr, nullptr);
}

int zero_step_noalloc(const zero_tensor* tensors, int32_t T, int32_t M, const zero_adamw_hparams* hp,
                      double external_sumsq, zero_result* res_dev, hipStream_t stream)
{
    static_assert(kScratchBytes == ZERO_NOALLOC_SCRATCH_BYTES, "the header states the scratch size");
    // arguments and size first: nothing is resolved or launched for a call
    // that is invalid or cannot fit
    int64_t total_n = 0;
    std::vector<PlanTensor> pts;
    const int arg = step_args(tensors, T, M, hp, external_sumsq, res_dev, &pts, &total_n);
    if (arg != ZERO_OK) return arg;
    const size_t need = plan_offsets(sizes_of(tensors, T), M, two_pass_of(hp) ? PlanKind::StepTwoPass : PlanKind::Step).total;
    if (need > kScratchBytes) return ZERO_ERR_SCRATCH_TOO_SMALL;
    void* ws = nullptr;
    if (scratch_workspace(&ws) != hipSuccess) return ZERO_ERR_HIP;
    return step_impl(tensors, T, M, hp, external_sumsq, ws, kScratchBytes, res_dev, stream, nullptr, nullptr);
}

int zero_loss_scale_init(const zero_loss_scale_config* cfg, zero_loss_scale* ls_dev, hipStream_t stream)
{
    if (!loss_scale_config_ok(cfg) || ls_dev == nullptr) return ZERO_ERR_INVALID_ARGUMENT;
    zero_loss_scale s;
    s.scale = static_cast<float>(std::ldexp(1.0, cfg->initial_scale_power));
    s.inv_scale = static_cast<float>(1.0 / static_cast<double>(s.scale));
    s.good_steps = 0;
    s.overflows = 0;
    return hip_status(launch_loss_scale_init(s, ls_dev, stream));
}

int zero_loss_scale_update(const zero_loss_scale_config* cfg, const zero_result* res_dev, zero_loss_scale* ls_dev,
                           hipStream_t stream)
{
    if (!loss_scale_config_ok(cfg) || res_dev == nullptr || ls_dev == nullptr) return ZERO_ERR_INVALID_ARGUMENT;
    return hip_status(launch_loss_scale_update(*cfg, res_dev, ls_dev, stream));
}

size_t zero_step_amp_workspace_bytes(const zero_tensor* tensors, int32_t T, int32_t M, const zero_adamw_hparams* hp)
{
    if (T < 0 || M < 1 || M > ZERO_MAX_RANKS || !hparams_ok(hp)) return 0;
    if (T > 0 && tensors == nullptr) return 0;
    for (int32_t t = 0; t < T; ++t)
        if (tensors[t].n < 0) return 0;
    return plan_offsets(sizes_of(tensors, T), M, PlanKind::StepTwoPass).total;
}

int zero_step_amp(const zero_tensor* tensors, int32_t T, int32_t M, const zero_adamw_hparams* hp,
                  const zero_loss_scale_config* cfg, zero_loss_scale* ls_dev, double external_sumsq, void* ws,
                  size_t ws_bytes, zero_result* res_dev, hipStream_t stream)
{
    if (!loss_scale_config_ok(cfg) || ls_dev == nullptr) return ZERO_ERR_INVALID_ARGUMENT;
    return step_impl(tensors, T, M, hp, external_sumsq, ws, ws_bytes, res_dev, stream, cfg, ls_dev);
}

// ------------------------------------------------------------------ ZeRO-2 streaming

size_t zero_bucket_reduce_workspace_bytes(const zero_grad_shard* shards, int32_t T, int32_t M)
{
    if (T < 0 || M < 1 || M > ZERO_MAX_RANKS) return 0;
    if (T > 0 && shards == nullptr) return 0;
    std::vector<int64_t> ns;
    for (int32_t t = 0; t < T; ++t) {
        if (shards[t].n < 0) return 0;
        ns.push_back(shards[t].n);
    }
    return plan_offsets(ns, M, PlanKind::Bucket).total;
}

}  // extern "C"

// The bucket reduce; ls non-null for the AMP form (the final pass squares
// acc * fl32(grad_scale) * ls->inv_scale).
static int bucket_impl(const zero_grad_shard* shards, int32_t T, int32_t M, int32_t flags, double grad_scale,
                       const zero_loss_scale* ls, uint64_t stamp, zero_bucket_partial* partial_dev, void* ws,
                       size_t ws_bytes, hipStream_t stream)
{
    if (T < 0 || M < 1 || M > ZERO_MAX_RANKS) return ZERO_ERR_INVALID_ARGUMENT;
    if ((flags & ~(ZERO_BUCKET_ACCUMULATE | ZERO_BUCKET_FINAL)) != 0) return ZERO_ERR_INVALID_ARGUMENT;
    const bool final = (flags & ZERO_BUCKET_FINAL) != 0;
    if (final && (partial_dev == nullptr || !scale_ok(grad_scale)))
        return ZERO_ERR_INVALID_ARGUMENT;
    if (T > 0 && shards == nullptr) return ZERO_ERR_INVALID_ARGUMENT;
    int64_t total_n = 0;
    std::vector<PlanTensor> pts(static_cast<size_t>(T));
    for (int32_t t = 0; t < T; ++t) {
        const zero_grad_shard& x = shards[t];
        if (x.n < 0) return ZERO_ERR_INVALID_ARGUMENT;
        pts[t].n = x.n;
        if (x.n == 0) continue;
        if (!x.grads || !x.grad_acc) return ZERO_ERR_INVALID_ARGUMENT;
        for (int32_t r = 0; r < M; ++r)
            if (x.grads[r] == nullptr) return ZERO_ERR_INVALID_ARGUMENT;
        pts[t].grads = x.grads;
        pts[t].acc = x.grad_acc;
        total_n += x.n;
    }
    const float gscale = final ? static_cast<float>(grad_scale) : 1.0f;
    if (total_n == 0)
        return final ? hip_status(launch_bucket_partial_empty(partial_dev, stamp, gscale, ls, stream)) : ZERO_OK;
    Plan plan;
    const int st = make_plan(pts, M, PlanKind::Bucket, ws, ws_bytes, stream, &plan);
    if (st != ZERO_OK) return st;
    FinalizeArgs fin{};
    fin.counter = plan.counter;
    fin.scale_from = final ? ls : nullptr;
    fin.slot = partial_dev;
    fin.stamp = stamp;
    fin.accumulate = (flags & ZERO_BUCKET_ACCUMULATE) != 0;
    fin.final = final;
    return hip_status(launch_fused(Mode::Acc, plan.geom[0], plan.hdr, plan.desc, plan.map0, plan.tiles[0], plan.sig,
                                   M, gscale, AdamScalars{}, plan.parts, fin, nullptr, stream));
}

extern "C" {

int zero_bucket_reduce(const zero_grad_shard* shards, int32_t T, int32_t M, int32_t flags, double grad_scale,
                       uint64_t stamp, zero_bucket_partial* partial_dev, void* ws, size_t ws_bytes,
                       hipStream_t stream)
{
    return bucket_impl(shards, T, M, flags, grad_scale, nullptr, stamp, partial_dev, ws, ws_bytes, stream);
}

int zero_bucket_reduce_amp(const zero_grad_shard* shards, int32_t T, int32_t M, int32_t flags, double grad_scale,
                           const zero_loss_scale* ls_dev, uint64_t stamp, zero_bucket_partial* partial_dev, void* ws,
                           size_t ws_bytes, hipStream_t stream)
{
    if (ls_dev == nullptr) return ZERO_ERR_INVALID_ARGUMENT;
    return bucket_impl(shards, T, M, flags, grad_scale, ls_dev, stamp, partial_dev, ws, ws_bytes, stream);
}

static bool acc_tensors_ok(const zero_acc_tensor* tensors, int32_t T)
{
    if (T < 0 || (T > 0 && tensors == nullptr)) return false;
    for (int32_t t = 0; t < T; ++t)
        if (tensors[t].n < 0) return false;
    return true;
}

size_t zero_step_accumulated_workspace_bytes(const zero_acc_tensor* tensors, int32_t T)
{
    if (!acc_tensors_ok(tensors, T)) return 0;
    std::vector<int64_t> ns;
    for (int32_t t = 0; t < T; ++t) ns.push_back(tensors[t].n);
    return plan_offsets(ns, 0, PlanKind::AccStep).total;
}

}  // extern "C"

// The step from accumulated gradients; lscfg/ls non-null for the AMP form:
// the multiplier reads ls->inv_scale on the device, a non-finite gradient
// always skips, and the scale moves once the update has read it.
static int acc_step_impl(const zero_acc_tensor* tensors, int32_t T, const zero_adamw_hparams* hp,
                         const zero_loss_scale_config* lscfg, zero_loss_scale* ls,
                         const zero_bucket_partial* partials_dev, int32_t nbuckets, uint64_t stamp,
                         double external_sumsq, void* ws, size_t ws_bytes, zero_result* res_dev, hipStream_t stream)
{
    if (!acc_tensors_ok(tensors, T) || !hparams_ok(hp) || res_dev == nullptr || nbuckets < 0 ||
        !external_ok(external_sumsq))
        return ZERO_ERR_INVALID_ARGUMENT;
    if (nbuckets > 0 && partials_dev == nullptr) return ZERO_ERR_INVALID_ARGUMENT;
    int64_t total_n = 0;
    std::vector<PlanTensor> pts(static_cast<size_t>(T));
    for (int32_t t = 0; t < T; ++t) {
        const zero_acc_tensor& x = tensors[t];
        pts[t].n = x.n;
        if (x.n == 0) continue;
        if (!x.grad_acc || !x.master || !x.exp_avg || !x.exp_avg_sq || !x.param_out) return ZERO_ERR_INVALID_ARGUMENT;
        pts[t] = PlanTensor{x.n, nullptr, x.master, x.exp_avg, x.exp_avg_sq, x.param_out, const_cast<float*>(x.grad_acc)};
        total_n += x.n;
    }
    const float gscale = static_cast<float>(hp->grad_scale);
    const bool amp = ls != nullptr;
    const int skip = amp || hp->skip_on_nonfinite != 0;
    hipError_t e;
    if (total_n == 0) {
        e = launch_bucket_finalize(nullptr, 0, partials_dev, nbuckets, stamp, gscale, ls, external_sumsq,
                                   hp->max_grad_norm, skip, res_dev, stream);
    } else {
        Plan plan;
        const int st = make_plan(pts, 0, PlanKind::AccStep, ws, ws_bytes, stream, &plan);
        if (st != ZERO_OK) return st;
        e = launch_bucket_finalize(plan.hdr, plan.sig, partials_dev, nbuckets, stamp, gscale, ls, external_sumsq,
                                   hp->max_grad_norm, skip, res_dev, stream);
        if (e != hipSuccess) return ZERO_ERR_HIP;
        FinalizeArgs fin{};
        fin.scale_from = ls;
        fin.stream = stream_state_stores(total_n);
        e = launch_fused(Mode::PassB, plan.geom[1], plan.hdr, plan.desc, plan.map1, plan.tiles[1], plan.sig, 0,
                         gscale, derive(hp), nullptr, fin, res_dev, stream);
    }
    if (e == hipSuccess && amp) e = launch_loss_scale_update(*lscfg, res_dev, ls, stream);
    return hip_status(e);
}

extern "C" {

int zero_step_accumulated(const zero_acc_tensor* tensors, int32_t T, const zero_adamw_hparams* hp,
                          const zero_bucket_partial* partials_dev, int32_t nbuckets, uint64_t stamp,
                          double external_sumsq, void* ws, size_t ws_bytes, zero_result* res_dev,
                          hipStream_t stream)
{
    return acc_step_impl(tensors, T, hp, nullptr, nullptr, partials_dev, nbuckets, stamp, external_sumsq, ws,
                         ws_bytes, res_dev, stream);
}

int zero_step_accumulated_amp(const zero_acc_tensor* tensors, int32_t T, const zero_adamw_hparams* hp,
                              const zero_loss_scale_config* cfg, zero_loss_scale* ls_dev,
                              const zero_bucket_partial* partials_dev, int32_t nbuckets, uint64_t stamp,
                              double external_sumsq, void* ws, size_t ws_bytes, zero_result* res_dev,
                              hipStream_t stream)
{
    if (!loss_scale_config_ok(cfg) || ls_dev == nullptr) return ZERO_ERR_INVALID_ARGUMENT;
    return acc_step_impl(tensors, T, hp, cfg, ls_dev, partials_dev, nbuckets, stamp, external_sumsq, ws, ws_bytes,
                         res_dev, stream);
}

// ------------------------------------------------------------------ ZeRO-2, fused final pass

static bool bucket_tensors_ok(const zero_bucket_tensor* ts, int32_t T, int32_t M)
{
    if (T < 0 || M < 1 || M > ZERO_MAX_RANKS || (T > 0 && ts == nullptr)) return false;
    for (int32_t t = 0; t < T; ++t)
        if (ts[t].n < 0) return false;
    return true;
}

size_t zero_bucket_step_workspace_bytes(const zero_bucket_tensor* tensors, int32_t T, int32_t M)
{
    if (!bucket_tensors_ok(tensors, T, M)) return 0;
    std::vector<int64_t> ns;
    for (int32_t t = 0; t < T; ++t) ns.push_back(tensors[t].n);
    return plan_offsets(ns, M, PlanKind::BucketStep).total;
}

int zero_bucket_step(const zero_bucket_tensor* tensors, int32_t T, int32_t M, int32_t flags,
                     const zero_adamw_hparams* hp, uint64_t stamp, zero_bucket_partial* partial_dev, void* ws,
                     size_t ws_bytes, hipStream_t stream)
{
    // the update cannot wait for the global norm: no clipping, no skipping
    if (!bucket_tensors_ok(tensors, T, M) || !hparams_ok(hp) || partial_dev == nullptr) return ZERO_ERR_INVALID_ARGUMENT;
    if (hp->max_grad_norm > 0.0 || hp->skip_on_nonfinite != 0) return ZERO_ERR_INVALID_ARGUMENT;
    if ((flags & ~(ZERO_BUCKET_ACCUMULATE | ZERO_BUCKET_STREAM_STORES)) != 0) return ZERO_ERR_INVALID_ARGUMENT;
    const bool accumulate = (flags & ZERO_BUCKET_ACCUMULATE) != 0;
    int64_t total_n = 0;
    std::vector<PlanTensor> pts(static_cast<size_t>(T));
    for (int32_t t = 0; t < T; ++t) {
        const zero_bucket_tensor& x = tensors[t];
        pts[t].n = x.n;
        if (x.n == 0) continue;
        if (!x.grads || !x.master || !x.exp_avg || !x.exp_avg_sq || !x.param_out) return ZERO_ERR_INVALID_ARGUMENT;
        if (accumulate && x.grad_acc == nullptr) return ZERO_ERR_INVALID_ARGUMENT;
        for (int32_t r = 0; r < M; ++r)
            if (x.grads[r] == nullptr) return ZERO_ERR_INVALID_ARGUMENT;
        // the accumulator is read only, and only when accumulating
        pts[t] = PlanTensor{x.n, x.grads, x.master, x.exp_avg, x.exp_avg_sq, x.param_out,
                            accumulate ? const_cast<float*>(x.grad_acc) : nullptr};
        total_n += x.n;
    }
    const float gscale = static_cast<float>(hp->grad_scale);
    if (total_n == 0) return hip_status(launch_bucket_partial_empty(partial_dev, stamp, gscale, nullptr, stream));
    Plan plan;
    const int st = make_plan(pts, M, PlanKind::BucketStep, ws, ws_bytes, stream, &plan);
    if (st != ZERO_OK) return st;
    FinalizeArgs fin{};
    fin.counter = plan.counter;
    fin.slot = partial_dev;
    fin.stamp = stamp;
    fin.accumulate = accumulate ? 1 : 0;
    fin.final = 1;
    fin.stream = (flags & ZERO_BUCKET_STREAM_STORES) != 0;
    return hip_status(launch_fused(Mode::BucketFull, plan.geom[0], plan.hdr, plan.desc, plan.map0, plan.tiles[0],
                                   plan.sig, M, gscale, derive(hp), plan.parts, fin, nullptr, stream));
}

// ------------------------------------------------------------------ CPU-offloaded step

static HostAdamScalars host_scalars(const zero_adamw_hparams* hp, double coef)
{
    const AdamScalars a = derive(hp);
    return HostAdamScalars{a.b1, a.omb1, a.b2, a.omb2, a.decay, a.lr, a.bc1, a.bc2, a.eps, coef};
}

static int team_size(int32_t threads) { return threads > 0 ? threads : host_threads_available(); }

}  // extern "C"

namespace {

// Host thread teams, one per size, kept for the life of the process (their
// threads sleep between calls). A team serves one call at a time: callers
// hold `use` while they run it.
struct TeamSlot {
    std::mutex use;
    std::unique_ptr<ThreadTeam> team;
};

TeamSlot& team_slot(int n)
{
    static std::mutex mu;
    static std::map<int, std::unique_ptr<TeamSlot>> slots;
    std::lock_guard<std::mutex> lk(mu);
    std::unique_ptr<TeamSlot>& p = slots[n];
    if (!p) {
        p.reset(new TeamSlot);
        p->team.reset(new ThreadTeam(n));
    }
    return *p;
}

}  // namespace

extern "C" {

int zero_offload_adamw_host(float* master, float* exp_avg, float* exp_avg_sq, const float* g, void* param_out,
                            int64_t n, const zero_adamw_hparams* hp, double clip_coef, int32_t threads)
{
    if (n < 0 || !hparams_ok(hp) || threads < 0 || std::isnan(clip_coef)) return ZERO_ERR_INVALID_ARGUMENT;
    if (n == 0) return ZERO_OK;
    if (!master || !exp_avg || !exp_avg_sq || !g || !param_out) return ZERO_ERR_INVALID_ARGUMENT;
    TeamSlot& slot = team_slot(team_size(threads));
    std::lock_guard<std::mutex> lk(slot.use);
    host_adamw_parallel(*slot.team, master, exp_avg, exp_avg_sq, g, static_cast<uint16_t*>(param_out), n,
                        host_scalars(hp, clip_coef));
    return ZERO_OK;
}

}  // extern "C"

namespace {

constexpr int64_t kOffloadChunk = int64_t(1) << 22;  // elements per transfer-and-update chunk
constexpr size_t kHostAlign = 64;

// The pipelined offloaded step keeps one 32-byte partial per fold chunk after
// the plan; a chunk holds at least one tile, so the tile bound bounds them.
int64_t offload_chunks_bound(const std::vector<int64_t>& ns)
{
    int64_t b = 0;
    for (int64_t n : ns) b += tiles_bound(n);
    return b;
}

size_t offload_partials_offset(const std::vector<int64_t>& ns, int32_t M)
{
    return align_up(plan_offsets(ns, M, PlanKind::Fold).total, kAlign);
}

// Host staging of an offloaded step: the record, then every tensor's fp32
// gradient, then every tensor's bf16 output (64-byte aligned regions).
struct HostLayout {
    std::vector<size_t> g, out;
    size_t total;
};

HostLayout host_layout(const zero_offload_tensor* ts, int32_t T)
{
    HostLayout h;
    size_t pos = kHostAlign;  // the 32-byte result record first
    for (int32_t t = 0; t < T; ++t) {
        h.g.push_back(pos);
        pos = align_up(pos + 4 * static_cast<size_t>(ts[t].n), kHostAlign);
    }
    for (int32_t t = 0; t < T; ++t) {
        h.out.push_back(pos);
        pos = align_up(pos + 2 * static_cast<size_t>(ts[t].n), kHostAlign);
    }
    h.total = pos;
    return h;
}

bool offload_tensors_ok(const zero_offload_tensor* ts, int32_t T, int32_t M)
{
    if (T < 0 || M < 1 || M > ZERO_MAX_RANKS || (T > 0 && ts == nullptr)) return false;
    for (int32_t t = 0; t < T; ++t)
        if (ts[t].n < 0) return false;
    return true;
}

// One copy stream per device for the host-to-device copies of the bf16
// shard, so they overlap the device-to-host copies of the gradient.
hipStream_t copy_stream()
{
    static std::mutex mu;
    static std::map<int, hipStream_t> streams;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return nullptr;
    std::lock_guard<std::mutex> lk(mu);
    auto it = streams.find(dev);
    if (it != streams.end()) return it->second;
    hipStream_t s = nullptr;
    if (hipStreamCreateWithFlags(&s, hipStreamNonBlocking) != hipSuccess) return nullptr;
    streams[dev] = s;
    return s;
}

}  // namespace

extern "C" {

size_t zero_offload_workspace_bytes(const zero_offload_tensor* tensors, int32_t T, int32_t M)
{
    if (!offload_tensors_ok(tensors, T, M)) return 0;
    std::vector<int64_t> ns;
    for (int32_t t = 0; t < T; ++t) ns.push_back(tensors[t].n);
    return offload_partials_offset(ns, M) + sizeof(zero_bucket_partial) * static_cast<size_t>(offload_chunks_bound(ns));
}

size_t zero_offload_host_workspace_bytes(const zero_offload_tensor* tensors, int32_t T)
{
    if (!offload_tensors_ok(tensors, T, 1)) return 0;
    return host_layout(tensors, T).total;
}

}  // extern "C"

// The offloaded step when the update needs nothing global (no clipping, no
// skip, a fixed scale): the fold runs group by group (tile ranges of the fold
// plan of one tile per CU, launched in the accumulate mode so that
// each group leaves a stamped partial of its sum of squares), each group's
// gradient goes down behind its fold in pieces of kOffloadChunk elements, and
// the host updates piece k while the GPU folds and copies the next ones. The
// record is combined from the group partials at the end. The host applies
// grad_scale in binary32 to the staged (unscaled) fold, the product the fold
// pass stores, so the state is the one zero_step gives; the reported sum of
// squares combines the partials in group order instead of tile order.
static int offload_pipelined(const zero_offload_tensor* tensors, int32_t T, int32_t M, const zero_adamw_hparams* hp,
                             double external_sumsq, uint8_t* wsb, size_t ws_bytes, const Plan& plan, uint8_t* hb,
                             const HostLayout& hl, zero_result* rec_d, zero_result* res_host, int32_t threads,
                             hipStream_t stream)
{
    const int64_t tile_vecs = static_cast<int64_t>(kGeoms[plan.geom[0]].nt) * kGeoms[plan.geom[0]].u;
    const int64_t tile_elems = tile_vecs * kVec;
    const int64_t per = std::max<int64_t>(static_cast<int64_t>(compute_units()), kOffloadChunk / tile_elems);
    struct Group {
        int32_t t;
        int64_t j0, j1;  // tile range within the tensor
        int64_t b, e;    // element range its fold writes
    };
    struct Piece {
        int32_t t;
        int64_t b, e;
        hipEvent_t ready;
    };
    std::vector<Group> groups;
    for (int32_t t = 0; t < T; ++t) {
        const Layout& L = plan.layouts[t];
        const int64_t nt = plan.fold_tiles[t], n = tensors[t].n;
        for (int64_t j0 = 0; j0 < nt; j0 += per) {
            const int64_t j1 = std::min(nt, j0 + per);
            int64_t b, e;
            if (L.nvec >= 0) {  // tile j: vectors [j, j+1) * tile_vecs; the head with tile 0, the tail with the last
                b = j0 == 0 ? 0 : L.head + j0 * tile_elems;
                e = j1 == nt ? n : L.head + j1 * tile_elems;
            } else {
                b = j0 * tile_elems;
                e = std::min(n, j1 * tile_elems);
            }
            groups.push_back(Group{t, j0, j1, b, e});
        }
    }
    std::vector<int64_t> ns;
    for (int32_t t = 0; t < T; ++t) ns.push_back(tensors[t].n);
    const size_t poff = offload_partials_offset(ns, M);
    if (ws_bytes < poff + sizeof(zero_bucket_partial) * groups.size()) return ZERO_ERR_WORKSPACE_TOO_SMALL;
    zero_bucket_partial* parts_d = reinterpret_cast<zero_bucket_partial*>(wsb + poff);
    zero_result* rec_h = reinterpret_cast<zero_result*>(hb);
    zero_bucket_partial* first_h = reinterpret_cast<zero_bucket_partial*>(hb + sizeof(zero_result));
    static std::atomic<uint64_t> g_stamps{1};
    const uint64_t stamp = g_stamps.fetch_add(1);
    const float gscale = static_cast<float>(hp->grad_scale);
    hipStream_t up = copy_stream();
    if (up == nullptr) return ZERO_ERR_HIP;

    // ---- every group's fold and its pieces down, then the record, all on `stream`
    int status = ZERO_OK;
    std::vector<Piece> pieces;
    for (size_t c = 0; c < groups.size() && status == ZERO_OK; ++c) {
        const Group& k = groups[c];
        const int64_t tb = plan.fold_begin[k.t] + k.j0;
        FinalizeArgs fin{};
        fin.counter = plan.counter;
        fin.slot = parts_d + c;
        fin.stamp = stamp;
        fin.accumulate = 0;
        fin.final = 1;
        if (launch_fused(Mode::Acc, plan.geom[0], plan.hdr, plan.desc, plan.map0 + tb, k.j1 - k.j0, plan.sig, M,
                         gscale, AdamScalars{}, plan.parts + tb, fin, nullptr, stream) != hipSuccess ||
            (c == 0 && hipMemcpyAsync(first_h, parts_d, sizeof(zero_bucket_partial), hipMemcpyDeviceToHost,
                                      stream) != hipSuccess)) {
            status = ZERO_ERR_HIP;
            break;
        }
        for (int64_t b = k.b; b < k.e && status == ZERO_OK; b += kOffloadChunk) {
            Piece q{k.t, b, std::min(k.e, b + kOffloadChunk), nullptr};
            if (hipEventCreateWithFlags(&q.ready, hipEventDisableTiming) != hipSuccess) {
                status = ZERO_ERR_HIP;
                break;
            }
            pieces.push_back(q);
            float* g_h = reinterpret_cast<float*>(hb + hl.g[q.t]) + q.b;
            if (hipMemcpyAsync(g_h, plan.gbuf[q.t] + q.b, 4 * static_cast<size_t>(q.e - q.b), hipMemcpyDeviceToHost,
                               stream) != hipSuccess ||
                hipEventRecord(q.ready, stream) != hipSuccess)
                status = ZERO_ERR_HIP;
        }
    }
    if (status == ZERO_OK &&
        (launch_bucket_finalize(plan.hdr, plan.sig, parts_d, static_cast<int32_t>(groups.size()), stamp, gscale,
                                nullptr, external_sumsq, hp->max_grad_norm, 0, rec_d, stream) != hipSuccess ||
         hipMemcpyAsync(rec_h, rec_d, sizeof(zero_result), hipMemcpyDeviceToHost, stream) != hipSuccess))
        status = ZERO_ERR_HIP;

    // ---- the host update piece by piece, each bf16 piece up on the copy stream
    bool stale = false;
    if (status == ZERO_OK) {
        TeamSlot& slot = team_slot(team_size(threads));
        std::lock_guard<std::mutex> lk(slot.use);
        ThreadTeam& team = *slot.team;
        HostAdamScalars sc = host_scalars(hp, 1.0);
        sc.gscale = gscale;
        for (size_t c = 0; c < pieces.size(); ++c) {
            const Piece& q = pieces[c];
            if (hipEventSynchronize(q.ready) != hipSuccess) {
                status = ZERO_ERR_HIP;
                break;
            }
            // a workspace that no longer holds the plan poisons every stamp:
            // then nothing is updated and the record says so
            if (c == 0 && first_h->stamp != stamp) {
                stale = true;
                break;
            }
            const zero_offload_tensor& x = tensors[q.t];
            const float* g_h = reinterpret_cast<const float*>(hb + hl.g[q.t]) + q.b;
            uint16_t* o_h = reinterpret_cast<uint16_t*>(hb + hl.out[q.t]) + q.b;
            host_adamw_parallel(team, x.master + q.b, x.exp_avg + q.b, x.exp_avg_sq + q.b, g_h, o_h, q.e - q.b, sc);
            if (hipMemcpyAsync(static_cast<uint16_t*>(x.param_out) + q.b, o_h, 2 * static_cast<size_t>(q.e - q.b),
                               hipMemcpyHostToDevice, up) != hipSuccess) {
                status = ZERO_ERR_HIP;
                break;
            }
        }
    }
    hipEvent_t done = nullptr;
    if (status == ZERO_OK) {
        if (hipEventCreateWithFlags(&done, hipEventDisableTiming) != hipSuccess ||
            hipEventRecord(done, up) != hipSuccess || hipStreamWaitEvent(stream, done, 0) != hipSuccess)
            status = ZERO_ERR_HIP;
    }
    // the record (and, on any early exit, every copy still in flight)
    const hipError_t sync = hipStreamSynchronize(stream);
    if (status != ZERO_OK) (void)hipStreamSynchronize(up);
    if (done != nullptr) (void)hipEventDestroy(done);
    for (const Piece& q : pieces) (void)hipEventDestroy(q.ready);
    if (status != ZERO_OK) return status;
    if (sync != hipSuccess) return ZERO_ERR_HIP;
    *res_host = *rec_h;
    if (stale && res_host->status == ZERO_OK) res_host->status = ZERO_ERR_STALE_WORKSPACE;
    return ZERO_OK;
}

// The offloaded step; lscfg/ls non-null for the AMP form: the fold reads
// ls->inv_scale, always skips on a non-finite gradient, and its last
// workgroup moves the scale (the stored gradient is already unscaled).
static int offload_impl(const zero_offload_tensor* tensors, int32_t T, int32_t M, const zero_adamw_hparams* hp,
                        const zero_loss_scale_config* lscfg, zero_loss_scale* ls, double external_sumsq, void* ws,
                        size_t ws_bytes, void* host_ws, size_t host_ws_bytes, zero_result* res_host,
                        int32_t threads, hipStream_t stream)
{
    // ---- arguments (nothing is launched on an error)
    if (!offload_tensors_ok(tensors, T, M) || !hparams_ok(hp) || res_host == nullptr || threads < 0 ||
        !external_ok(external_sumsq))
        return ZERO_ERR_INVALID_ARGUMENT;
    std::vector<PlanTensor> pts(static_cast<size_t>(T));
    int64_t total_n = 0;
    for (int32_t t = 0; t < T; ++t) {
        const zero_offload_tensor& x = tensors[t];
        pts[t].n = x.n;
        if (x.n == 0) continue;
        if (!x.grads || !x.master || !x.exp_avg || !x.exp_avg_sq || !x.param_out) return ZERO_ERR_INVALID_ARGUMENT;
        for (int32_t r = 0; r < M; ++r)
            if (x.grads[r] == nullptr) return ZERO_ERR_INVALID_ARGUMENT;
        pts[t].grads = x.grads;  // only the replicas are device memory the fold reads
        total_n += x.n;
    }
    if (ws == nullptr || reinterpret_cast<uintptr_t>(ws) % kAlign != 0) return ZERO_ERR_INVALID_ARGUMENT;
    if (host_ws == nullptr || reinterpret_cast<uintptr_t>(host_ws) % kHostAlign != 0)
        return ZERO_ERR_INVALID_ARGUMENT;
    if (total_n > 0) {  // the whole size query's answer, whichever form of the step runs
        std::vector<int64_t> ns;
        for (int32_t t = 0; t < T; ++t) ns.push_back(tensors[t].n);
        if (ws_bytes < offload_partials_offset(ns, M) + sizeof(zero_bucket_partial) *
                                                             static_cast<size_t>(offload_chunks_bound(ns)))
            return ZERO_ERR_WORKSPACE_TOO_SMALL;
    }
    const HostLayout hl = host_layout(tensors, T);
    if (host_ws_bytes < hl.total) return ZERO_ERR_WORKSPACE_TOO_SMALL;
    uint8_t* hb = static_cast<uint8_t*>(host_ws);
    zero_result* rec_h = reinterpret_cast<zero_result*>(hb);
    zero_result* rec_d = reinterpret_cast<zero_result*>(static_cast<uint8_t*>(ws) + kRecordOffset);
    const bool amp = ls != nullptr;
    const int skip = amp || hp->skip_on_nonfinite != 0;

    // ---- the fold on the GPU, then its record to the host
    if (total_n == 0) {
        if (ws_bytes < kAlign) return ZERO_ERR_WORKSPACE_TOO_SMALL;
        if (launch_finalize(nullptr, 0, external_sumsq, hp->max_grad_norm, skip, rec_d, stream) != hipSuccess)
            return ZERO_ERR_HIP;
        if (amp && launch_loss_scale_update(*lscfg, rec_d, ls, stream) != hipSuccess) return ZERO_ERR_HIP;
    } else {
        Plan plan;
        const int st = make_plan(pts, M, PlanKind::Fold, ws, ws_bytes, stream, &plan);
        if (st != ZERO_OK) return st;
        if (!amp && !(hp->max_grad_norm > 0.0) && hp->skip_on_nonfinite == 0)
            return offload_pipelined(tensors, T, M, hp, external_sumsq, static_cast<uint8_t*>(ws), ws_bytes, plan,
                                     hb, hl, rec_d, res_host, threads, stream);
        FinalizeArgs fin{};
        fin.res = rec_d;
        fin.counter = plan.counter;
        fin.external = external_sumsq;
        fin.max_norm = hp->max_grad_norm;
        fin.skip = skip;
        fin.ls = ls;
        fin.scale_from = ls;
        if (amp) fin.lscfg = *lscfg;
        if (launch_fused(Mode::PassA, plan.geom[0], plan.hdr, plan.desc, plan.map0, plan.tiles[0], plan.sig, M,
                         static_cast<float>(hp->grad_scale), AdamScalars{}, plan.parts, fin, nullptr,
                         stream) != hipSuccess)
            return ZERO_ERR_HIP;
        if (hipMemcpyAsync(rec_h, rec_d, sizeof(zero_result), hipMemcpyDeviceToHost, stream) != hipSuccess ||
            hipStreamSynchronize(stream) != hipSuccess)
            return ZERO_ERR_HIP;
        const zero_result rec = *rec_h;
        if (rec.status != ZERO_OK || rec.skipped != 0) {
            *res_host = rec;
            return ZERO_OK;
        }

        // ---- chunks: gradient down (stream), update on the host, bf16 up (copy stream)
        struct Chunk {
            int32_t t;
            int64_t b, e;
            hipEvent_t ready;
        };
        std::vector<Chunk> chunks;
        for (int32_t t = 0; t < T; ++t)
            for (int64_t b = 0; b < tensors[t].n; b += kOffloadChunk)
                chunks.push_back(Chunk{t, b, std::min(tensors[t].n, b + kOffloadChunk), nullptr});
        hipStream_t up = copy_stream();
        if (up == nullptr) return ZERO_ERR_HIP;
        int status = ZERO_OK;
        size_t made = 0;
        for (Chunk& c : chunks) {
            float* g_h = reinterpret_cast<float*>(hb + hl.g[c.t]) + c.b;
            if (hipEventCreateWithFlags(&c.ready, hipEventDisableTiming) != hipSuccess) { status = ZERO_ERR_HIP; break; }
            ++made;
            if (hipMemcpyAsync(g_h, plan.gbuf[c.t] + c.b, 4 * static_cast<size_t>(c.e - c.b), hipMemcpyDeviceToHost,
                               stream) != hipSuccess ||
                hipEventRecord(c.ready, stream) != hipSuccess) {
                status = ZERO_ERR_HIP;
                break;
            }
        }
        if (status == ZERO_OK) {
            TeamSlot& slot = team_slot(team_size(threads));
            std::lock_guard<std::mutex> lk(slot.use);
            ThreadTeam& team = *slot.team;
            const HostAdamScalars sc = host_scalars(hp, rec.clip_coef);
            for (Chunk& c : chunks) {
                if (hipEventSynchronize(c.ready) != hipSuccess) { status = ZERO_ERR_HIP; break; }
                const zero_offload_tensor& x = tensors[c.t];
                const float* g_h = reinterpret_cast<const float*>(hb + hl.g[c.t]) + c.b;
                uint16_t* o_h = reinterpret_cast<uint16_t*>(hb + hl.out[c.t]) + c.b;
                host_adamw_parallel(team, x.master + c.b, x.exp_avg + c.b, x.exp_avg_sq + c.b, g_h, o_h, c.e - c.b,
                                    sc);
                if (hipMemcpyAsync(static_cast<uint16_t*>(x.param_out) + c.b, o_h, 2 * static_cast<size_t>(c.e - c.b),
                                   hipMemcpyHostToDevice, up) != hipSuccess) {
                    status = ZERO_ERR_HIP;
                    break;
                }
            }
        }
        // the caller's stream waits for the bf16 shard; then the events go
        hipEvent_t done = nullptr;
        if (status == ZERO_OK) {
            if (hipEventCreateWithFlags(&done, hipEventDisableTiming) != hipSuccess ||
                hipEventRecord(done, up) != hipSuccess || hipStreamWaitEvent(stream, done, 0) != hipSuccess)
                status = ZERO_ERR_HIP;
        }
        if (status != ZERO_OK) {
            // no copy into or out of host_ws may outlive a failed call
            (void)hipStreamSynchronize(stream);
            (void)hipStreamSynchronize(up);
        }
        if (done != nullptr) (void)hipEventDestroy(done);
        for (size_t i = 0; i < made; ++i) (void)hipEventDestroy(chunks[i].ready);
        if (status != ZERO_OK) return status;
        *res_host = rec;
        return ZERO_OK;
    }
    if (hipMemcpyAsync(rec_h, rec_d, sizeof(zero_result), hipMemcpyDeviceToHost, stream) != hipSuccess ||
        hipStreamSynchronize(stream) != hipSuccess)
        return ZERO_ERR_HIP;
    *res_host = *rec_h;
    return ZERO_OK;
}

extern "C" {

int zero_offload_step(const zero_offload_tensor* tensors, int32_t T, int32_t M, const zero_adamw_hparams* hp,
                      double external_sumsq, void* ws, size_t ws_bytes, void* host_ws, size_t host_ws_bytes,
                      zero_result* res_host, int32_t threads, hipStream_t stream)
{
    return offload_impl(tensors, T, M, hp, nullptr, nullptr, external_sumsq, ws, ws_bytes, host_ws, host_ws_bytes,
                        res_host, threads, stream);
}

int zero_offload_step_amp(const zero_offload_tensor* tensors, int32_t T, int32_t M, const zero_adamw_hparams* hp,
                          const zero_loss_scale_config* cfg, zero_loss_scale* ls_dev, double external_sumsq, void* ws,
                          size_t ws_bytes, void* host_ws, size_t host_ws_bytes, zero_result* res_host,
                          int32_t threads, hipStream_t stream)
{
    if (!loss_scale_config_ok(cfg) || ls_dev == nullptr) return ZERO_ERR_INVALID_ARGUMENT;
    return offload_impl(tensors, T, M, hp, cfg, ls_dev, external_sumsq, ws, ws_bytes, host_ws, host_ws_bytes,
                        res_host, threads, stream);
}

int zero_workspace_forget(const void* ws)
{
    if (ws == nullptr) return ZERO_ERR_INVALID_ARGUMENT;
    forget_ws(ws);
    return ZERO_OK;
}

}  // extern "C"
