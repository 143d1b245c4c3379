// libssd C ABI: argument validation, aliasing rules and dispatch to the HIP
// kernels.  The contract of every entry point is documented in include/ssd.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <mutex>
#include <vector>

#include "ssd.h"
#include "ssd_kernels.h"

#define SSD_EXPORT extern "C" __attribute__((visibility("default")))

namespace ssd {

hipError_t log_begin(EventLog *log, hipStream_t s)
{
    if (!log || !log->on)
        return hipSuccess;
    log->n = 0;
    return hipEventRecord(log->ev[0], s);
}

hipError_t log_kernel(EventLog *log, const char *name, hipStream_t s)
{
    if (!log || !log->on)
        return hipSuccess;
    if (log->n >= kMaxTimedKernels)
        return hipErrorInvalidValue;
    log->name[log->n] = name;
    ++log->n;
    return hipEventRecord(log->ev[log->n], s);
}

}  // namespace ssd

namespace {

constexpr int64_t kMaxHeads = 1 << 16;

bool mul_ok(int64_t a, int64_t b, int64_t *out)
{
    return !__builtin_mul_overflow(a, b, out) && *out < (int64_t(1) << 60);
}

// Basic size checks shared by every entry point.
ssd_status check_dims(const ssd_dims *d, bool uses_chunk)
{
    if (!d)
        return SSD_ERR_NULL;
    if ((d->flags & ~SSD_DT_SOFTPLUS) != 0)
        return SSD_ERR_SHAPE;
    if (d->batch < 0 || d->nheads < 1 || d->headdim < 1 || d->dstate < 1 || d->ngroups < 1)
        return SSD_ERR_SHAPE;
    if (uses_chunk && (d->seqlen < 0 || d->chunk < 1))
        return SSD_ERR_SHAPE;
    if (d->nheads % d->ngroups != 0)
        return SSD_ERR_SHAPE;
    if (d->io_dtype != SSD_F32 && d->io_dtype != SSD_BF16)
        return SSD_ERR_UNSUPPORTED;
    if (d->nheads > kMaxHeads)
        return SSD_ERR_UNSUPPORTED;
    int64_t t;
    const int64_t L = uses_chunk ? (d->seqlen > 0 ? d->seqlen : 1) : 1;
    if (!mul_ok(d->batch, L, &t) || !mul_ok(t, d->nheads, &t) || !mul_ok(t, d->headdim, &t) ||
        !mul_ok(t, 4, &t))
        return SSD_ERR_SHAPE;
    if (!mul_ok(d->batch, L, &t) || !mul_ok(t, d->ngroups, &t) || !mul_ok(t, d->dstate, &t) ||
        !mul_ok(t, 4, &t))
        return SSD_ERR_SHAPE;
    if (!mul_ok(d->batch, d->nheads, &t) || !mul_ok(t, d->headdim, &t) ||
        !mul_ok(t, d->dstate, &t) || !mul_ok(t, 4, &t))
        return SSD_ERR_SHAPE;
    if (d->batch * d->nheads > INT32_MAX)
        return SSD_ERR_UNSUPPORTED;
    return SSD_OK;
}

struct Span {
    uintptr_t lo, hi;
};
Span span(const void *p, int64_t bytes)
{
    const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    return {lo, lo + (uintptr_t)(bytes > 0 ? bytes : 0)};
}
bool overlap(Span a, Span b)
{
    return a.lo < a.hi && b.lo < b.hi && a.lo < b.hi && b.lo < a.hi;
}
bool aligned(const void *p, uintptr_t n)
{
    return reinterpret_cast<uintptr_t>(p) % n == 0;
}

ssd::DtPrep dt_prep(const ssd_dims *d)
{
    const bool sp = (d->flags & SSD_DT_SOFTPLUS) != 0;
    return ssd::DtPrep{sp ? d->dt_bias : nullptr, sp ? 1 : 0};
}

// The bias of the fused step-size prep: 4-byte aligned and outside every
// output span.
ssd_status check_dt_bias(const ssd_dims *d, const Span *outs, int nouts)
{
    const ssd::DtPrep pr = dt_prep(d);
    if (!pr.bias)
        return SSD_OK;
    if (!aligned(pr.bias, 4))
        return SSD_ERR_ALIGNMENT;
    const Span sb = span(pr.bias, d->nheads * 4);
    for (int i = 0; i < nouts; ++i)
        if (overlap(sb, outs[i]))
            return SSD_ERR_ALIAS;
    return SSD_OK;
}

ssd_status device_status(hipError_t e)
{
    return e == hipSuccess ? SSD_OK : SSD_ERR_DEVICE;
}

ssd_status scan_supported(const ssd_dims *d)
{
    if (d->io_dtype == SSD_BF16) {
        if (d->headdim != 64 || d->dstate != 128 || d->chunk % 64 != 0 || d->chunk > 512)
            return SSD_ERR_UNSUPPORTED;
    } else {
        if (d->headdim > 64 || d->dstate > 128 || d->chunk > 256)
            return SSD_ERR_UNSUPPORTED;
    }
    return SSD_OK;
}

size_t scan_workspace(const ssd_dims *d)
{
    if (d->io_dtype != SSD_BF16 || d->batch == 0 || d->seqlen == 0)
        return 0;
    return ssd::plan_scan_bf16(d->batch, d->seqlen, d->nheads, d->ngroups, d->chunk).ws_bytes;
}

// Validates a scan call and, when `launch`, enqueues it.
ssd_status run_scan(const ssd_dims *d, const void *x, const float *dt, const float *A,
                    const void *B, const void *C, const float *D, const float *init, void *y,
                    float *fin, void *ws, size_t ws_bytes, hipStream_t s, ssd::EventLog *log,
                    bool launch = true, bool check_ws = true)
{
    ssd_status st = check_dims(d, true);
    if (st != SSD_OK)
        return st;
    if ((st = scan_supported(d)) != SSD_OK)
        return st;
    if (d->batch == 0)
        return SSD_OK;
    if (!fin)
        return SSD_ERR_NULL;
    const int64_t esz = d->io_dtype == SSD_BF16 ? 2 : 4;
    const int64_t Bn = d->batch, L = d->seqlen, H = d->nheads, P = d->headdim, N = d->dstate,
                  G = d->ngroups;
    const int64_t state_bytes = Bn * H * P * N * 4;
    if (!aligned(fin, 16) || (init && !aligned(init, 16)))
        return SSD_ERR_ALIGNMENT;
    const Span sfin = span(fin, state_bytes), sinit = span(init, state_bytes);
    if (init && init != fin && overlap(sfin, sinit))
        return SSD_ERR_ALIAS;
    if (L == 0) {
        // no tokens: the cache is handed through unchanged
        if (!launch)
            return SSD_OK;
        return device_status(ssd::launch_state_init(fin, init, Bn * H * P * N, s));
    }
    if (!x || !dt || !A || !B || !C || !D || !y)
        return SSD_ERR_NULL;
    if (!aligned(x, 16) || !aligned(B, 16) || !aligned(C, 16) || !aligned(y, 16) ||
        !aligned(dt, 4) || !aligned(A, 4) || !aligned(D, 4))
        return SSD_ERR_ALIGNMENT;
    const size_t need = check_ws ? scan_workspace(d) : 0;
    if (need > 0 && (!ws || ws_bytes < need))
        return SSD_ERR_WORKSPACE;
    if (need > 0 && !aligned(ws, 16))
        return SSD_ERR_ALIGNMENT;
    const Span sy = span(y, Bn * L * H * P * esz);
    const Span sws = span(ws, (int64_t)need);
    const Span ins[] = {span(x, Bn * L * H * P * esz), span(dt, Bn * L * H * 4), span(A, H * 4),
                        span(B, Bn * L * G * N * esz), span(C, Bn * L * G * N * esz),
                        span(D, H * 4), sinit, sfin, sws};
    for (const Span &in : ins)
        if (overlap(sy, in))
            return SSD_ERR_ALIAS;
    const Span ins2[] = {span(x, Bn * L * H * P * esz), span(dt, Bn * L * H * 4),
                         span(A, H * 4), span(B, Bn * L * G * N * esz),
                         span(C, Bn * L * G * N * esz), span(D, H * 4)};
    for (const Span &in : ins2)
        if (overlap(sfin, in) || overlap(sws, in))
            return SSD_ERR_ALIAS;
    if (overlap(sws, sfin) || overlap(sws, sinit))
        return SSD_ERR_ALIAS;
    const Span outs[] = {sy, sfin, sws};
    if ((st = check_dt_bias(d, outs, 3)) != SSD_OK)
        return st;
    if (!launch)
        return SSD_OK;

    hipError_t e;
    if (d->io_dtype == SSD_BF16) {
        const ssd::Bf16Plan plan = ssd::plan_scan_bf16(Bn, L, H, G, d->chunk);
        e = ssd::launch_scan_bf16(plan, Bn, L, H, G, d->chunk, x, dt, A, B, C, D, init, y, fin,
                                  ws, dt_prep(d), s, log);
    } else {
        e = ssd::launch_scan_f32(Bn, L, H, P, N, G, d->chunk, static_cast<const float *>(x), dt,
                                 A, static_cast<const float *>(B),
                                 static_cast<const float *>(C), D, init,
                                 static_cast<float *>(y), fin, dt_prep(d), s, log);
    }
    return device_status(e);
}

// Packed variable-length batches: sequence i holds tokens cu[i] .. cu[i+1]-1
// of the [T, ...] inputs.  Consecutive sequences of equal length are laid out
// exactly like a [b, L, ...] batch, so each such run is one scan call.
ssd_status varlen_check(const ssd_dims *d, const int64_t *cu)
{
    if (!d || !cu)
        return SSD_ERR_NULL;
    if (d->batch < 0 || d->seqlen < 0)
        return SSD_ERR_SHAPE;
    if (cu[0] != 0 || cu[d->batch] != d->seqlen)
        return SSD_ERR_SHAPE;
    for (int64_t i = 0; i < d->batch; ++i)
        if (cu[i + 1] < cu[i])
            return SSD_ERR_SHAPE;
    ssd_dims one = *d;   // the packed token arrays as one sequence of T tokens
    one.batch = 1;
    ssd_status st = check_dims(&one, true);
    if (st != SSD_OK)
        return st;
    ssd_dims seqs = *d;  // the per-sequence states
    seqs.seqlen = 0;
    if ((st = check_dims(&seqs, true)) != SSD_OK)
        return st;
    return scan_supported(d);
}

// bf16 runs are scanned kMaxRuns at a time, each group in one state-kernel and
// one scan-kernel launch; a run plans for its share of the 256 CUs
// (proportional to its tokens) and gets its own workspace region.
struct RunRef {
    int64_t seq, tok, B, L;
};

std::vector<std::vector<RunRef>> bf16_groups(const ssd_dims *d, const int64_t *cu);

// Segment counts for the runs of one launch (two or more runs).  Both kernels
// run one work-group per CU, and the hardware starts work-groups in index
// order, the runs being laid out longest segments first.  Modelled time of a
// choice: the state kernel's 64-token tile-quads (the tiles of every segment
// but a run's last, times its sequences and head quads) spread over the chip,
// plus the longest-first list schedule of the scan kernel's work-groups on 256
// CUs, each as long as its segment's tiles plus about one tile per unit state
// it chains -- so that short work-groups may run in a second round on CUs
// that free up early.  Costs per tile as measured at the 2.7B layer: ~2.8 us
// per tile-quad and CU (state kernel), ~4.85 us per tile (scan kernel).  The
// candidates share a longest segment length T: each run takes the fewest
// segments of at most T chunks, for T = ceil(nchunks / k) of the longest run,
// k = 1 .. 64.
constexpr int64_t kCUsModel = 256;
constexpr double kStateTileUs = 2.8, kScanTileUs = 4.85;

int64_t run_cus(const RunRef &r, int64_t total)
{
    return std::max<int64_t>(8, (256 * r.B * r.L + total - 1) / std::max<int64_t>(total, 1));
}

// A run's segment shape for a segment count, memoised per run.
struct SegShape {
    int64_t nseg, seg_tok, last_tok, nsub;
};

struct GroupModel {
    const ssd_dims *d;
    const std::vector<RunRef> &grp;
    int64_t total;
    std::vector<std::vector<std::pair<int64_t, SegShape>>> memo;
    std::vector<std::pair<double, int64_t>> jobs, load, next, raised;   // reused buffers

    GroupModel(const ssd_dims *dd, const std::vector<RunRef> &g, int64_t t)
        : d(dd), grp(g), total(t), memo(g.size()) {}

    SegShape shape(size_t r, int64_t nseg)
    {
        for (const auto &m : memo[r])
            if (m.first == nseg)
                return m.second;
        const ssd::Bf16Plan p = ssd::plan_scan_bf16(grp[r].B, grp[r].L, d->nheads, d->ngroups,
                                                    d->chunk, run_cus(grp[r], total), nseg, false);
        const int64_t seg_tok = p.seg_tokens;
        const SegShape sh{p.nseg, seg_tok, grp[r].L - (p.nseg - 1) * seg_tok, p.nsub};
        memo[r].push_back({nseg, sh});
        return sh;
    }

    double cost(const std::vector<int64_t> &nseg)
    {
        const int64_t hg = d->nheads / d->ngroups, quads = d->ngroups * ((hg + 3) / 4);
        double state_tiles = 0.0;
        jobs.clear();   // (tiles, work-groups)
        for (size_t r = 0; r < grp.size(); ++r) {
            const SegShape sh = shape(r, nseg[r]);
            const int64_t wgs = grp[r].B * quads;
            state_tiles += (double)wgs * (double)(grp[r].L - sh.last_tok) / 64.0;
            for (int64_t sg = 0; sg < sh.nseg; ++sg) {
                const int64_t tok = sg + 1 < sh.nseg ? sh.seg_tok : sh.last_tok;
                jobs.push_back({std::max(1.0, (double)tok / 64.0) + (double)(sg * sh.nsub), wgs});
            }
        }
        std::sort(jobs.begin(), jobs.end(), [](const auto &x, const auto &y) { return x.first > y.first; });
        // CU loads as (load, CUs) buckets in ascending load; each job goes to
        // a least-loaded CU
        load.assign(1, {0.0, kCUsModel});
        for (const auto &j : jobs) {
            const int64_t full = j.second / kCUsModel;
            int64_t rem = j.second % kCUsModel;
            next.clear();
            raised.clear();
            for (auto &bk : load) {
                bk.first += (double)full * j.first;
                const int64_t take = std::min(rem, bk.second);
                rem -= take;
                if (take > 0)
                    raised.push_back({bk.first + j.first, take});
                if (bk.second > take)
                    next.push_back({bk.first, bk.second - take});
            }
            // merge the two ascending lists back into load, joining equal loads
            load.clear();
            size_t a = 0, b = 0;
            while (a < next.size() || b < raised.size()) {
                const bool from_next = b == raised.size() || (a < next.size() && next[a].first < raised[b].first);
                const std::pair<double, int64_t> bk = from_next ? next[a++] : raised[b++];
                if (!load.empty() && load.back().first == bk.first)
                    load.back().second += bk.second;
                else
                    load.push_back(bk);
            }
        }
        return kStateTileUs * state_tiles / (double)kCUsModel + kScanTileUs * load.back().first;
    }
};

std::vector<int64_t> group_nseg_search(const ssd_dims *d, const std::vector<RunRef> &grp,
                                       int64_t total)
{
    const int64_t Q = d->chunk;
    int64_t maxch = 1;
    for (const RunRef &r : grp)
        maxch = std::max(maxch, (r.L + Q - 1) / Q);
    GroupModel model(d, grp, total);
    std::vector<int64_t> best;
    double best_cost = 0.0;
    int64_t last_T = -1;
    for (int64_t k = 1; k <= std::min<int64_t>(maxch, 64); ++k) {
        const int64_t T = (maxch + k - 1) / k;           // longest segment, chunks
        if (T == last_T)
            continue;
        last_T = T;
        std::vector<int64_t> nseg(grp.size());
        for (size_t r = 0; r < grp.size(); ++r)
            nseg[r] = ((grp[r].L + Q - 1) / Q + T - 1) / T;
        const double c = model.cost(nseg);
        if (best.empty() || c < best_cost) {
            best = nseg;
            best_cost = c;
        }
    }
    return best;
}

// The search above takes ~20 us for eight runs; an entry point plans the same
// group several times (workspace query, validation, launch), and serving
// loops repeat batch shapes, so the last few answers are kept per thread.
std::vector<int64_t> group_nseg(const ssd_dims *d, const std::vector<RunRef> &grp, int64_t total)
{
    struct Entry {
        std::vector<int64_t> key, nseg;
    };
    thread_local std::vector<Entry> cache;
    std::vector<int64_t> key{d->nheads, d->ngroups, d->chunk};
    for (const RunRef &r : grp) {
        key.push_back(r.B);
        key.push_back(r.L);
    }
    for (const Entry &e : cache)
        if (e.key == key)
            return e.nseg;
    std::vector<int64_t> nseg = group_nseg_search(d, grp, total);
    if (cache.size() == 8)
        cache.erase(cache.begin());
    cache.push_back(Entry{key, nseg});
    return nseg;
}

size_t group_plans(const ssd_dims *d, const std::vector<RunRef> &grp,
                   std::vector<ssd::Bf16Plan> *plans)
{
    int64_t total = 0;
    for (const RunRef &r : grp)
        total += r.B * r.L;
    // one run: the planner of the batched scan (a packed batch of equal
    // lengths is then the batched scan, bit for bit)
    const std::vector<int64_t> nseg = grp.size() > 1 ? group_nseg(d, grp, total)
                                                     : std::vector<int64_t>(grp.size(), 0);
    size_t bytes = 0;
    for (size_t i = 0; i < grp.size(); ++i) {
        const RunRef &r = grp[i];
        const ssd::Bf16Plan p = ssd::plan_scan_bf16(r.B, r.L, d->nheads, d->ngroups, d->chunk,
                                                    run_cus(r, total), nseg[i]);
        if (plans)
            plans->push_back(p);
        bytes += (p.ws_bytes + 255) / 256 * 256;
    }
    return bytes;
}

template <class F>
ssd_status for_each_run(const ssd_dims *d, const int64_t *cu, F f)
{
    for (int64_t i = 0; i < d->batch;) {
        const int64_t len = cu[i + 1] - cu[i];
        int64_t j = i + 1;
        while (j < d->batch && cu[j + 1] - cu[j] == len)
            ++j;
        ssd_dims r = *d;
        r.batch = j - i;
        r.seqlen = len;
        const ssd_status st = f(r, i, cu[i]);
        if (st != SSD_OK)
            return st;
        i = j;
    }
    return SSD_OK;
}

std::vector<std::vector<RunRef>> bf16_groups(const ssd_dims *d, const int64_t *cu)
{
    std::vector<std::vector<RunRef>> groups(1);
    for_each_run(d, cu, [&](const ssd_dims &r, int64_t seq, int64_t tok) {
        if (r.seqlen == 0)
            return SSD_OK;
        if ((int)groups.back().size() == ssd::kMaxRuns)
            groups.emplace_back();
        groups.back().push_back(RunRef{seq, tok, r.batch, r.seqlen});
        return SSD_OK;
    });
    if (groups.back().empty())
        groups.pop_back();
    return groups;
}

}  // namespace

SSD_EXPORT const char *ssd_status_string(ssd_status status)
{
    switch (status) {
    case SSD_OK: return "SSD_OK";
    case SSD_ERR_NULL: return "SSD_ERR_NULL: a required pointer is NULL";
    case SSD_ERR_SHAPE: return "SSD_ERR_SHAPE: a size is out of range or nheads % ngroups != 0";
    case SSD_ERR_UNSUPPORTED: return "SSD_ERR_UNSUPPORTED: shape/dtype combination not implemented";
    case SSD_ERR_ALIAS: return "SSD_ERR_ALIAS: an output overlaps a buffer it must not overlap";
    case SSD_ERR_WORKSPACE: return "SSD_ERR_WORKSPACE: workspace missing or too small";
    case SSD_ERR_DEVICE: return "SSD_ERR_DEVICE: a HIP call or kernel launch failed";
    case SSD_ERR_ALIGNMENT: return "SSD_ERR_ALIGNMENT: a pointer is not aligned as required";
    }
    return "SSD_ERR_UNKNOWN";
}

SSD_EXPORT int ssd_version(void)
{
    return 10200;
}

SSD_EXPORT ssd_status ssd_state_init(const ssd_dims *dims, float *state, const float *src,
                                     void *stream)
{
    ssd_status st = check_dims(dims, false);
    if (st != SSD_OK)
        return st;
    if (dims->batch == 0)
        return SSD_OK;
    if (!state)
        return SSD_ERR_NULL;
    if (!aligned(state, 4) || (src && !aligned(src, 4)))
        return SSD_ERR_ALIGNMENT;
    const int64_t n = dims->batch * dims->nheads * dims->headdim * dims->dstate;
    if (src && src != state && overlap(span(state, n * 4), span(src, n * 4)))
        return SSD_ERR_ALIAS;
    return device_status(
        ssd::launch_state_init(state, src, n, static_cast<hipStream_t>(stream)));
}

SSD_EXPORT ssd_status ssd_chunk_scan_workspace_size(const ssd_dims *dims, size_t *bytes)
{
    ssd_status st = check_dims(dims, true);
    if (st != SSD_OK)
        return st;
    if (!bytes)
        return SSD_ERR_NULL;
    if ((st = scan_supported(dims)) != SSD_OK)
        return st;
    *bytes = scan_workspace(dims);
    return SSD_OK;
}

SSD_EXPORT ssd_status ssd_chunk_scan(const ssd_dims *dims, const void *x, const float *dt,
                                     const float *A, const void *B, const void *C,
                                     const float *D, const float *initial_state, void *y,
                                     float *final_state, void *workspace, size_t workspace_bytes,
                                     void *stream)
{
    return run_scan(dims, x, dt, A, B, C, D, initial_state, y, final_state, workspace,
                    workspace_bytes, static_cast<hipStream_t>(stream), nullptr);
}

namespace {

// Scratch memory of ssd_chunk_scan_noalloc: the scan's workspace (unit states
// and their decays) for callers that cannot allocate.  Each device the library
// runs on holds its own copy from the library's first use there until the
// process ends.  Host code never names the array except to look up its device
// address: in host code the name is a host-side stand-in, and a kernel handed
// it would fault.
constexpr size_t kScratchBytes = SSD_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void *scratch_addr[kMaxDevices];   // per device, set once (guarded by scratch_mu)

// The device address of the current device's scratch array, looked up the first
// time a call runs on that device.
ssd_status scratch_for_current_device(void **out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0)
        return SSD_ERR_DEVICE;
    if (dev >= kMaxDevices)
        return SSD_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (!scratch_addr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
            return SSD_ERR_DEVICE;
        scratch_addr[dev] = p;
    }
    *out = scratch_addr[dev];
    return SSD_OK;
}

}  // namespace

SSD_EXPORT ssd_status ssd_chunk_scan_noalloc(const ssd_dims *dims, const void *x, const float *dt,
                                             const float *A, const void *B, const void *C,
                                             const float *D, const float *initial_state, void *y,
                                             float *final_state, void *stream)
{
    ssd_status st = check_dims(dims, true);
    if (st != SSD_OK)
        return st;
    if ((st = scan_supported(dims)) != SSD_OK)
        return st;
    // the same plan as ssd_chunk_scan, so the same kernels and the same results;
    // a plan whose workspace exceeds the scratch array is refused before any
    // device call
    const size_t need = scan_workspace(dims);
    if (need > kScratchBytes)
        return SSD_ERR_WORKSPACE;
    void *ws = nullptr;
    if (need > 0 && (st = scratch_for_current_device(&ws)) != SSD_OK)
        return st;
    return run_scan(dims, x, dt, A, B, C, D, initial_state, y, final_state, ws,
                    need > 0 ? kScratchBytes : 0, static_cast<hipStream_t>(stream), nullptr);
}

SSD_EXPORT ssd_status ssd_chunk_scan_timed(const ssd_dims *dims, const void *x, const float *dt,
                                           const float *A, const void *B, const void *C,
                                           const float *D, const float *initial_state, void *y,
                                           float *final_state, void *workspace,
                                           size_t workspace_bytes, void *stream,
                                           float *kernel_ms, const char **kernel_names,
                                           int *n_kernels)
{
    if (!n_kernels || !kernel_ms)
        return SSD_ERR_NULL;
    ssd::EventLog log;
    int created = 0;
    hipError_t e = hipSuccess;
    for (; created <= ssd::kMaxTimedKernels; ++created)
        if ((e = hipEventCreate(&log.ev[created])) != hipSuccess)
            break;
    ssd_status st = SSD_OK;
    if (e != hipSuccess) {
        st = SSD_ERR_DEVICE;
    } else {
        log.on = true;
        const hipStream_t s = static_cast<hipStream_t>(stream);
        st = run_scan(dims, x, dt, A, B, C, D, initial_state, y, final_state, workspace,
                      workspace_bytes, s, &log);
        if (st == SSD_OK && hipStreamSynchronize(s) != hipSuccess)
            st = SSD_ERR_DEVICE;
        if (st == SSD_OK) {
            if (log.n > *n_kernels) {
                st = SSD_ERR_NULL;
            } else {
                for (int i = 0; i < log.n; ++i) {
                    float ms = 0.f;
                    if (hipEventElapsedTime(&ms, log.ev[i], log.ev[i + 1]) != hipSuccess)
                        st = SSD_ERR_DEVICE;
                    kernel_ms[i] = ms;
                    if (kernel_names)
                        kernel_names[i] = log.name[i];
                }
                *n_kernels = log.n;
            }
        }
    }
    for (int i = 0; i < created; ++i)
        hipEventDestroy(log.ev[i]);
    return st;
}

SSD_EXPORT ssd_status ssd_decode_step(const ssd_dims *dims, const void *x, const float *dt,
                                      const float *A, const void *B, const void *C,
                                      const float *D, float *state, void *y, void *stream)
{
    ssd_status st = check_dims(dims, false);
    if (st != SSD_OK)
        return st;
    const int64_t N = dims->dstate;
    if ((N != 16 && N != 32 && N != 64 && N != 128 && N != 256) || dims->headdim > (1 << 24))
        return SSD_ERR_UNSUPPORTED;
    if (dims->batch == 0)
        return SSD_OK;
    if (!x || !dt || !A || !B || !C || !D || !state || !y)
        return SSD_ERR_NULL;
    const int64_t esz = dims->io_dtype == SSD_BF16 ? 2 : 4;
    const int64_t Bn = dims->batch, H = dims->nheads, P = dims->headdim, G = dims->ngroups;
    if (!aligned(state, 16) || !aligned(B, 16) || !aligned(C, 16) || !aligned(x, esz) ||
        !aligned(y, esz) || !aligned(dt, 4) || !aligned(A, 4) || !aligned(D, 4))
        return SSD_ERR_ALIGNMENT;
    const Span ss = span(state, Bn * H * P * N * 4), sy = span(y, Bn * H * P * esz);
    const Span ins[] = {span(x, Bn * H * P * esz), span(dt, Bn * H * 4), span(A, H * 4),
                        span(B, Bn * G * N * esz), span(C, Bn * G * N * esz), span(D, H * 4)};
    for (const Span &in : ins)
        if (overlap(sy, in) || overlap(ss, in))
            return SSD_ERR_ALIAS;
    if (overlap(sy, ss))
        return SSD_ERR_ALIAS;
    const Span outs[] = {sy, ss};
    if ((st = check_dt_bias(dims, outs, 2)) != SSD_OK)
        return st;
    return device_status(ssd::launch_decode(dims->io_dtype == SSD_BF16, Bn, H, P, N, G, x, dt, A,
                                            B, C, D, state, y, dt_prep(dims),
                                            static_cast<hipStream_t>(stream)));
}

SSD_EXPORT ssd_status ssd_decode_steps(const ssd_dims *dims, int64_t nsteps, const void *x,
                                       const float *dt, const float *A, const void *B,
                                       const void *C, const float *D, float *state, void *y,
                                       void *stream)
{
    ssd_status st = check_dims(dims, false);
    if (st != SSD_OK)
        return st;
    if (nsteps < 0)
        return SSD_ERR_SHAPE;
    const int64_t N = dims->dstate;
    if ((N != 16 && N != 32 && N != 64 && N != 128 && N != 256) || dims->headdim > (1 << 24))
        return SSD_ERR_UNSUPPORTED;
    const int64_t Bn = dims->batch, H = dims->nheads, P = dims->headdim, G = dims->ngroups;
    // the kernel indexes steps and waves (at most one per two state rows) in 32 bits
    if (nsteps > INT32_MAX || Bn * H * ((P + 1) / 2) > INT32_MAX - 4)
        return SSD_ERR_UNSUPPORTED;
    if (Bn == 0 || nsteps == 0)
        return SSD_OK;
    if (!x || !dt || !A || !B || !C || !D || !state || !y)
        return SSD_ERR_NULL;
    const int64_t esz = dims->io_dtype == SSD_BF16 ? 2 : 4;
    int64_t xbytes, bbytes, dbytes;
    if (!mul_ok(nsteps, Bn * H * P, &xbytes) || !mul_ok(xbytes, esz, &xbytes) ||
        !mul_ok(nsteps, Bn * G * N, &bbytes) || !mul_ok(bbytes, esz, &bbytes) ||
        !mul_ok(nsteps, Bn * H, &dbytes) || !mul_ok(dbytes, 4, &dbytes))
        return SSD_ERR_SHAPE;
    if (!aligned(state, 16) || !aligned(B, 16) || !aligned(C, 16) || !aligned(x, esz) ||
        !aligned(y, esz) || !aligned(dt, 4) || !aligned(A, 4) || !aligned(D, 4))
        return SSD_ERR_ALIGNMENT;
    const Span ss = span(state, Bn * H * P * N * 4), sy = span(y, xbytes);
    const Span ins[] = {span(x, xbytes), span(dt, dbytes), span(A, H * 4), span(B, bbytes),
                        span(C, bbytes), span(D, H * 4)};
    for (const Span &in : ins)
        if (overlap(sy, in) || overlap(ss, in))
            return SSD_ERR_ALIAS;
    if (overlap(sy, ss))
        return SSD_ERR_ALIAS;
    const Span outs[] = {sy, ss};
    if ((st = check_dt_bias(dims, outs, 2)) != SSD_OK)
        return st;
    return device_status(ssd::launch_decode_steps(dims->io_dtype == SSD_BF16, nsteps, Bn, H, P,
                                                  N, G, x, dt, A, B, C, D, state, y,
                                                  dt_prep(dims), static_cast<hipStream_t>(stream)));
}

SSD_EXPORT ssd_status ssd_chunk_scan_varlen_workspace_size(const ssd_dims *dims,
                                                           const int64_t *cu_seqlens,
                                                           size_t *bytes)
{
    ssd_status st = varlen_check(dims, cu_seqlens);
    if (st != SSD_OK)
        return st;
    if (!bytes)
        return SSD_ERR_NULL;
    size_t need = 0;
    if (dims->io_dtype == SSD_BF16) {
        for (const auto &grp : bf16_groups(dims, cu_seqlens))
            need = std::max(need, group_plans(dims, grp, nullptr));
    }
    *bytes = need;
    return SSD_OK;
}

SSD_EXPORT ssd_status ssd_chunk_scan_varlen(const ssd_dims *dims, const int64_t *cu_seqlens,
                                            const void *x, const float *dt, const float *A,
                                            const void *B, const void *C, const float *D,
                                            const float *initial_states, void *y,
                                            float *final_states, void *workspace,
                                            size_t workspace_bytes, void *stream)
{
    ssd_status st = varlen_check(dims, cu_seqlens);
    if (st != SSD_OK)
        return st;
    if (dims->batch == 0)
        return SSD_OK;
    if (!final_states)
        return SSD_ERR_NULL;
    const int64_t esz = dims->io_dtype == SSD_BF16 ? 2 : 4;
    const int64_t T = dims->seqlen, H = dims->nheads, P = dims->headdim, N = dims->dstate,
                  G = dims->ngroups, HPN = H * P * N;
    // whole buffers: no output may overlap an input of another sequence either
    const Span sy = span(y, T * H * P * esz), sfin = span(final_states, dims->batch * HPN * 4);
    const Span sinit = span(initial_states, dims->batch * HPN * 4);
    const Span sws = span(workspace, (int64_t)workspace_bytes);
    const Span ins[] = {span(x, T * H * P * esz), span(dt, T * H * 4), span(A, H * 4),
                        span(B, T * G * N * esz), span(C, T * G * N * esz), span(D, H * 4)};
    for (const Span &in : ins)
        if (overlap(sy, in) || overlap(sfin, in) || overlap(sws, in))
            return SSD_ERR_ALIAS;
    if (overlap(sy, sfin) || overlap(sy, sinit) || overlap(sy, sws) || overlap(sws, sfin) ||
        overlap(sws, sinit))
        return SSD_ERR_ALIAS;
    if (initial_states && initial_states != final_states && overlap(sfin, sinit))
        return SSD_ERR_ALIAS;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const bool bf16 = dims->io_dtype == SSD_BF16;
    const char *xb = static_cast<const char *>(x), *bb = static_cast<const char *>(B),
               *cb = static_cast<const char *>(C);
    char *yb = static_cast<char *>(y);
    // fp32 runs: one scan call each (launch = true); bf16 runs: validation only
    // here (their workspace is the group's, checked below), and empty runs
    // (the state handed through) are enqueued by the same call
    auto call = [&](bool launch) {
        return for_each_run(dims, cu_seqlens, [&](const ssd_dims &r, int64_t seq, int64_t tok) {
            const bool go = launch && (!bf16 || r.seqlen == 0);
            return run_scan(&r, xb ? xb + tok * H * P * esz : nullptr, dt ? dt + tok * H : nullptr,
                            A, bb ? bb + tok * G * N * esz : nullptr,
                            cb ? cb + tok * G * N * esz : nullptr, D,
                            initial_states ? initial_states + seq * HPN : nullptr,
                            yb ? yb + tok * H * P * esz : nullptr, final_states + seq * HPN,
                            workspace, workspace_bytes, s, nullptr, go, !bf16);
        });
    };
    // every run is validated before the first is enqueued
    if ((st = call(false)) != SSD_OK)
        return st;
    std::vector<std::vector<RunRef>> groups;
    if (bf16) {
        groups = bf16_groups(dims, cu_seqlens);
        size_t need = 0;
        for (const auto &grp : groups)
            need = std::max(need, group_plans(dims, grp, nullptr));
        if (need > 0 && (!workspace || workspace_bytes < need))
            return SSD_ERR_WORKSPACE;
        if (need > 0 && !aligned(workspace, 16))
            return SSD_ERR_ALIGNMENT;
    }
    if ((st = call(true)) != SSD_OK)
        return st;
    for (const auto &grp : groups) {
        std::vector<ssd::Bf16Plan> plans;
        group_plans(dims, grp, &plans);
        // runs with the longest segments first: the hardware starts their
        // work-groups first, and short ones fill the CUs that free up
        std::vector<size_t> order(grp.size());
        for (size_t r = 0; r < order.size(); ++r)
            order[r] = r;
        std::stable_sort(order.begin(), order.end(), [&](size_t a, size_t b) {
            return plans[a].seg_tokens > plans[b].seg_tokens;
        });
        ssd::Bf16Run runs[ssd::kMaxRuns];
        char *wsp = static_cast<char *>(workspace);
        for (size_t i = 0; i < grp.size(); ++i) {
            const size_t r = order[i];
            const RunRef &u = grp[r];
            runs[i] = ssd::Bf16Run{plans[r], u.B, u.L, xb + u.tok * H * P * esz, dt + u.tok * H,
                                   bb + u.tok * G * N * esz, cb + u.tok * G * N * esz,
                                   initial_states ? initial_states + u.seq * HPN : nullptr,
                                   yb + u.tok * H * P * esz, final_states + u.seq * HPN, wsp};
            wsp += (plans[r].ws_bytes + 255) / 256 * 256;
        }
        const hipError_t e = ssd::launch_scan_bf16_multi(runs, (int)grp.size(), H, G, dims->chunk,
                                                         A, D, dt_prep(dims), s);
        if (e != hipSuccess)
            return SSD_ERR_DEVICE;
    }
    return SSD_OK;
}

namespace {

// Validation shared by the GDN entry points; S = 1 for the single step.
ssd_status gdn_check(const ssd_gdn_dims *dims, int64_t S, const void *q, const void *k,
                     const void *v, const float *g, const float *beta, float *state, void *o)
{
    if (!dims)
        return SSD_ERR_NULL;
    if (dims->reserved != 0 || dims->batch < 0 || dims->qk_heads < 1 || dims->v_heads < 1 ||
        dims->v_heads % dims->qk_heads != 0 || S < 0)
        return SSD_ERR_SHAPE;
    if (dims->io_dtype != SSD_F32 && dims->io_dtype != SSD_BF16)
        return SSD_ERR_UNSUPPORTED;
    const int64_t Bn = dims->batch, Hk = dims->qk_heads, Hv = dims->v_heads, dk = dims->dk,
                  dv = dims->dv;
    if ((dk != 64 && dk != 128 && dk != 256) || (dv != 64 && dv != 128 && dv != 256))
        return SSD_ERR_UNSUPPORTED;
    int64_t t;
    const int64_t Sx = S > 0 ? S : 1;
    if (!mul_ok(Bn, Hv, &t) || !mul_ok(t, dk, &t) || !mul_ok(t, dv, &t) || !mul_ok(t, 4, &t) ||
        !mul_ok(Sx, Bn, &t) || !mul_ok(t, Hv, &t) || !mul_ok(t, dv, &t) || !mul_ok(t, 4, &t) ||
        !mul_ok(Sx, Bn, &t) || !mul_ok(t, Hk, &t) || !mul_ok(t, dk, &t) || !mul_ok(t, 4, &t))
        return SSD_ERR_SHAPE;
    if (Bn * Hv * (dv / 64) > INT32_MAX || Hv > kMaxHeads || S > INT32_MAX)
        return SSD_ERR_UNSUPPORTED;
    if (Bn == 0 || S == 0)
        return SSD_OK;
    if (!q || !k || !v || !g || !beta || !state || !o)
        return SSD_ERR_NULL;
    const int64_t esz = dims->io_dtype == SSD_BF16 ? 2 : 4;
    if (!aligned(state, 16) || !aligned(q, esz) || !aligned(k, esz) || !aligned(v, esz) ||
        !aligned(o, esz) || !aligned(g, 4) || !aligned(beta, 4))
        return SSD_ERR_ALIGNMENT;
    const Span ss = span(state, Bn * Hv * dk * dv * 4), so = span(o, S * Bn * Hv * dv * esz);
    const Span ins[] = {span(q, S * Bn * Hk * dk * esz), span(k, S * Bn * Hk * dk * esz),
                        span(v, S * Bn * Hv * dv * esz), span(g, S * Bn * Hv * 4),
                        span(beta, S * Bn * Hv * 4)};
    for (const Span &in : ins)
        if (overlap(so, in) || overlap(ss, in))
            return SSD_ERR_ALIAS;
    if (overlap(so, ss))
        return SSD_ERR_ALIAS;
    return SSD_OK;
}

}  // namespace

SSD_EXPORT ssd_status ssd_gdn_decode_step(const ssd_gdn_dims *dims, const void *q, const void *k,
                                          const void *v, const float *g, const float *beta,
                                          float *state, void *o, void *stream)
{
    const ssd_status st = gdn_check(dims, 1, q, k, v, g, beta, state, o);
    if (st != SSD_OK || dims->batch == 0)
        return st;
    return device_status(ssd::launch_gdn_decode(dims->io_dtype == SSD_BF16, dims->batch,
                                                dims->qk_heads, dims->v_heads, dims->dk, dims->dv,
                                                q, k, v, g, beta, state, o,
                                                static_cast<hipStream_t>(stream)));
}

SSD_EXPORT ssd_status ssd_gdn_decode_steps(const ssd_gdn_dims *dims, int64_t nsteps, const void *q,
                                           const void *k, const void *v, const float *g,
                                           const float *beta, float *state, void *o, void *stream)
{
    const ssd_status st = gdn_check(dims, nsteps, q, k, v, g, beta, state, o);
    if (st != SSD_OK || dims->batch == 0 || nsteps == 0)
        return st;
    return device_status(ssd::launch_gdn_decode_steps(
        dims->io_dtype == SSD_BF16, nsteps, dims->batch, dims->qk_heads, dims->v_heads, dims->dk,
        dims->dv, q, k, v, g, beta, state, o, static_cast<hipStream_t>(stream)));
}
