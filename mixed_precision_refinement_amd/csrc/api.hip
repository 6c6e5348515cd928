// C-ABI bookkeeping: error text, workspace sizes, version and the optional
// kernel timing registry.
#include <algorithm>
#include <atomic>
#include <mutex>
#include <string>
#include <vector>

#include "common.hpp"

namespace msolve {

namespace {
thread_local std::string g_last_error;
}

void set_error(const std::string &msg) { g_last_error = msg; }

int fail(int status, const std::string &msg)
{
    set_error(msg);
    return status;
}

int hip_fail(hipError_t e, const char *what)
{
    set_error(std::string(what) + ": " + hipGetErrorString(e));
    return MSOLVE_E_HIP;
}

RefineLayout refine_layout(int64_t n, int64_t nrhs, int64_t nf)
{
    RefineLayout l;
    l.nblk = nblocks(n);
    l.npad = l.nblk * kNB;
    l.nf = nf;
    const size_t r_bytes = align256(size_t(16) * size_t(n) * size_t(nrhs));
    const size_t yd_bytes = align256(size_t(8) * size_t(l.npad) * size_t(nrhs));
    const size_t norm_bytes = align256(sizeof(uint64_t) * norm_slots(nrhs));
    l.r_stride = int64_t(r_bytes / sizeof(double));
    l.yd_stride = int64_t(yd_bytes / sizeof(float));
    l.norm_stride = int64_t(norm_bytes / sizeof(uint64_t));
    size_t off = 0;
    l.r128 = off; off += r_bytes * size_t(nf);
    l.y64 = off;  off += yd_bytes * size_t(nf);
    l.d64 = off;  off += yd_bytes * size_t(nf);
    // the ticket counters of the forward and back solves
    l.tickets = off; off += align256(sizeof(uint32_t) * 2);
    // norms, masks and per right-hand side state are contiguous, so that the
    // host reads the outcome of a batch with one copy
    l.norms = off; off += norm_bytes * size_t(nf);
    l.active = off; off += align256(sizeof(uint32_t) * size_t(3 * nf + 4));
    l.state = off; off += align256(kRhsStateBytes * size_t(nf) * size_t(nrhs));
    l.total = off;
    return l;
}

namespace {
// per-frequency bytes of a sweep batch (the complex128 matrix is not stored:
// one spare slot serves the frequencies that fall back)
size_t sweep_slot_bytes(int64_t n, int64_t nrhs)
{
    return align256(size_t(8) * size_t(n) * size_t(n)) +
           align256(sizeof(float) * msolve_dinv_floats(n)) + align256(sizeof(double) * size_t(n)) +
           refine_layout(n, nrhs, 1).total;
}
}  // namespace

int64_t sweep_batch_max(int64_t n, int64_t nrhs)
{
    // frequencies in flight together: as many as fit in 24 GiB of workspace
    const size_t budget = size_t(24) << 30;
    const size_t spare = align256(size_t(16) * size_t(n) * size_t(n));
    const int64_t b = spare < budget ? int64_t((budget - spare) / sweep_slot_bytes(n, nrhs)) : 0;
    return std::max<int64_t>(1, std::min<int64_t>(kMaxBatch, b));
}

SweepLayout sweep_layout(int64_t n, int64_t nrhs, int64_t nf, int64_t sets)
{
    SweepLayout l;
    l.nf = nf;
    l.sets = sets;
    const size_t z128 = align256(size_t(16) * size_t(n) * size_t(n));
    const size_t z64 = align256(size_t(8) * size_t(n) * size_t(n));
    const size_t dinv = align256(sizeof(float) * msolve_dinv_floats(n));
    const size_t zrow = align256(sizeof(double) * size_t(n));
    l.z128_stride = int64_t(z128 / sizeof(double));
    l.z64_stride = int64_t(z64 / sizeof(float));
    l.dinv_stride = int64_t(dinv / sizeof(float));
    l.zrow_stride = int64_t(zrow / sizeof(double));
    size_t off = 0;
    l.z128 = off; off += z128;   // one spare slot
    const size_t set0 = off;
    l.z64 = off;  off += z64 * size_t(nf);
    l.dinv = off; off += dinv * size_t(nf);
    l.zrow = off; off += zrow * size_t(nf);
    l.info = off; off += align256(sizeof(int32_t) * size_t(nf));
    l.fflags = off; off += align256(msolve_factor_batch_workspace_bytes(n, nf));
    l.set_bytes = off - set0;
    off += l.set_bytes * size_t(sets - 1);
    l.gepp_aux = off; off += align256(gepp_aux_bytes(n));
    l.refine = off; off += refine_layout(n, nrhs, nf).total;
    l.total = off;
    return l;
}

// ---------------------------------------------------------------- timing

namespace {
struct ProfRecord {
    int kernel;
    hipEvent_t e0, e1;
    double work;
    int64_t tag;
};
thread_local int64_t g_prof_tag = 0;
struct ProfState {
    std::mutex mu;
    bool on = false;
    std::vector<ProfRecord> recs;
    std::vector<hipEvent_t> pool;
};
ProfState &prof_state()
{
    static ProfState st;
    return st;
}
hipEvent_t take_event(ProfState &st)
{
    if (!st.pool.empty()) {
        hipEvent_t e = st.pool.back();
        st.pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}
}  // namespace

ProfScope::ProfScope(int k, hipStream_t s, double w) : kernel(k), stream(s), work(w), ev0(nullptr)
{
    ProfState &st = prof_state();
    if (!st.on) return;
    std::lock_guard<std::mutex> g(st.mu);
    hipEvent_t e = take_event(st);
    if (e && hipEventRecord(e, s) == hipSuccess) ev0 = e;
}

ProfScope::~ProfScope()
{
    if (!ev0) return;
    ProfState &st = prof_state();
    std::lock_guard<std::mutex> g(st.mu);
    hipEvent_t e1 = take_event(st);
    if (!e1 || hipEventRecord(e1, stream) != hipSuccess) return;
    st.recs.push_back(ProfRecord{kernel, static_cast<hipEvent_t>(ev0), e1, work, g_prof_tag});
}

int64_t prof_new_tag()
{
    static std::atomic<int64_t> next{1};
    return next.fetch_add(1);
}

void prof_set_tag(int64_t tag) { g_prof_tag = tag; }

void prof_scale_tag(int64_t tag, double factor)
{
    if (tag == 0) return;
    ProfState &st = prof_state();
    std::lock_guard<std::mutex> g(st.mu);
    for (auto &r : st.recs)
        if (r.tag == tag) r.work *= factor;
}

}  // namespace msolve

using namespace msolve;

extern "C" int32_t msolve_version(void) { return 100; }

extern "C" const char *msolve_last_error(void) { return g_last_error.c_str(); }

extern "C" int64_t msolve_block_size(int64_t n)
{
    (void)n;
    return kNB;
}

extern "C" size_t msolve_dinv_floats(int64_t n)
{
    if (n < 1) return 0;
    // per block: the inverses of its unit-lower and upper parts; per pair of
    // blocks (2t, 2t+1): the coupling blocks of the pair's inverses
    const size_t nblk = size_t(nblocks(n)), npair = nblk / 2;
    return (nblk + npair) * 2 * 2 * size_t(kNB) * size_t(kNB);
}

extern "C" size_t msolve_factor_workspace_bytes(int64_t n)
{
    return msolve_factor_batch_workspace_bytes(n, 1);
}

extern "C" size_t msolve_factor_batch_workspace_bytes(int64_t n, int64_t nf)
{
    // one hand-off word per matrix for the general diagonal steps
    (void)n;
    return align256(sizeof(uint32_t) * size_t(nf < 1 ? 1 : nf));
}

extern "C" size_t msolve_refine_workspace_bytes(int64_t n, int64_t nrhs)
{
    if (n < 1 || nrhs < 1) return 0;
    return refine_layout(n, nrhs).total;
}

extern "C" int64_t msolve_sweep_batch(int64_t n, int64_t nrhs, int64_t nfreq)
{
    if (n < 1 || nrhs < 1 || nfreq < 1) return 0;
    // equal batches: ceil(nfreq / bmax) of them
    const int64_t bmax = sweep_batch_max(n, nrhs);
    const int64_t batches = (nfreq + bmax - 1) / bmax;
    return (nfreq + batches - 1) / batches;
}

extern "C" size_t msolve_sweep_workspace_bytes(int64_t n, int64_t nrhs, int64_t nfreq)
{
    if (n < 1 || nrhs < 1 || nfreq < 1) return 0;
    const int64_t nb = msolve_sweep_batch(n, nrhs, nfreq);
    return sweep_layout(n, nrhs, nb, nfreq > nb ? 2 : 1).total;
}

extern "C" size_t msolve_workspace_bytes(int64_t n, int64_t nrhs, int64_t nfreq)
{
    size_t a = msolve_factor_workspace_bytes(n);
    size_t b = msolve_refine_workspace_bytes(n, nrhs);
    size_t c = msolve_sweep_workspace_bytes(n, nrhs, nfreq < 1 ? 1 : nfreq);
    return a > b ? (a > c ? a : c) : (b > c ? b : c);
}

extern "C" int msolve_profile_enable(int32_t on)
{
    ProfState &st = prof_state();
    std::lock_guard<std::mutex> g(st.mu);
    st.on = on != 0;
    return MSOLVE_OK;
}

extern "C" int msolve_profile_reset(void)
{
    ProfState &st = prof_state();
    std::lock_guard<std::mutex> g(st.mu);
    for (auto &r : st.recs) {
        (void)hipEventSynchronize(r.e1);
        st.pool.push_back(r.e0);
        st.pool.push_back(r.e1);
    }
    st.recs.clear();
    return MSOLVE_OK;
}

extern "C" int msolve_profile_query(int32_t kernel, int64_t *launches, double *total_ms,
                                    double *flops_or_bytes)
{
    if (kernel < 0 || kernel >= MSOLVE_K_COUNT)
        return fail(MSOLVE_E_ARG, "msolve_profile_query: unknown kernel id");
    ProfState &st = prof_state();
    std::lock_guard<std::mutex> g(st.mu);
    int64_t cnt = 0;
    double ms = 0.0, work = 0.0;
    for (auto &r : st.recs) {
        if (r.kernel != kernel) continue;
        MS_HIP(hipEventSynchronize(r.e1));
        float t = 0.0f;
        MS_HIP(hipEventElapsedTime(&t, r.e0, r.e1));
        ++cnt;
        ms += double(t);
        work += r.work;
    }
    if (launches) *launches = cnt;
    if (total_ms) *total_ms = ms;
    if (flops_or_bytes) *flops_or_bytes = work;
    return MSOLVE_OK;
}
