// adamw4_api.cpp -- host runtime behind the C ABI in include/adamw4.h: argument checks,
// per-step scalars, the multi-tensor work plan (descriptor + chunk tables in device memory,
// cached across steps), and the launches.
//
// Per-step scalars follow the AdamW of the pages (bias-corrected moments inside
// h(v) = 1/(sqrt(v/(1-beta2^t)) + eps) on daiwk.github.io "ZIP-SR / ZE-EDEN: 4-bit AdamW state
// quantization", section "Core equation"; decoupled weight decay as on the kongchang.com
// explainer): bc1 = 1 - beta1^t and bc2 = 1 - beta2^t in binary64, then
// step_size = lr/bc1, rs2 = 1/sqrt(bc2), decay = 1 - lr*wd each rounded once to FP32.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cfloat>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <vector>

#include "../../include/adamw4.h"
#include "adamw4_internal.h"

using namespace adamw4;

namespace {

constexpr size_t kNoOffset = SIZE_MAX;
constexpr int kMaxPlans = 8;

size_t align16(size_t x) { return (x + 15) & ~size_t(15); }

bool quantized(int64_t n, uint32_t flags) {
    return (n >= kMinQuant || (flags & ADAMW4_T_SHARD)) && !(flags & ADAMW4_T_NORM);
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Section offsets and total size of one tensor's state.
size_t layout(int64_t n, uint32_t flags, size_t off[4]) {
    if (quantized(n, flags) && (flags & ADAMW4_T_FP32_M)) {
        const size_t m32 = align16(size_t(n) * 4);
        const size_t codes = align16(size_t((n + 1) / 2));
        const size_t scales = align16(size_t((n + kBlock - 1) / kBlock) * 4);
        off[0] = 0;
        off[1] = m32;
        off[2] = kNoOffset;
        off[3] = m32 + codes;
        return m32 + codes + scales;
    }
    if (quantized(n, flags)) {
        const size_t codes = align16(size_t((n + 1) / 2));
        const size_t scales = align16(size_t((n + kBlock - 1) / kBlock) * 4);
        off[0] = 0;
        off[1] = codes;
        off[2] = 2 * codes;
        off[3] = 2 * codes + scales;
        return 2 * codes + 2 * scales;
    }
    const size_t mv = align16(size_t(n) * 4);
    off[0] = 0;
    off[1] = mv;
    off[2] = kNoOffset;
    off[3] = kNoOffset;
    return 2 * mv;
}

adamw4_status check_tensor_common(const adamw4_tensor& t) {
    if (t.numel < 1) return ADAMW4_EINVAL;
    if (t.numel > ADAMW4_MAX_NUMEL) return ADAMW4_ESIZE;
    if (t.flags & ~uint32_t(ADAMW4_T_NORM | ADAMW4_T_HEAD | ADAMW4_T_FP32_M | ADAMW4_T_SHARD |
                            ADAMW4_T_KEYED))
        return ADAMW4_EINVAL;
    if ((t.flags & ADAMW4_T_SHARD) && (t.flags & ADAMW4_T_NORM)) return ADAMW4_EINVAL;
    if (t.offset < 0 || (t.offset % kBlock) != 0 || t.offset > ADAMW4_MAX_NUMEL - t.numel)
        return ADAMW4_EINVAL;
    if (t.reserved != 0) return ADAMW4_EINVAL;
    if (!t.state) return ADAMW4_EINVAL;
    if (!aligned16(t.state)) return ADAMW4_EALIGN;
    size_t off[4];
    if (t.state_size < layout(t.numel, t.flags, off)) return ADAMW4_ESIZE;
    return ADAMW4_OK;
}

adamw4_status check_tensor_step(const adamw4_tensor& t) {
    adamw4_status s = check_tensor_common(t);
    if (s != ADAMW4_OK) return s;
    if (!t.param || !t.grad) return ADAMW4_EINVAL;
    if (t.grad_dtype != ADAMW4_GRAD_F32 && t.grad_dtype != ADAMW4_GRAD_BF16) return ADAMW4_EINVAL;
    if (!aligned16(t.param) || !aligned16(t.grad) || !aligned16(t.param_bf16)) return ADAMW4_EALIGN;
    return ADAMW4_OK;
}

bool finite(float x) { return std::isfinite(x); }

bool valid_mode(int32_t m) { return m >= ADAMW4_ZIP_SR && m <= ADAMW4_V_ZE_RTN; }

adamw4_status check_hparams(const adamw4_hparams& h) {
    if (h.step < 1 || h.step > int64_t(UINT32_MAX)) return ADAMW4_EINVAL;
    if (!(h.beta1 >= 0.0f && h.beta1 < 1.0f)) return ADAMW4_EINVAL;
    if (!(h.beta2 >= 0.0f && h.beta2 < 1.0f)) return ADAMW4_EINVAL;
    // a normal float no larger than 2^64: with sqrt(v') < 2^64 and 1/sqrt(1-beta2^t) <= 2^12
    // the update's denominator stays inside [2^-126, 2^77], where the kernel's division is exact
    if (!(h.eps >= FLT_MIN) || !(h.eps <= 0x1p64f)) return ADAMW4_EINVAL;
    if (!finite(h.lr) || !finite(h.weight_decay)) return ADAMW4_EINVAL;
    if (!valid_mode(h.mode)) return ADAMW4_EINVAL;
    if (h.prev_mode != -1 && !valid_mode(h.prev_mode)) return ADAMW4_EINVAL;
    if (h.sr_head != 0 && h.sr_head != 1) return ADAMW4_EINVAL;
    return ADAMW4_OK;
}

StepArgs step_args(const adamw4_hparams& h) {
    const double b1 = h.beta1, b2 = h.beta2, t = double(h.step);
    const double bc1 = 1.0 - std::pow(b1, t);
    const double bc2 = 1.0 - std::pow(b2, t);
    StepArgs a;
    a.step_size = float(double(h.lr) / bc1);
    a.rs2 = float(1.0 / std::sqrt(bc2));
    a.decay = float(1.0 - double(h.lr) * double(h.weight_decay));
    a.omb1 = float(1.0 - b1);
    a.omb2 = float(1.0 - b2);
    a.beta1 = h.beta1;
    a.beta2 = h.beta2;
    a.eps = h.eps;
    a.seed_lo = uint32_t(h.seed);
    a.seed_hi = uint32_t(h.seed >> 32);
    a.t = uint32_t(h.step);
    a.mode = h.mode;
    // codebook of the incoming v: zero-excluding after ZE-EDEN, zero-inclusive after any other
    const int32_t vin = (h.prev_mode < 0) ? h.mode : h.prev_mode;
    a.vin_mode = (vin == ADAMW4_ZE_EDEN || vin == ADAMW4_V_ZE_RTN) ? 1 : 0;
    a.sr_head = h.sr_head;
    return a;
}

TensorDesc make_desc(const adamw4_tensor& t, uint32_t pos) {
    TensorDesc d;
    std::memset(&d, 0, sizeof(d));
    size_t off[4];
    layout(t.numel, t.flags, off);
    char* base = static_cast<char*>(t.state);
    d.param = t.param;
    d.grad = t.grad;
    d.numel = t.numel;
    d.pos = (t.flags & ADAMW4_T_KEYED) ? t.key : pos;
    d.base = t.offset;
    d.flags = 0;
    if (quantized(t.numel, t.flags)) d.flags |= D_QUANT;
    if (t.flags & ADAMW4_T_HEAD) d.flags |= D_HEAD;
    if (t.grad_dtype == ADAMW4_GRAD_BF16) d.flags |= D_BF16;
    if ((d.flags & D_QUANT) && (t.flags & ADAMW4_T_FP32_M)) d.flags |= D_FP32M;
    d.s0 = base + off[0];
    d.s1 = base + off[1];
    if (d.flags & D_QUANT) {
        d.s2 = (d.flags & D_FP32M) ? nullptr : reinterpret_cast<float*>(base + off[2]);
        d.s3 = reinterpret_cast<float*>(base + off[3]);
    }
    return d;
}

// Device memory for one launch's descriptors and chunk table.
struct Plan {
    int device = -1;
    int workgroups = 0;             // the launch grid the chunk table is dealt for
    std::vector<TensorDesc> descs;  // host copy, also the cache key
    uint32_t nchunks = 0;
    uint32_t ntails = 0;
    bool extra = false;             // some tensor has a BF16 copy or a shard offset
    size_t tails_off = 0;           // byte offset of the tail list in dbuf
    void* dbuf = nullptr;
    uint64_t last_use = 0;
};

struct DeviceInfo {
    int cus = 0;
    int step_bpc[6] = {0, 0, 0, 0, 0, 0};   // per v rule (adamw4_mode)
    int aux_bpc = 0;
};

std::mutex g_mu;
std::vector<Plan*> g_plans;
uint64_t g_clock = 0;
std::vector<DeviceInfo> g_dev;

adamw4_status device_info(int dev, DeviceInfo& out) {
    if (dev < 0) return ADAMW4_EHIP;
    if (size_t(dev) >= g_dev.size()) g_dev.resize(dev + 1);
    DeviceInfo& di = g_dev[dev];
    if (di.cus == 0) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return ADAMW4_EHIP;
        di.cus = std::max(cus, 1);
        for (int m = 0; m < 6; ++m) di.step_bpc[m] = step_blocks_per_cu(m);
        di.aux_bpc = aux_blocks_per_cu();
    }
    out = di;
    return ADAMW4_OK;
}


// Units (128-value blocks) a launch walks for tensor d.  Step plans (split_tails) leave the
// partial last block of a quantized tensor to the tail list.
uint64_t plan_units(const TensorDesc& d, bool split_tails) {
    if (split_tails && (d.flags & D_QUANT)) return uint64_t(d.numel / kBlock);
    return uint64_t((d.numel + kBlock - 1) / kBlock);
}



// Build descriptor, chunk and tail tables and copy them to a fresh device buffer.
adamw4_status build_plan(std::vector<TensorDesc>&& descs, int dev, int workgroups, bool split_tails,
                         Plan*& out) {
    uint64_t total_units = 0;
    for (const TensorDesc& d : descs) {
        // chunk starts are 32-bit block indices (2^32 blocks = 2^39 values per tensor)
        if (plan_units(d, split_tails) > uint64_t(UINT32_MAX)) return ADAMW4_ESIZE;
        total_units += plan_units(d, split_tails);
    }
    const uint32_t cu = pick_chunk_units(total_units, uint64_t(workgroups));
    std::vector<Chunk> chunks;
    std::vector<uint32_t> tails;
    uint64_t nch = 0;
    for (const TensorDesc& d : descs) nch += (plan_units(d, split_tails) + cu - 1) / cu;
    if (nch > UINT32_MAX) return ADAMW4_ESIZE;
    chunks.reserve(size_t(nch));
    for (size_t i = 0; i < descs.size(); ++i) {
        const uint64_t units = plan_units(descs[i], split_tails);
        for (uint64_t u = 0; u < units; u += cu)
            chunks.push_back(Chunk{uint32_t(i), uint32_t(u), uint32_t(std::min<uint64_t>(cu, units - u)), 0});
        if (split_tails && (descs[i].flags & D_QUANT) && descs[i].numel % kBlock != 0)
            tails.push_back(uint32_t(i));
    }
    balance_chunks(chunks, uint64_t(workgroups));
    if (chunks.size() > UINT32_MAX) return ADAMW4_ESIZE;
    const size_t dbytes = align16(descs.size() * sizeof(TensorDesc));
    const size_t cbytes = align16(chunks.size() * sizeof(Chunk));
    const size_t bytes = dbytes + cbytes + tails.size() * sizeof(uint32_t);
    void* dbuf = nullptr;
    if (hipMalloc(&dbuf, std::max<size_t>(bytes, 16)) != hipSuccess) return ADAMW4_ENOMEM;
    std::vector<char> host(bytes);
    std::memcpy(host.data(), descs.data(), descs.size() * sizeof(TensorDesc));
    std::memcpy(host.data() + dbytes, chunks.data(), chunks.size() * sizeof(Chunk));
    std::memcpy(host.data() + dbytes + cbytes, tails.data(), tails.size() * sizeof(uint32_t));
    // a fresh buffer: a blocking copy orders it before any later use on any stream
    if (hipMemcpy(dbuf, host.data(), bytes, hipMemcpyHostToDevice) != hipSuccess) {
        (void)hipFree(dbuf);
        return ADAMW4_EHIP;
    }
    Plan* p = new Plan;
    p->device = dev;
    p->workgroups = workgroups;
    p->descs = std::move(descs);
    p->nchunks = uint32_t(chunks.size());
    p->ntails = uint32_t(tails.size());
    for (const TensorDesc& d : p->descs) p->extra = p->extra || d.wcopy != nullptr || d.base != 0;
    p->tails_off = dbytes + cbytes;
    p->dbuf = dbuf;
    out = p;
    return ADAMW4_OK;
}

void free_plan(Plan* p) {
    if (p->dbuf) (void)hipFree(p->dbuf);
    delete p;
}

Launch launch_of(const Plan& p, int grid_cap) {
    Launch L;
    L.descs = static_cast<const TensorDesc*>(p.dbuf);
    L.chunks = reinterpret_cast<const Chunk*>(static_cast<const char*>(p.dbuf) +
                                              align16(p.descs.size() * sizeof(TensorDesc)));
    L.nchunks = p.nchunks;
    L.grid = int(std::min<uint64_t>(p.nchunks, uint64_t(std::max(grid_cap, 1))));
    L.tails = reinterpret_cast<const uint32_t*>(static_cast<const char*>(p.dbuf) + p.tails_off);
    L.ntails = p.ntails;
    L.extra = p.extra;
    return L;
}

// Find or create the cached plan for this descriptor list (the common case in training: the
// same buffers every step, so the tables are uploaded once).  Evicting a plan waits for the
// device so no in-flight launch still reads it.
adamw4_status get_plan(std::vector<TensorDesc>&& descs, int dev, int workgroups, Plan*& out) {
    for (Plan* p : g_plans) {
        if (p->device == dev && p->workgroups == workgroups && p->descs.size() == descs.size() &&
            std::memcmp(p->descs.data(), descs.data(), descs.size() * sizeof(TensorDesc)) == 0) {
            p->last_use = ++g_clock;
            out = p;
            return ADAMW4_OK;
        }
    }
    Plan* p = nullptr;
    adamw4_status s = build_plan(std::move(descs), dev, workgroups, true, p);
    if (s != ADAMW4_OK) return s;
    if (g_plans.size() >= size_t(kMaxPlans)) {
        auto lru = std::min_element(g_plans.begin(), g_plans.end(),
                                    [](const Plan* a, const Plan* b) { return a->last_use < b->last_use; });
        (void)hipDeviceSynchronize();
        free_plan(*lru);
        g_plans.erase(lru);
    }
    p->last_use = ++g_clock;
    g_plans.push_back(p);
    out = p;
    return ADAMW4_OK;
}

adamw4_status current_device(int& dev) {
    if (hipGetDevice(&dev) != hipSuccess) return ADAMW4_EHIP;
    return ADAMW4_OK;
}

}  // namespace

extern "C" {

size_t adamw4_state_bytes(int64_t numel, uint32_t flags) {
    if (numel < 1 || numel > ADAMW4_MAX_NUMEL) return 0;
    size_t off[4];
    return layout(numel, flags, off);
}

adamw4_status adamw4_state_layout(int64_t numel, uint32_t flags, size_t offsets[4]) {
    if (!offsets || numel < 1 || numel > ADAMW4_MAX_NUMEL) return ADAMW4_EINVAL;
    layout(numel, flags, offsets);
    return ADAMW4_OK;
}

adamw4_status adamw4_codebook(int32_t which, float out[16]) {
    if (!out || which < 0 || which > 2) return ADAMW4_EINVAL;
    codebook_words(which, out);
    return ADAMW4_OK;
}

adamw4_status adamw4_step(const adamw4_tensor* ts, int32_t n, const adamw4_hparams* hp,
                          void* stream) {
    if (!hp || n < 0 || (n > 0 && !ts)) return ADAMW4_EINVAL;
    if (n > ADAMW4_MAX_TENSORS) return ADAMW4_ESIZE;
    adamw4_status s = check_hparams(*hp);
    if (s != ADAMW4_OK) return s;
    for (int32_t i = 0; i < n; ++i)
        if ((s = check_tensor_step(ts[i])) != ADAMW4_OK) return s;
    if (n == 0) return ADAMW4_OK;

    std::vector<TensorDesc> descs(static_cast<size_t>(n));
    for (int32_t i = 0; i < n; ++i) {
        descs[i] = make_desc(ts[i], uint32_t(i));
        descs[i].wcopy = ts[i].param_bf16;
    }
    const StepArgs a = step_args(*hp);

    std::lock_guard<std::mutex> lock(g_mu);
    int dev = 0;
    if ((s = current_device(dev)) != ADAMW4_OK) return s;
    DeviceInfo di;
    if ((s = device_info(dev, di)) != ADAMW4_OK) return s;
    Plan* p = nullptr;
    const int grid = di.cus * di.step_bpc[hp->mode];
    if ((s = get_plan(std::move(descs), dev, grid, p)) != ADAMW4_OK) return s;
    const Launch L = launch_of(*p, grid);
    if (launch_step(L, a, static_cast<hipStream_t>(stream)) != hipSuccess) return ADAMW4_EHIP;
    return ADAMW4_OK;
}

// init and decode: a one-off plan, freed after the stream has finished with it.
static adamw4_status run_aux(std::vector<TensorDesc>&& descs, bool init, int32_t mode,
                             void* stream) {
    std::lock_guard<std::mutex> lock(g_mu);
    int dev = 0;
    adamw4_status s;
    if ((s = current_device(dev)) != ADAMW4_OK) return s;
    DeviceInfo di;
    if ((s = device_info(dev, di)) != ADAMW4_OK) return s;
    Plan* p = nullptr;
    if ((s = build_plan(std::move(descs), dev, di.cus * di.aux_bpc, false, p)) != ADAMW4_OK) return s;
    const Launch L = launch_of(*p, di.cus * di.aux_bpc);
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e = init ? launch_init(L, mode, st) : launch_decode(L, mode, st);
    hipError_t e2 = hipStreamSynchronize(st);
    free_plan(p);
    return (e == hipSuccess && e2 == hipSuccess) ? ADAMW4_OK : ADAMW4_EHIP;
}

adamw4_status adamw4_init_state(const adamw4_tensor* ts, int32_t n, int32_t mode,
                                const float* const* m0, const float* const* v0, void* stream) {
    if (n < 0 || (n > 0 && !ts)) return ADAMW4_EINVAL;
    if (n > ADAMW4_MAX_TENSORS) return ADAMW4_ESIZE;
    if (!valid_mode(mode)) return ADAMW4_EINVAL;
    adamw4_status s;
    for (int32_t i = 0; i < n; ++i) {
        if ((s = check_tensor_common(ts[i])) != ADAMW4_OK) return s;
        const float* a = m0 ? m0[i] : nullptr;
        const float* b = v0 ? v0[i] : nullptr;
        if ((a && !aligned16(a)) || (b && !aligned16(b))) return ADAMW4_EALIGN;
    }
    if (n == 0) return ADAMW4_OK;
    std::vector<TensorDesc> descs(static_cast<size_t>(n));
    for (int32_t i = 0; i < n; ++i) {
        adamw4_tensor t = ts[i];
        descs[i] = make_desc(t, uint32_t(i));
        descs[i].aux0 = const_cast<float*>(m0 ? m0[i] : nullptr);
        descs[i].aux1 = const_cast<float*>(v0 ? v0[i] : nullptr);
    }
    return run_aux(std::move(descs), true, mode, stream);
}

adamw4_status adamw4_decode_state(const adamw4_tensor* t, int32_t mode, float* m_out,
                                  float* v_out, void* stream) {
    if (!t) return ADAMW4_EINVAL;
    if (!valid_mode(mode)) return ADAMW4_EINVAL;
    adamw4_status s = check_tensor_common(*t);
    if (s != ADAMW4_OK) return s;
    if ((m_out && !aligned16(m_out)) || (v_out && !aligned16(v_out))) return ADAMW4_EALIGN;
    std::vector<TensorDesc> descs(1);
    descs[0] = make_desc(*t, 0);
    descs[0].aux0 = m_out;
    descs[0].aux1 = v_out;
    return run_aux(std::move(descs), false, mode, stream);
}

const char* adamw4_status_string(int32_t status) {
    switch (status) {
    case ADAMW4_OK: return "ok";
    case ADAMW4_EINVAL: return "invalid argument";
    case ADAMW4_EALIGN: return "device pointer not 16-byte aligned";
    case ADAMW4_ESIZE: return "size out of range or state buffer too small";
    case ADAMW4_EHIP: return "HIP runtime error";
    case ADAMW4_ENOMEM: return "out of device memory for internal tables";
    default: return "unknown status";
    }
}

}  // extern "C"
