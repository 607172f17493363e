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
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <vector>

#include "../../include/adamw4.h"
#include "adamw4_internal.h"

using namespace adamw4;

namespace {

constexpr size_t kNoOffset = SIZE_MAX;

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

struct DeviceInfo {
    int cus = 0;
    int step_bpc[6] = {0, 0, 0, 0, 0, 0};   // per v rule (adamw4_mode)
    int aux_bpc = 0;
};

std::mutex g_mu;
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

// The chunk table and the tail list of a launch, built on the host.  cu = 0 picks the chunk
// size from the list's size and the grid.
adamw4_status make_tables(const std::vector<TensorDesc>& descs, uint64_t workgroups, uint32_t cu,
                          bool split_tails, std::vector<Chunk>& chunks, std::vector<uint32_t>& tails) {
    uint64_t total_units = 0;
    for (const TensorDesc& d : descs) {
        // chunk starts are 32-bit block indices (2^32 blocks = 2^39 values per tensor)
        if (plan_units(d, split_tails) > uint64_t(UINT32_MAX)) return ADAMW4_ESIZE;
        total_units += plan_units(d, split_tails);
    }
    if (cu == 0) cu = pick_chunk_units(total_units, workgroups);
    uint64_t nch = 0;
    for (const TensorDesc& d : descs) nch += (plan_units(d, split_tails) + cu - 1) / cu;
    if (nch > UINT32_MAX) return ADAMW4_ESIZE;
    chunks.clear();
    tails.clear();
    chunks.reserve(size_t(nch));
    for (size_t i = 0; i < descs.size(); ++i) {
        const uint64_t units = plan_units(descs[i], split_tails);
        for (uint64_t u = 0; u < units; u += cu)
            chunks.push_back(Chunk{uint32_t(i), uint32_t(u), uint32_t(std::min<uint64_t>(cu, units - u)), 0});
        if (split_tails && (descs[i].flags & D_QUANT) && descs[i].numel % kBlock != 0)
            tails.push_back(uint32_t(i));
    }
    balance_chunks(chunks, workgroups);
    if (chunks.size() > UINT32_MAX) return ADAMW4_ESIZE;
    return ADAMW4_OK;
}

// The last launch of each stream that read a device table: before the table is rewritten or
// freed, the host waits for these launches only (never for the whole device).
struct Uses {
    std::vector<std::pair<hipStream_t, hipEvent_t>> ev;

    adamw4_status record(hipStream_t s) {
        for (auto& e : ev)
            if (e.first == s) return hipEventRecord(e.second, s) == hipSuccess ? ADAMW4_OK : ADAMW4_EHIP;
        hipEvent_t e = nullptr;
        if (hipEventCreateWithFlags(&e, hipEventDisableTiming) != hipSuccess) return ADAMW4_EHIP;
        ev.emplace_back(s, e);
        return hipEventRecord(e, s) == hipSuccess ? ADAMW4_OK : ADAMW4_EHIP;
    }
    adamw4_status wait() const {
        for (const auto& e : ev)
            if (hipEventSynchronize(e.second) != hipSuccess) return ADAMW4_EHIP;
        return ADAMW4_OK;
    }
    void release() {
        for (auto& e : ev) (void)hipEventDestroy(e.second);
        ev.clear();
    }
};

// The launch shape of a step: chunk and tail tables in device memory.  They depend only on each
// tensor's numel and on whether it is quantized (and on the grid and chunk size), so a training
// loop builds one shape plan and keeps it however its buffers move.
struct ShapePlan {
    int device = -1;
    int workgroups = 0;
    uint32_t chunk_override = 0;
    std::vector<uint64_t> key;      // per tensor: numel << 1 | quantized
    uint32_t nchunks = 0;
    uint32_t ntails = 0;
    size_t tails_off = 0;           // byte offset of the tail list in dbuf
    void* dbuf = nullptr;
    Uses uses;
    uint64_t last_use = 0;
};

// One descriptor table in device memory with its pinned staging copy.  A step whose descriptors
// (pointers, sizes, flags, keys) equal a resident table's reuses it; otherwise the least
// recently used slot of the device is refilled by an asynchronous copy on the caller's stream.
struct DescSlot {
    int device = -1;
    void* dev = nullptr;
    void* host = nullptr;           // pinned staging
    size_t cap = 0;
    std::vector<TensorDesc> content;
    bool valid = false;
    hipEvent_t uploaded = nullptr;  // after the copy into dev
    hipStream_t upload_stream = nullptr;
    Uses uses;
    uint64_t last_use = 0;
};

constexpr int kMaxShapePlans = 8;
constexpr int kDescSlotsPerDevice = 4;
std::vector<ShapePlan*> g_shapes;
std::vector<DescSlot*> g_slots;

adamw4_status free_shape(ShapePlan* p) {
    adamw4_status s = p->uses.wait();
    p->uses.release();
    if (p->dbuf) (void)hipFree(p->dbuf);
    delete p;
    return s;
}

std::vector<uint64_t> shape_key(const std::vector<TensorDesc>& descs) {
    std::vector<uint64_t> k(descs.size());
    for (size_t i = 0; i < descs.size(); ++i)
        k[i] = (uint64_t(descs[i].numel) << 1) | ((descs[i].flags & D_QUANT) ? 1u : 0u);
    return k;
}

// Find or build the shape plan (built once per list shape: one allocation and a blocking
// upload of the tables).  Evicting the least recently used of more than kMaxShapePlans plans
// waits for that plan's own last launches.
adamw4_status get_shape(const std::vector<TensorDesc>& descs, int dev, int workgroups,
                        uint32_t chunk_override, ShapePlan*& out) {
    std::vector<uint64_t> key = shape_key(descs);
    for (ShapePlan* p : g_shapes) {
        if (p->device == dev && p->workgroups == workgroups && p->chunk_override == chunk_override &&
            p->key == key) {
            p->last_use = ++g_clock;
            out = p;
            return ADAMW4_OK;
        }
    }
    std::vector<Chunk> chunks;
    std::vector<uint32_t> tails;
    adamw4_status s = make_tables(descs, uint64_t(workgroups), chunk_override, true, chunks, tails);
    if (s != ADAMW4_OK) return s;
    if (g_shapes.size() >= size_t(kMaxShapePlans)) {
        auto lru = std::min_element(g_shapes.begin(), g_shapes.end(), [](const ShapePlan* a, const ShapePlan* b) {
            return a->last_use < b->last_use;
        });
        ShapePlan* victim = *lru;
        g_shapes.erase(lru);
        if ((s = free_shape(victim)) != ADAMW4_OK) return s;
    }
    const size_t cbytes = align16(chunks.size() * sizeof(Chunk));
    const size_t bytes = cbytes + tails.size() * sizeof(uint32_t);
    void* dbuf = nullptr;
    if (hipMalloc(&dbuf, std::max<size_t>(bytes, 16)) != hipSuccess) return ADAMW4_ENOMEM;
    std::vector<char> host(bytes);
    std::memcpy(host.data(), chunks.data(), chunks.size() * sizeof(Chunk));
    std::memcpy(host.data() + cbytes, tails.data(), tails.size() * sizeof(uint32_t));
    // a fresh buffer: a blocking copy orders it before any later use on any stream
    if (bytes && hipMemcpy(dbuf, host.data(), bytes, hipMemcpyHostToDevice) != hipSuccess) {
        (void)hipFree(dbuf);
        return ADAMW4_EHIP;
    }
    ShapePlan* p = new ShapePlan;
    p->device = dev;
    p->workgroups = workgroups;
    p->chunk_override = chunk_override;
    p->key = std::move(key);
    p->nchunks = uint32_t(chunks.size());
    p->ntails = uint32_t(tails.size());
    p->tails_off = cbytes;
    p->dbuf = dbuf;
    p->last_use = ++g_clock;
    g_shapes.push_back(p);
    out = p;
    return ADAMW4_OK;
}

// A device-resident descriptor table equal to descs, uploaded on `stream` if none is.  Only a
// list larger than the slot has held before allocates (device buffer and pinned staging, grown
// to at least twice the old size); refilling a slot waits for the launches that last read it.
adamw4_status get_descs(const std::vector<TensorDesc>& descs, int dev, hipStream_t stream,
                        DescSlot*& out) {
    const size_t bytes = descs.size() * sizeof(TensorDesc);
    DescSlot* lru = nullptr;
    int on_dev = 0;
    for (DescSlot* d : g_slots) {
        if (d->device != dev) continue;
        ++on_dev;
        if (d->valid && d->content.size() == descs.size() &&
            std::memcmp(d->content.data(), descs.data(), bytes) == 0) {
            // resident: a launch on another stream waits for the upload on the device
            if (d->upload_stream != stream && hipStreamWaitEvent(stream, d->uploaded, 0) != hipSuccess)
                return ADAMW4_EHIP;
            d->last_use = ++g_clock;
            out = d;
            return ADAMW4_OK;
        }
        if (!lru || d->last_use < lru->last_use) lru = d;
    }
    DescSlot* d = lru;
    if (on_dev < kDescSlotsPerDevice) {
        d = new DescSlot;
        d->device = dev;
        if (hipEventCreateWithFlags(&d->uploaded, hipEventDisableTiming) != hipSuccess) {
            delete d;
            return ADAMW4_EHIP;
        }
        g_slots.push_back(d);
    } else {
        // the slot's readers and its last upload (which read the staging copy) must be done
        if (d->uses.wait() != ADAMW4_OK || hipEventSynchronize(d->uploaded) != hipSuccess)
            return ADAMW4_EHIP;
    }
    d->valid = false;
    if (d->cap < bytes) {
        const size_t cap = std::max(bytes, 2 * d->cap);
        if (d->dev) (void)hipFree(d->dev);
        if (d->host) (void)hipHostFree(d->host);
        d->dev = d->host = nullptr;
        d->cap = 0;
        if (hipMalloc(&d->dev, cap) != hipSuccess) return ADAMW4_ENOMEM;
        if (hipHostMalloc(&d->host, cap, hipHostMallocDefault) != hipSuccess) {
            (void)hipFree(d->dev);
            d->dev = nullptr;
            return ADAMW4_ENOMEM;
        }
        d->cap = cap;
    }
    std::memcpy(d->host, descs.data(), bytes);
    if (hipMemcpyAsync(d->dev, d->host, bytes, hipMemcpyHostToDevice, stream) != hipSuccess ||
        hipEventRecord(d->uploaded, stream) != hipSuccess)
        return ADAMW4_EHIP;
    d->upload_stream = stream;
    d->content = descs;
    d->valid = true;
    d->last_use = ++g_clock;
    out = d;
    return ADAMW4_OK;
}

// Test hooks: the step launch's workgroup count and chunk size (128-value blocks per chunk, a
// power of two from 16 to 4096) can be forced through the environment; they change only how
// the work is cut, never a result.  0 = the library's choice.
int env_int(const char* name) {
    const char* v = std::getenv(name);
    if (!v || !*v) return 0;
    char* end = nullptr;
    const long x = std::strtol(v, &end, 10);
    return (end && *end == 0 && x > 0 && x < (1L << 20)) ? int(x) : 0;
}

uint32_t chunk_override() {
    const int c = env_int("ADAMW4_CHUNK_OVERRIDE");
    return (c >= kPlanRows && c <= 4096 && (c & (c - 1)) == 0) ? uint32_t(c) : 0u;
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

// Argument checks and descriptors shared by the two step entry points.
static adamw4_status prepare_step(const adamw4_tensor* ts, int32_t n, const adamw4_hparams* hp,
                                  int32_t max_tensors, std::vector<TensorDesc>& descs) {
    if (!hp || n < 0 || (n > 0 && !ts)) return ADAMW4_EINVAL;
    if (n > max_tensors) return ADAMW4_ESIZE;
    adamw4_status s = check_hparams(*hp);
    if (s != ADAMW4_OK) return s;
    for (int32_t i = 0; i < n; ++i)
        if ((s = check_tensor_step(ts[i])) != ADAMW4_OK) return s;
    descs.resize(static_cast<size_t>(n));
    for (int32_t i = 0; i < n; ++i) {
        descs[i] = make_desc(ts[i], uint32_t(i));
        descs[i].wcopy = ts[i].param_bf16;
    }
    return ADAMW4_OK;
}

// Workgroups for a step launch: the v rule's count per CU for the plain byte mix of 12.125 B
// per quantized value (step_blocks_per_cu), lowered when the list's quantized values move more
// bytes with the same arithmetic, which streams faster with fewer waves.  Extra bytes per
// value: 2 for FP32 grads (read), 2 for a BF16 weight copy (written), 6.94 for an FP32 m (read
// and written instead of its codes and scales).  Averaged over the list's quantized values, 1 B
// or more takes one workgroup per CU fewer and 5 B or more two fewer.  Measured, each against
// the rule's plain count: FP32 grads (the stress list) 2.1-3.1% faster one lower; BF16 copies
// (the 2.7B list) 1.3-2.4% faster one lower and slower two lower; FP32 m (the 834M study list)
// 4.4-4.6% faster for ZIP-SR and state-space SR at 3 than at 5, 2.4-3.3% for the
// round-to-nearest rules at 2 than at 4.
static int step_grid(const DeviceInfo& di, int32_t mode, const std::vector<TensorDesc>& descs) {
    uint64_t quant = 0, extra16 = 0;   // extra bytes in sixteenths
    for (const TensorDesc& d : descs) {
        if (!(d.flags & D_QUANT)) continue;
        const uint64_t n = uint64_t(d.numel);
        quant += n;
        if (!(d.flags & D_BF16)) extra16 += 32 * n;
        if (d.wcopy) extra16 += 32 * n;
        if (d.flags & D_FP32M) extra16 += 111 * n;
    }
    int bpc = di.step_bpc[mode];
    if (quant > 0 && extra16 >= 80 * quant) bpc -= 2;
    else if (quant > 0 && extra16 >= 16 * quant) bpc -= 1;
    return di.cus * std::max(bpc, 1);
}

adamw4_status adamw4_step(const adamw4_tensor* ts, int32_t n, const adamw4_hparams* hp,
                          void* stream) {
    std::vector<TensorDesc> descs;
    adamw4_status s = prepare_step(ts, n, hp, ADAMW4_MAX_TENSORS, descs);
    if (s != ADAMW4_OK || n == 0) return s;
    const StepArgs a = step_args(*hp);

    std::lock_guard<std::mutex> lock(g_mu);
    int dev = 0;
    if ((s = current_device(dev)) != ADAMW4_OK) return s;
    DeviceInfo di;
    if ((s = device_info(dev, di)) != ADAMW4_OK) return s;
    const int grid_env = env_int("ADAMW4_GRID_OVERRIDE");
    const int grid = grid_env ? grid_env : step_grid(di, hp->mode, descs);
    hipStream_t st = static_cast<hipStream_t>(stream);
    ShapePlan* sp = nullptr;
    if ((s = get_shape(descs, dev, grid, chunk_override(), sp)) != ADAMW4_OK) return s;
    DescSlot* ds = nullptr;
    if ((s = get_descs(descs, dev, st, ds)) != ADAMW4_OK) return s;
    Launch L;
    L.descs = static_cast<const TensorDesc*>(ds->dev);
    L.chunks = static_cast<const Chunk*>(sp->dbuf);
    L.nchunks = sp->nchunks;
    L.grid = int(std::min<uint64_t>(sp->nchunks, uint64_t(grid)));
    L.tails = reinterpret_cast<const uint32_t*>(static_cast<const char*>(sp->dbuf) + sp->tails_off);
    L.ntails = sp->ntails;
    L.extra = false;
    for (const TensorDesc& d : descs) L.extra = L.extra || d.wcopy != nullptr || d.base != 0;
    if (launch_step(L, a, st) != hipSuccess) return ADAMW4_EHIP;
    if ((s = sp->uses.record(st)) != ADAMW4_OK) return s;
    return ds->uses.record(st);
}

// The allocation-free step: the same launch with its tables in the fixed device array.  Layout
// of the array: descriptors | first[0..n] (prefix sums of chunks per tensor) | tail list |
// chunk table, each part 256-byte aligned.  The first three are built on the host and travel in
// kernel arguments; the chunk table is written by plan_kernel.  Chunks are taken in list order
// (no re-cut of the last rounds), starting from the size adamw4_step would pick and doubling
// until the table fits.
adamw4_status adamw4_step_noalloc(const adamw4_tensor* ts, int32_t n, const adamw4_hparams* hp,
                                  void* stream) {
    static_assert(ADAMW4_NOALLOC_SCRATCH_BYTES == kNoallocScratchBytes, "array size");
    std::vector<TensorDesc> descs;
    adamw4_status s = prepare_step(ts, n, hp, ADAMW4_NOALLOC_MAX_TENSORS, descs);
    if (s != ADAMW4_OK || n == 0) return s;
    const StepArgs a = step_args(*hp);
    const auto al = [](size_t x) { return (x + 255) & ~size_t(255); };
    std::vector<uint64_t> units(descs.size());
    uint64_t total = 0;
    for (size_t i = 0; i < descs.size(); ++i) {
        units[i] = plan_units(descs[i], true);
        if (units[i] > uint64_t(UINT32_MAX)) return ADAMW4_ESIZE;
        total += units[i];
    }
    const size_t off_first = al(descs.size() * sizeof(TensorDesc));
    const size_t off_tails = off_first + al((descs.size() + 1) * sizeof(uint32_t));
    const size_t off_chunks = off_tails + al(descs.size() * sizeof(uint32_t));

    std::lock_guard<std::mutex> lock(g_mu);
    int dev = 0;
    if ((s = current_device(dev)) != ADAMW4_OK) return s;
    DeviceInfo di;
    if ((s = device_info(dev, di)) != ADAMW4_OK) return s;
    const int grid = step_grid(di, hp->mode, descs);
    uint32_t cu = pick_chunk_units(total, uint64_t(grid));
    uint64_t nchunks = 0;
    for (;;) {
        nchunks = 0;
        for (uint64_t u : units) nchunks += (u + cu - 1) / cu;
        if (off_chunks + nchunks * sizeof(Chunk) <= kNoallocScratchBytes) break;
        if (cu >= 4096) return ADAMW4_ESIZE;
        cu *= 2;
    }
    // host image of descriptors | first | tails
    std::vector<uint32_t> image(off_chunks / 4, 0u);
    char* img = reinterpret_cast<char*>(image.data());
    std::memcpy(img, descs.data(), descs.size() * sizeof(TensorDesc));
    uint32_t* first = reinterpret_cast<uint32_t*>(img + off_first);
    uint32_t* tails = reinterpret_cast<uint32_t*>(img + off_tails);
    uint32_t acc = 0, ntails = 0;
    for (size_t i = 0; i < descs.size(); ++i) {
        first[i] = acc;
        acc += uint32_t((units[i] + cu - 1) / cu);
        if ((descs[i].flags & D_QUANT) && descs[i].numel % kBlock != 0) tails[ntails++] = uint32_t(i);
    }
    first[descs.size()] = acc;
    void* base = nullptr;
    if (noalloc_scratch(&base) != hipSuccess) return ADAMW4_EHIP;
    char* b = static_cast<char*>(base);
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (launch_upload(base, 0, image.data(), image.size(), st) != hipSuccess) return ADAMW4_EHIP;
    const TensorDesc* d_descs = reinterpret_cast<const TensorDesc*>(b);
    Chunk* d_chunks = reinterpret_cast<Chunk*>(b + off_chunks);
    if (launch_plan(d_descs, reinterpret_cast<const uint32_t*>(b + off_first), uint32_t(descs.size()),
                    cu, d_chunks, uint32_t(nchunks), st) != hipSuccess)
        return ADAMW4_EHIP;
    Launch L;
    L.descs = d_descs;
    L.chunks = d_chunks;
    L.nchunks = uint32_t(nchunks);
    L.grid = int(std::min<uint64_t>(nchunks, uint64_t(grid)));
    L.tails = reinterpret_cast<const uint32_t*>(b + off_tails);
    L.ntails = ntails;
    L.extra = false;
    for (const TensorDesc& d : descs) L.extra = L.extra || d.wcopy != nullptr || d.base != 0;
    return launch_step(L, a, st) == hipSuccess ? ADAMW4_OK : ADAMW4_EHIP;
}

// init and decode: one-off tables in a temporary buffer, freed after the stream has finished
// with them (these calls wait for their work).
static adamw4_status run_aux(std::vector<TensorDesc>&& descs, bool init, int32_t mode,
                             void* stream) {
    std::lock_guard<std::mutex> lock(g_mu);
    int dev = 0;
    adamw4_status s;
    if ((s = current_device(dev)) != ADAMW4_OK) return s;
    DeviceInfo di;
    if ((s = device_info(dev, di)) != ADAMW4_OK) return s;
    const int grid = di.cus * di.aux_bpc;
    std::vector<Chunk> chunks;
    std::vector<uint32_t> tails;
    if ((s = make_tables(descs, uint64_t(grid), 0, false, chunks, tails)) != ADAMW4_OK) return s;
    const size_t dbytes = align16(descs.size() * sizeof(TensorDesc));
    const size_t bytes = dbytes + chunks.size() * sizeof(Chunk);
    void* dbuf = nullptr;
    if (hipMalloc(&dbuf, std::max<size_t>(bytes, 16)) != hipSuccess) return ADAMW4_ENOMEM;
    std::vector<char> host(bytes);
    std::memcpy(host.data(), descs.data(), descs.size() * sizeof(TensorDesc));
    std::memcpy(host.data() + dbytes, chunks.data(), chunks.size() * sizeof(Chunk));
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e = hipMemcpy(dbuf, host.data(), bytes, hipMemcpyHostToDevice);
    if (e == hipSuccess) {
        Launch L;
        L.descs = static_cast<const TensorDesc*>(dbuf);
        L.chunks = reinterpret_cast<const Chunk*>(static_cast<const char*>(dbuf) + dbytes);
        L.nchunks = uint32_t(chunks.size());
        L.grid = int(std::min<uint64_t>(chunks.size(), uint64_t(grid)));
        L.tails = nullptr;
        L.ntails = 0;
        L.extra = false;
        e = init ? launch_init(L, mode, st) : launch_decode(L, mode, st);
    }
    const hipError_t e2 = hipStreamSynchronize(st);
    (void)hipFree(dbuf);
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
