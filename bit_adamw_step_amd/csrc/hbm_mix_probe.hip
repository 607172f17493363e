// hbm_mix_probe.hip -- measurement program, not part of the optimizer: how fast this GPU moves the
// 4-bit AdamW step's byte mix (per 128 values: FP32 weights read and written, BF16 gradients
// read, two 4-bit code arrays read and written, two FP32 block scales read and written; 12.125 B
// per value) with trivial arithmetic, over the 2.7B list's 2,701,393,920 quantized values.  It
// sweeps what a streaming kernel can choose: the lane map, the store and load cache policy, the
// workgroups per CU, the chunk size, batching two or four iterations' loads before their stores,
// software pipelining (the next iteration's loads issued before the current one's stores), and a
// synthetic VALU load of 40 or 75 FMAs per value; plus read-only, write-only, copy and
// weights-plus-gradients ("triad") streams.  Each variant runs twice untimed and `reps` times
// timed with HIP events; one CSV line per variant: name, mean ms, algorithmic GB/s, bytes.
//
//   hbm_mix_probe [FILTER [REPS]]   FILTER: comma-separated variant names, or a substring
//
// Variant names: KIND_MAP_STORE_LOAD[_bBATCH]/gWORKGROUPS_PER_CU/cCHUNK_BLOCKS, with KIND mix,
// read, write, pipe (software-pipelined mix), triad, mixcN / pipecN (N FMAs per value); MAP row
// (a 16-lane row per 128-value block, lane r holding values 4r..4r+3 and 64+4r..64+4r+3, as the
// step) or wave (each wave instruction covers 1 KiB contiguous); STORE ntS (non-temporal), S0
// (default), sc1, sc01 (sc0 sc1), ntsc1; LOAD ntL (non-temporal) or L0 (default).
//
// Every access stays inside its buffer: the chunk size divides the block count exactly (checked
// before each launch) and each workgroup iteration covers 16 whole blocks.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
#include <vector>
#include <string>

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
#define G1 __attribute__((address_space(1)))

enum { K_MIX = 0, K_READ = 1, K_WRITE = 2, K_PIPE = 3, K_TRIAD = 4 };

template <class T> __device__ inline T* up(T* p) {
    const uint64_t a = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    return reinterpret_cast<T*>(((uint64_t)hi << 32) | lo);
}

template <int LPOL, class T> __device__ inline T ld(const char* base, uint32_t off) {
    const G1 T* p = (const G1 T*)(base + off);
    if (LPOL == 1) return __builtin_nontemporal_load(p);
    return *p;
}

// store with policy: 0 plain, 1 nt, 2 sc1, 3 sc0 sc1, 4 nt sc1.  The policy bits have no
// builtin, so those forms are written as asm; the s_nop after a 16-byte store keeps a following
// VALU write from reaching the store's data registers before the store has read them.
template <int SPOL> __device__ inline void st4(char* base, uint32_t off, f32x4 v) {
    G1 f32x4* p = (G1 f32x4*)(base + off);
    if (SPOL == 0) *p = v;
    else if (SPOL == 1) __builtin_nontemporal_store(v, p);
    else if (SPOL == 2) asm volatile("global_store_dwordx4 %0, %1, off sc1\n s_nop 1" :: "v"(p), "v"(v) : "memory");
    else if (SPOL == 3) asm volatile("global_store_dwordx4 %0, %1, off sc0 sc1\n s_nop 1" :: "v"(p), "v"(v) : "memory");
    else asm volatile("global_store_dwordx4 %0, %1, off sc1 nt\n s_nop 1" :: "v"(p), "v"(v) : "memory");
}
template <int SPOL> __device__ inline void st1(char* base, uint32_t off, uint32_t v) {
    G1 uint32_t* p = (G1 uint32_t*)(base + off);
    if (SPOL == 0) *p = v;
    else if (SPOL == 1) __builtin_nontemporal_store(v, p);
    else if (SPOL == 2) asm volatile("global_store_dword %0, %1, off sc1" :: "v"(p), "v"(v) : "memory");
    else if (SPOL == 3) asm volatile("global_store_dword %0, %1, off sc0 sc1" :: "v"(p), "v"(v) : "memory");
    else asm volatile("global_store_dword %0, %1, off sc1 nt" :: "v"(p), "v"(v) : "memory");
}

struct Offs { uint32_t wA, wB, gA, gB, cd; int sidx; };

template <int MAP> __device__ inline Offs offs() {
    Offs o;
    const int t = threadIdx.x;
    if (MAP == 0) {
        const int row = t >> 4, rl = t & 15;
        o.wA = row * 512 + rl * 16; o.wB = o.wA + 256;
        o.gA = row * 256 + rl * 8; o.gB = o.gA + 128;
        o.cd = row * 64 + (rl >> 1) * 4 + (rl & 1) * 32;
        o.sidx = rl == 0 ? row : -1;
    } else {
        const int wv = t >> 6, l = t & 63;
        o.wA = wv * 2048 + l * 16; o.wB = o.wA + 1024;
        o.gA = wv * 1024 + l * 8; o.gB = o.gA + 512;
        o.cd = wv * 256 + l * 4;
        o.sidx = l < 4 ? 4 * wv + l : -1;
    }
    return o;
}

struct Data { f32x4 a, b; u32x2 g0, g1; uint32_t m, v; float s0, s1; };

template <int LPOL> __device__ inline void load_grp(Data& d, const Offs& o, char* wb, const char* gb,
                                                    const char* mb, const char* vb, const float* smb,
                                                    const float* svb) {
    d.m = ld<LPOL, uint32_t>(mb, o.cd);
    d.v = ld<LPOL, uint32_t>(vb, o.cd);
    d.s0 = d.s1 = 0.0f;
    if (o.sidx >= 0) { d.s0 = *(const G1 float*)(smb + o.sidx); d.s1 = *(const G1 float*)(svb + o.sidx); }
    d.g0 = ld<LPOL, u32x2>(gb, o.gA);
    d.g1 = ld<LPOL, u32x2>(gb, o.gB);
    d.a = ld<LPOL, f32x4>(wb, o.wA);
    d.b = ld<LPOL, f32x4>(wb, o.wB);
}

template <int NOPS> __device__ inline void burn(Data& d) {
    float x[8] = {d.a.x, d.a.y, d.a.z, d.a.w, d.b.x, d.b.y, d.b.z, d.b.w};
#pragma unroll
    for (int k = 0; k < NOPS; ++k)
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] = __builtin_fmaf(x[j], 0.99999f, 1e-30f);
    d.a = f32x4{x[0], x[1], x[2], x[3]}; d.b = f32x4{x[4], x[5], x[6], x[7]};
}

__device__ inline void compute(Data& d) {
    d.a.x -= __uint_as_float(d.g0.x << 16); d.a.y -= __uint_as_float(d.g0.x & 0xFFFF0000u);
    d.a.z -= __uint_as_float(d.g0.y << 16); d.a.w -= __uint_as_float(d.g0.y & 0xFFFF0000u);
    d.b.x -= __uint_as_float(d.g1.x << 16); d.b.y -= __uint_as_float(d.g1.x & 0xFFFF0000u);
    d.b.z -= __uint_as_float(d.g1.y << 16); d.b.w -= __uint_as_float(d.g1.y & 0xFFFF0000u);
    d.m ^= 0x11111111u; d.v ^= 0x22222222u; d.s0 *= 0.5f; d.s1 *= 0.5f;
}

template <int SPOL> __device__ inline void store_grp(const Data& d, const Offs& o, char* wb, char* mb,
                                                     char* vb, float* smb, float* svb) {
    st4<SPOL>(wb, o.wA, d.a);
    st4<SPOL>(wb, o.wB, d.b);
    st1<SPOL>(mb, o.cd, d.m);
    st1<SPOL>(vb, o.cd, d.v);
    if (o.sidx >= 0) { *(G1 float*)(smb + o.sidx) = d.s0; *(G1 float*)(svb + o.sidx) = d.s1; }
}

template <int KIND, int MAP, int SPOL, int LPOL, int BATCH, int NOPS = 0>
__global__ void __launch_bounds__(256) probe(float* w, const uint16_t* g, uint32_t* mc, uint32_t* vc,
                                             float* sm, float* sv, uint32_t nchunks, uint32_t cb) {
    const Offs o = offs<MAP>();
    for (uint32_t c = blockIdx.x; c < nchunks; c += gridDim.x) {
        const uint64_t b0 = (uint64_t)c * cb;
        if (KIND == K_PIPE) {
            Data cur, nxt;
            uint64_t gbk = b0;
            load_grp<LPOL>(cur, o, up((char*)w + (gbk << 9)), up((const char*)g + (gbk << 8)),
                           up((const char*)mc + (gbk << 6)), up((const char*)vc + (gbk << 6)),
                           up(sm + gbk), up(sv + gbk));
            for (uint32_t it = 16; it <= cb; it += 16) {
                const uint64_t nb = b0 + it;
                if (it < cb)
                    load_grp<LPOL>(nxt, o, up((char*)w + (nb << 9)), up((const char*)g + (nb << 8)),
                                   up((const char*)mc + (nb << 6)), up((const char*)vc + (nb << 6)),
                                   up(sm + nb), up(sv + nb));
                compute(cur);
                if (NOPS) burn<NOPS>(cur);
                store_grp<SPOL>(cur, o, up((char*)w + (gbk << 9)), up((char*)mc + (gbk << 6)),
                                up((char*)vc + (gbk << 6)), up(sm + gbk), up(sv + gbk));
                cur = nxt;
                gbk = nb;
            }
            continue;
        }
        for (uint32_t it = 0; it < cb; it += 16 * BATCH) {
            Data d[BATCH];
#pragma unroll
            for (int k = 0; k < BATCH; ++k) {
                const uint64_t gbk = b0 + it + 16 * k;
                char* wb = up((char*)w + (gbk << 9));
                const char* gb = up((const char*)g + (gbk << 8));
                char* mb = up((char*)mc + (gbk << 6));
                char* vb = up((char*)vc + (gbk << 6));
                float* smb = up(sm + gbk);
                float* svb = up(sv + gbk);
                if (KIND == K_WRITE) {
                    const float f = (float)threadIdx.x;
                    d[k].a = f32x4{f, f, f, f}; d[k].b = d[k].a; d[k].m = threadIdx.x; d[k].v = ~threadIdx.x;
                    d[k].s0 = f; d[k].s1 = f;
                } else if (KIND == K_TRIAD) {
                    d[k].g0 = ld<LPOL, u32x2>(gb, o.gA);
                    d[k].g1 = ld<LPOL, u32x2>(gb, o.gB);
                    d[k].a = ld<LPOL, f32x4>(wb, o.wA);
                    d[k].b = ld<LPOL, f32x4>(wb, o.wB);
                } else {
                    load_grp<LPOL>(d[k], o, wb, gb, mb, vb, smb, svb);
                }
            }
#pragma unroll
            for (int k = 0; k < BATCH; ++k) {
                const uint64_t gbk = b0 + it + 16 * k;
                char* wb = up((char*)w + (gbk << 9));
                char* mb = up((char*)mc + (gbk << 6));
                char* vb = up((char*)vc + (gbk << 6));
                float* smb = up(sm + gbk);
                float* svb = up(sv + gbk);
                if (KIND == K_READ) {
                    const float acc = d[k].a.x + d[k].a.y + d[k].b.z + d[k].b.w +
                                      __uint_as_float(d[k].g0.x ^ d[k].g1.y ^ d[k].m ^ d[k].v) + d[k].s0 + d[k].s1;
                    if (__float_as_uint(acc) == 0x7fc01234u) *(G1 float*)(wb + o.wA) = acc;
                } else if (KIND == K_TRIAD) {
                    compute(d[k]);
                    st4<SPOL>(wb, o.wA, d[k].a);
                    st4<SPOL>(wb, o.wB, d[k].b);
                } else {
                    if (KIND != K_WRITE) compute(d[k]);
                    if (NOPS) burn<NOPS>(d[k]);
                    store_grp<SPOL>(d[k], o, wb, mb, vb, smb, svb);
                }
            }
        }
    }
}

// plain copy kernel, 16 B per lane per access, grid stride over 4 KiB pieces
__global__ void __launch_bounds__(256) copyk(const f32x4* __restrict__ a, f32x4* __restrict__ b, uint64_t n4) {
    for (uint64_t i = (uint64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (uint64_t)gridDim.x * 256)
        __builtin_nontemporal_store(__builtin_nontemporal_load(a + i), b + i);
}

typedef void (*KFn)(float*, const uint16_t*, uint32_t*, uint32_t*, float*, float*, uint32_t, uint32_t);

struct Var { std::string name; KFn fn; int kind; int gpc; uint32_t cb; };

#define V(K, M, S, L, B) (KFn)probe<K, M, S, L, B>
#define VC(K, M, S, L, B, C) (KFn)probe<K, M, S, L, B, C>

#define CK(x) do { hipError_t e_ = (x); if (e_ != hipSuccess) { fprintf(stderr, "HIP %s at %d\n", hipGetErrorString(e_), __LINE__); exit(1); } } while (0)

int main(int argc, char** argv) {
    const uint64_t NB = 21104640ull;             // blocks of 128 values: the 2.7B list's quantized count
    const uint64_t N = NB * 128;
    const char* only = argc > 1 ? argv[1] : nullptr;   // run only variants whose name contains this
    const int reps = argc > 2 ? atoi(argv[2]) : 5;
    float* w; uint16_t* g; uint32_t *mc, *vc; float *sm, *sv;
    CK(hipMalloc(&w, N * 4)); CK(hipMalloc(&g, N * 2)); CK(hipMalloc(&mc, N / 2)); CK(hipMalloc(&vc, N / 2));
    CK(hipMalloc(&sm, NB * 4)); CK(hipMalloc(&sv, NB * 4));
    CK(hipMemset(w, 0, N * 4)); CK(hipMemset(g, 0, N * 2)); CK(hipMemset(mc, 0, N / 2)); CK(hipMemset(vc, 0, N / 2));
    CK(hipMemset(sm, 0, NB * 4)); CK(hipMemset(sv, 0, NB * 4));
    int cus = 0; CK(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, 0));
    std::vector<Var> vs;
    auto add = [&](const char* nm, KFn f, int kind, int gpc, uint32_t cb = 256) {
        char b[128]; snprintf(b, sizeof b, "%s/g%d/c%u", nm, gpc, cb); vs.push_back({b, f, kind, gpc, cb}); };
    // the step's pattern: row map, non-temporal loads and stores
    for (int k : {1, 2, 3, 4, 5, 6, 8}) add("mix_row_ntS_ntL", V(K_MIX, 0, 1, 1, 1), K_MIX, k);
    for (int k : {1, 2, 4, 5, 8}) add("read_row_ntL", V(K_READ, 0, 1, 1, 1), K_READ, k);
    for (int k : {2, 4, 5}) add("read_row_L0", V(K_READ, 0, 1, 0, 1), K_READ, k);
    for (int k : {1, 2, 4, 5, 8}) add("write_row_ntS", V(K_WRITE, 0, 1, 1, 1), K_WRITE, k);
    for (int k : {2, 4, 5}) add("write_row_S0", V(K_WRITE, 0, 0, 1, 1), K_WRITE, k);
    for (int k : {2, 4}) add("write_row_sc1", V(K_WRITE, 0, 2, 1, 1), K_WRITE, k);
    for (int k : {2, 4}) add("write_row_sc01", V(K_WRITE, 0, 3, 1, 1), K_WRITE, k);
    for (int k : {2, 4}) add("write_row_ntsc1", V(K_WRITE, 0, 4, 1, 1), K_WRITE, k);
    for (int k : {2, 4}) add("write_wave_ntS", V(K_WRITE, 1, 1, 1, 1), K_WRITE, k);
    for (int k : {2, 4, 5}) add("mix_wave_ntS_ntL", V(K_MIX, 1, 1, 1, 1), K_MIX, k);
    for (int k : {2, 5}) add("mix_row_S0_ntL", V(K_MIX, 0, 0, 1, 1), K_MIX, k);
    for (int k : {2, 5}) add("mix_row_sc1_ntL", V(K_MIX, 0, 2, 1, 1), K_MIX, k);
    for (int k : {2, 5}) add("mix_row_sc01_ntL", V(K_MIX, 0, 3, 1, 1), K_MIX, k);
    for (int k : {2, 5}) add("mix_row_ntsc1_ntL", V(K_MIX, 0, 4, 1, 1), K_MIX, k);
    for (int k : {2, 5}) add("mix_row_ntS_L0", V(K_MIX, 0, 1, 0, 1), K_MIX, k);
    for (int k : {1, 2, 4, 5}) add("mix_row_ntS_ntL_b2", V(K_MIX, 0, 1, 1, 2), K_MIX, k);
    for (int k : {1, 2, 4}) add("mix_row_ntS_ntL_b4", V(K_MIX, 0, 1, 1, 4), K_MIX, k);
    for (int k : {1, 2, 4, 5}) add("pipe_row_ntS_ntL", V(K_PIPE, 0, 1, 1, 1), K_PIPE, k);
    for (int k : {2, 4}) add("triad_row_ntS_ntL", V(K_TRIAD, 0, 1, 1, 1), K_TRIAD, k);
    for (uint32_t cb : {64u, 1024u}) add("mix_row_ntS_ntL", V(K_MIX, 0, 1, 1, 1), K_MIX, 2, cb);
    for (uint32_t cb : {64u, 1024u}) add("mix_row_ntS_ntL", V(K_MIX, 0, 1, 1, 1), K_MIX, 5, cb);
    // synthetic VALU load: 40 and 75 FMAs per value
    for (int k : {2, 3, 4, 5}) add("mixc40_row", VC(K_MIX, 0, 1, 1, 1, 40), K_MIX, k);
    for (int k : {2, 3, 4, 5}) add("mixc75_row", VC(K_MIX, 0, 1, 1, 1, 75), K_MIX, k);
    for (int k : {1, 2, 3}) add("pipec40_row", VC(K_PIPE, 0, 1, 1, 1, 40), K_PIPE, k);
    for (int k : {1, 2, 3}) add("pipec75_row", VC(K_PIPE, 0, 1, 1, 1, 75), K_PIPE, k);
    for (int k : {2, 3}) add("mixc75_row_b2", VC(K_MIX, 0, 1, 1, 2, 75), K_MIX, k);

    hipEvent_t e0, e1; CK(hipEventCreate(&e0)); CK(hipEventCreate(&e1));
    printf("variant,ms,GBs,bytes\n");
    for (const Var& v : vs) {
        if (only) {
            std::string ol = std::string(",") + only + ",";
            if (ol.find("," + v.name + ",") == std::string::npos && !strstr(v.name.c_str(), only)) continue;
        }
        if (NB % v.cb != 0) { fprintf(stderr, "bad cb\n"); return 1; }
        const uint32_t nch = (uint32_t)(NB / v.cb);
        double bytes;
        switch (v.kind) {
        case K_READ: bytes = N * 7.0 + NB * 8.0; break;
        case K_WRITE: bytes = N * 5.0 + NB * 8.0; break;
        case K_TRIAD: bytes = N * 10.0; break;
        default: bytes = N * 12.0 + NB * 16.0; break;
        }
        const int grid = v.gpc * cus;
        for (int r = 0; r < 2; ++r)
            hipLaunchKernelGGL(v.fn, dim3(grid), dim3(256), 0, 0, w, g, mc, vc, sm, sv, nch, v.cb);
        CK(hipGetLastError());
        CK(hipDeviceSynchronize());
        float tot = 0, best = 1e30f;
        for (int r = 0; r < reps; ++r) {
            CK(hipEventRecord(e0, 0));
            hipLaunchKernelGGL(v.fn, dim3(grid), dim3(256), 0, 0, w, g, mc, vc, sm, sv, nch, v.cb);
            CK(hipEventRecord(e1, 0));
            CK(hipEventSynchronize(e1));
            float ms; CK(hipEventElapsedTime(&ms, e0, e1)); tot += ms; if (ms < best) best = ms;
        }
        const double ms = tot / reps;
        printf("%s,%.4f,%.1f,%.0f\n", v.name.c_str(), ms, bytes / (ms * 1e-3) / 1e9, bytes);
        fflush(stdout);
    }
    if (!only || strstr(only, "copy")) {
        // plain copies of the 10.8 GB weight array into a second buffer: kernel and runtime copy
        float* w2; CK(hipMalloc(&w2, N * 4));
        const uint64_t n4 = N / 4;
        for (int gpc : {2, 4, 8}) {
            const int grid = gpc * cus;
            hipLaunchKernelGGL(copyk, dim3(grid), dim3(256), 0, 0, (const f32x4*)w, (f32x4*)w2, n4);
            CK(hipGetLastError()); CK(hipDeviceSynchronize());
            float tot = 0;
            for (int r = 0; r < reps; ++r) {
                CK(hipEventRecord(e0, 0));
                hipLaunchKernelGGL(copyk, dim3(grid), dim3(256), 0, 0, (const f32x4*)w, (f32x4*)w2, n4);
                CK(hipEventRecord(e1, 0)); CK(hipEventSynchronize(e1));
                float ms; CK(hipEventElapsedTime(&ms, e0, e1)); tot += ms;
            }
            printf("copyk/g%d,%.4f,%.1f,%.0f\n", gpc, tot / reps, N * 8.0 / (tot / reps * 1e-3) / 1e9, N * 8.0);
        }
        CK(hipMemcpy(w2, w, N * 4, hipMemcpyDeviceToDevice));
        float tot = 0;
        for (int r = 0; r < reps; ++r) {
            CK(hipEventRecord(e0, 0));
            CK(hipMemcpyAsync(w2, w, N * 4, hipMemcpyDeviceToDevice, 0));
            CK(hipEventRecord(e1, 0)); CK(hipEventSynchronize(e1));
            float ms; CK(hipEventElapsedTime(&ms, e0, e1)); tot += ms;
        }
        printf("hipMemcpyD2D,%.4f,%.1f,%.0f\n", tot / reps, N * 8.0 / (tot / reps * 1e-3) / 1e9, N * 8.0);
        CK(hipFree(w2));
    }
    return 0;
}
