// stream_ceiling.hip -- measurement kernel: the practical HBM ceiling for the 4-bit AdamW step's
// byte mix on this GPU.  Not part of the optimizer.  It moves exactly the bytes the step moves
// per quantized value (FP32 weight read and write, BF16 gradient read, 4-bit m and v codes read
// and write, and per 128-value block the two FP32 scales read and written: 12.125 B per value)
// with trivial arithmetic, in the step kernel's access pattern: each 256-thread workgroup walks
// runs of consecutive 128-value blocks, a 16-lane row per block, lane r of a row holding the
// block's values 4r..4r+3 and 64+4r..64+4r+3 (so a row's 16-byte weight accesses cover 256
// contiguous bytes), and each row moving its block's 64 code bytes per array as one dword per
// lane (lane 2k the dword at byte 4k, lane 2k+1 the one at byte 32 + 4k).  Like the step it
// streams the weights, gradients and codes non-temporally.  Its time is the floor any fused step with that
// byte mix can reach here.
//
// C entry point (loaded by the benchmark with ctypes):
//   int adamw4_ceiling_mix(float* w, const uint16_t* g, uint32_t* mcodes, uint32_t* vcodes,
//                          float* mscale, float* vscale, int64_t nblocks, int32_t grid,
//                          int32_t chunk_blocks, void* stream);
// All pointers are device memory: w and g hold 128 * nblocks values, mcodes and vcodes
// 16 * nblocks dwords, mscale and vscale nblocks floats; w and g 16-byte aligned.  Enqueues
// one launch on `stream` (hipStream_t) and returns 0, or -1 on a bad argument, or -4 if the
// launch failed.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__global__ void __launch_bounds__(256) ceiling_mix_kernel(float* __restrict__ w,
                                                          const uint16_t* __restrict__ g,
                                                          uint32_t* __restrict__ mc32,
                                                          uint32_t* __restrict__ vc32,
                                                          float* __restrict__ sm,
                                                          float* __restrict__ sv, int64_t nblocks,
                                                          int64_t chunk_blocks) {
    const int64_t lanes = nblocks * 16;                  // 16 lanes (one row) per block
    const int64_t chunk = chunk_blocks * 16;
    const int64_t nchunks = (lanes + chunk - 1) / chunk;
    for (int64_t c = blockIdx.x; c < nchunks; c += gridDim.x) {
        const int64_t end = min(lanes, (c + 1) * chunk);
        for (int64_t i = c * chunk + threadIdx.x; i < end; i += blockDim.x) {
            const int64_t blk = i >> 4;
            const int rl = (int)(i & 15);
            const int64_t q = blk * 32 + rl;             // the lane's first 4-value group
            f32x4* wp = reinterpret_cast<f32x4*>(w) + q;
            const u32x2* gp = reinterpret_cast<const u32x2*>(g) + q;
            const int64_t cd = blk * 16 + (rl >> 1) + (rl & 1) * 8;   // the lane's code dword
            const uint32_t m = __builtin_nontemporal_load(mc32 + cd);
            const uint32_t v = __builtin_nontemporal_load(vc32 + cd);
            const u32x2 g0 = __builtin_nontemporal_load(gp);
            const u32x2 g1 = __builtin_nontemporal_load(gp + 16);
            f32x4 a = __builtin_nontemporal_load(wp);
            f32x4 b = __builtin_nontemporal_load(wp + 16);
            float s0 = 0.0f, s1 = 0.0f;
            if (rl == 0) {
                s0 = sm[blk];
                s1 = sv[blk];
            }
            a.x -= __uint_as_float(g0.x << 16); a.y -= __uint_as_float(g0.x & 0xFFFF0000u);
            a.z -= __uint_as_float(g0.y << 16); a.w -= __uint_as_float(g0.y & 0xFFFF0000u);
            b.x -= __uint_as_float(g1.x << 16); b.y -= __uint_as_float(g1.x & 0xFFFF0000u);
            b.z -= __uint_as_float(g1.y << 16); b.w -= __uint_as_float(g1.y & 0xFFFF0000u);
            __builtin_nontemporal_store(a, wp);
            __builtin_nontemporal_store(b, wp + 16);
            const uint32_t nm = m ^ 0x11111111u, nv = v ^ 0x22222222u;
            __builtin_nontemporal_store(nm, mc32 + cd);
            __builtin_nontemporal_store(nv, vc32 + cd);
            if (rl == 0) {
                sm[blk] = s0 * 0.5f;
                sv[blk] = s1 * 0.5f;
            }
        }
    }
}

}  // namespace

extern "C" int adamw4_ceiling_mix(float* w, const uint16_t* g, uint32_t* mcodes, uint32_t* vcodes,
                                  float* mscale, float* vscale, int64_t nblocks, int32_t grid,
                                  int32_t chunk_blocks, void* stream) {
    if (!w || !g || !mcodes || !vcodes || !mscale || !vscale || nblocks < 1 || grid < 1 ||
        chunk_blocks < 1)
        return -1;
    if ((reinterpret_cast<uintptr_t>(w) | reinterpret_cast<uintptr_t>(g)) & 15u) return -1;
    hipLaunchKernelGGL(ceiling_mix_kernel, dim3(grid), dim3(256), 0,
                       static_cast<hipStream_t>(stream), w, g, mcodes, vcodes, mscale, vscale,
                       nblocks, (int64_t)chunk_blocks);
    return hipGetLastError() == hipSuccess ? 0 : -4;
}
