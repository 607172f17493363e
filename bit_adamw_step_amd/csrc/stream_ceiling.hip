// stream_ceiling.hip -- measurement kernel: the practical HBM ceiling for the 4-bit AdamW step's
// byte mix on this GPU.  Not part of the optimizer.  It moves exactly the bytes the step moves
// per quantized value (FP32 weight read and write, BF16 gradient read, 4-bit m and v codes read
// and write, and per 128-value block the two FP32 scales read and written: 12.125 B per value)
// with trivial arithmetic, in the step kernel's access pattern: each 256-thread workgroup walks
// runs of consecutive 128-value blocks, a 16-lane row per block, 8 values per lane.  Its time
// is the floor any fused step with that byte mix can reach here.  Like the step, it loads the
// read-once gradients non-temporally (1% faster here); non-temporal weight or code accesses
// were slower and are not used.
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

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ void __launch_bounds__(256) ceiling_mix_kernel(float* __restrict__ w,
                                                          const uint16_t* __restrict__ g,
                                                          uint32_t* __restrict__ mc,
                                                          uint32_t* __restrict__ vc,
                                                          float* __restrict__ sm,
                                                          float* __restrict__ sv, int64_t nblocks,
                                                          int64_t chunk_blocks) {
    const int64_t lanes = nblocks * 16;                  // one lane = 8 values
    const int64_t chunk = chunk_blocks * 16;
    const int64_t nchunks = (lanes + chunk - 1) / chunk;
    for (int64_t c = blockIdx.x; c < nchunks; c += gridDim.x) {
        const int64_t end = min(lanes, (c + 1) * chunk);
        for (int64_t i = c * chunk + threadIdx.x; i < end; i += blockDim.x) {
            float4* wp = reinterpret_cast<float4*>(w) + 2 * i;
            const uint32_t m = mc[i], v = vc[i];
            const u32x4 g4 = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(g) + i);
            const uint4 gg = make_uint4(g4.x, g4.y, g4.z, g4.w);
            float4 a = wp[0], b = wp[1];
            float s0 = 0.0f, s1 = 0.0f;
            if ((i & 15) == 0) {
                s0 = sm[i >> 4];
                s1 = sv[i >> 4];
            }
            a.x -= __uint_as_float(gg.x << 16); a.y -= __uint_as_float(gg.x & 0xFFFF0000u);
            a.z -= __uint_as_float(gg.y << 16); a.w -= __uint_as_float(gg.y & 0xFFFF0000u);
            b.x -= __uint_as_float(gg.z << 16); b.y -= __uint_as_float(gg.z & 0xFFFF0000u);
            b.z -= __uint_as_float(gg.w << 16); b.w -= __uint_as_float(gg.w & 0xFFFF0000u);
            wp[0] = a;
            wp[1] = b;
            mc[i] = m ^ 0x11111111u;
            vc[i] = v ^ 0x22222222u;
            if ((i & 15) == 0) {
                sm[i >> 4] = s0 * 0.5f;
                sv[i >> 4] = s1 * 0.5f;
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
