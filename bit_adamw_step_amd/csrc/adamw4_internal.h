// adamw4_internal.h -- layout of the device-side work description shared by the HIP kernels
// (adamw4_kernels.hip) and the host runtime (adamw4_api.cpp).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "chunk_plan.h"

namespace adamw4 {

constexpr int kBlock = 128;              // values per FP32 block scale
constexpr int kLanes = 16;               // lanes that share one 128-value block (a DPP row)
constexpr int kPerLane = 8;              // values held by one lane (two runs of 4 in the step)
constexpr int kWG = 256;                 // threads per workgroup (4 waves of 64)
constexpr int kRows = kWG / kLanes;      // blocks processed per workgroup iteration
constexpr int kMinQuant = 4096;          // smaller tensors keep FP32 moments

// descriptor flags
enum : uint32_t { D_QUANT = 1u, D_HEAD = 2u, D_BF16 = 4u, D_FP32M = 8u };

// One tensor of a launch.  For quantized tensors s0/s1 are the packed m/v codes and s2/s3 the
// m/v block scales (with D_FP32M: s0 is the FP32 m array and s2 is unused); for FP32 tensors
// s0/s1 are the FP32 m/v arrays.  aux0/aux1 carry the
// initial moments (init) or the decode outputs (decode); unused by the step.
struct alignas(16) TensorDesc {
    float* param;
    const void* grad;
    void* s0;
    void* s1;
    float* s2;
    float* s3;
    float* aux0;
    float* aux1;
    uint16_t* wcopy;   // step: optional BF16 copy of the updated weights
    int64_t base;      // global index of element 0 (a shard's offset): part of the RNG counter
    int64_t numel;
    uint32_t flags;
    uint32_t pos;      // the tensor's RNG key
};

static_assert(kRows == kPlanRows, "the chunk plan counts workgroup iterations of kRows blocks");

// Per-step scalars, formed on the host in binary64 and rounded once to FP32.
struct StepArgs {
    float step_size;  // lr / (1 - beta1^t)
    float rs2;        // 1 / sqrt(1 - beta2^t)
    float decay;      // 1 - lr * wd
    float omb1;       // 1 - beta1
    float omb2;       // 1 - beta2
    float beta1, beta2, eps;
    uint32_t seed_lo, seed_hi;
    uint32_t t;
    int32_t mode;      // v encoder (adamw4_mode)
    int32_t vin_mode;  // codebook of the incoming v: 0 V0, 1 V1
    int32_t sr_head;   // HEAD tensors' m stochastically rounded this step
};

struct Launch {
    const TensorDesc* descs;   // device
    const Chunk* chunks;       // device
    uint32_t nchunks;
    int grid;
    // Step launches only: quantized tensors whose last 128-value block is partial.  Their full
    // blocks are in the chunk table; the partial blocks go to a second, small launch so the
    // hot kernel carries no per-value tail guards.
    const uint32_t* tails;     // device, tensor indices
    uint32_t ntails;
    bool extra;                // some tensor has a BF16 weight copy or is a shard
};

hipError_t launch_step(const Launch& L, const StepArgs& a, hipStream_t s);

// The allocation-free step's fixed device array (the current device's address, taken once per
// device) and the kernels that fill it: upload copies host words carried in kernel arguments to
// the array (at byte offset dst_off, a multiple of 4); plan writes the chunk table of a list
// whose per-tensor chunk counts are prefix-summed in first[0..n] (first[n] = nchunks), chunks
// of cu blocks in list order.
constexpr size_t kNoallocScratchBytes = size_t(4) << 20;
hipError_t noalloc_scratch(void** ptr);
hipError_t launch_upload(void* scratch, size_t dst_off, const uint32_t* words, size_t nwords,
                         hipStream_t s);
hipError_t launch_plan(const TensorDesc* descs, const uint32_t* first, uint32_t ntensors,
                       uint32_t cu, Chunk* chunks, uint32_t nchunks, hipStream_t s);
hipError_t launch_init(const Launch& L, int32_t mode, hipStream_t s);
hipError_t launch_decode(const Launch& L, int32_t mode, hipStream_t s);

// Resident workgroups per CU of each kernel on the current device (for persistent grids).
int step_blocks_per_cu(int mode);   // workgroups per CU of the step launch for a v rule
int aux_blocks_per_cu();

// Host copies of the compiled-in codebooks (0 NF4, 1 V0, 2 V1).
void codebook_words(int which, float out[16]);

}  // namespace adamw4
