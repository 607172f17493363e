/*
 * adamw4.h -- C ABI of the fused 4-bit AdamW optimizer step (ZIP-SR / ZE-EDEN) on MI355X (gfx950).
 *
 * The method: "Rounding in Preconditioner Space: Redesigning 4-bit AdamW Optimizer-State
 * Quantization" (arXiv 2610.12444), as described on these pages:
 *   [daiwk-CE]  daiwk.github.io, "ZIP-SR / ZE-EDEN: 4-bit AdamW state quantization",
 *               section "Core equation" (h(v), ZIP-SR probability, ZE-EDEN rescale, update order)
 *   [daiwk-PM]  same page, "Paper method and evidence" (decode -> update -> weights -> quantize -> pack)
 *   [daiwk-LR]  same page, "Local reproduction" (uint8 nibble packing, FP32 block scales,
 *               FP32 fallback below 4096 elements)
 *   [lav-ST]    learnaivisually.com, "ZIP-SR 4-bit AdamW" explainer, storage paragraph
 *               (4-bit m and v, one FP32 scale per 128 values, norm-layer states in FP32)
 *   [lav-ZE]    same explainer, ZE-EDEN / LM-head paragraph (NF4 for m, LM-head m rounded
 *               stochastically over the last 10% of training)
 *   [kc-TC]     kongchang.com explainer, "Two Complementary Technical Approaches"
 *
 * Conventions for every entry point:
 *   - Every call returns an adamw4_status (0 = OK, < 0 = error).  Nothing throws across the ABI.
 *   - Pointers named "device" are HIP device memory owned by the caller; the library never frees
 *     or retains them beyond the call's stream-ordered work.  "host" pointers are read during
 *     the call only.
 *   - `stream` is a hipStream_t passed as void* (NULL = the device's default stream).  Work is
 *     enqueued on it and the call returns after enqueueing; results are visible to later work
 *     on the same stream.  The device is the caller's current HIP device.
 *   - Argument errors are detected on the host before anything is enqueued, and nothing is
 *     written when a call returns an error.
 *   - Gradients, weights and states must be finite.  Device data is not validated: a
 *     non-finite value, or a gradient whose square (1-beta2) g^2 overflows FP32, leaves that
 *     block's weights, codes and scales unspecified (no access outside the caller's buffers).
 *     For finite data every stored bit is the documented function of the inputs.
 */
#ifndef ADAMW4_H
#define ADAMW4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    ADAMW4_OK = 0,
    ADAMW4_EINVAL = -1, /* bad scalar argument, null pointer, unknown flag/mode/dtype, numel < 1 */
    ADAMW4_EALIGN = -2, /* a device pointer is not 16-byte aligned */
    ADAMW4_ESIZE = -3,  /* numel too large, or too many tensors */
    ADAMW4_EHIP = -4,   /* a HIP runtime call or kernel launch failed (no device, ...) */
    ADAMW4_ENOMEM = -5  /* the library could not allocate its small internal tables */
} adamw4_status;

/* v encoder.  ZIP-SR: zero-inclusive 16-level codebook k/15, stochastic choice between the two
 * levels around v with the preconditioner-space probability [h(v)-h(b)]/[h(a)-h(b)],
 * h(x) = 1/(sqrt(x/(1-beta2^t)) + eps) ([daiwk-CE], [kc-TC]).  ZE-EDEN: zero-excluding
 * codebook (k+1)/16, nearest level, then the block scale is multiplied by
 * |x|^2 / max(<x, Q(x)>, 1e-12 s^2) ([daiwk-CE], [kc-TC]).
 * The other three are the rules the method is compared with in the pages' controlled study,
 * all on the zero-inclusive codebook ([lav-RO]): V_RTN, nearest level in v (ties low);
 * V_SSR, state-space stochastic rounding (lower level with probability (b-v)/(b-a)); V_PRTN,
 * preconditioner-space round to nearest (the level with the nearest h, ties low).
 * V_ZE_RTN is the baseline the pages measure against ([lav-ZE]: TorchAO's positive floor;
 * [lav-ST]: a positive lowest level): the zero-excluding codebook, nearest level, the
 * plain absmax block scale -- ZE-EDEN without its rescale.  A v encoded by ZE-EDEN or V_ZE_RTN
 * decodes with the zero-excluding codebook, by any other mode with the zero-inclusive one. */
typedef enum {
    ADAMW4_ZIP_SR = 0,
    ADAMW4_ZE_EDEN = 1,
    ADAMW4_V_RTN = 2,
    ADAMW4_V_SSR = 3,
    ADAMW4_V_PRTN = 4,
    ADAMW4_V_ZE_RTN = 5
} adamw4_mode;

/* per-tensor flags */
enum {
    ADAMW4_T_NORM = 1u,  /* normalization-layer tensor: m and v stay FP32 ([lav-ST]) */
    ADAMW4_T_HEAD = 2u,  /* LM-head tensor: its m is rounded stochastically when sr_head is set ([lav-ZE]) */
    ADAMW4_T_FP32_M = 4u,/* a quantized tensor keeps m in FP32 and only v in 4 bits: the pages'
                            controlled study of v rounding rules ([lav-RO]); no effect on tensors
                            that keep both moments in FP32 */
    ADAMW4_T_SHARD = 8u, /* the entry is a shard of a larger tensor that is quantized (the whole
                            tensor has >= 4096 elements and is not NORM): the shard is quantized
                            whatever its own numel.  Not valid with ADAMW4_T_NORM. */
    ADAMW4_T_KEYED = 16u /* the entry's RNG key is its `key` field rather than its position in
                            the list */
};

enum { ADAMW4_GRAD_F32 = 0, ADAMW4_GRAD_BF16 = 1 };

/* codebook ids for adamw4_codebook */
enum { ADAMW4_CB_NF4 = 0, ADAMW4_CB_V0 = 1, ADAMW4_CB_V1 = 2 };

#define ADAMW4_BLOCK 128        /* values per FP32 block scale ([lav-ST]) */
#define ADAMW4_MIN_QUANT 4096   /* tensors with fewer elements keep FP32 m, v ([daiwk-LR]) */
#define ADAMW4_MAX_TENSORS 65536
#define ADAMW4_MAX_NUMEL (((int64_t)1) << 38)   /* 2^38 values (1 TiB of FP32 weights) */

/* One parameter tensor, or one shard of a tensor, of the step's list.  The RNG counter of
 * element i of the entry is (key, offset + i), key being the entry's position in the list or,
 * with ADAMW4_T_KEYED, its `key` field; so with keys given, stochastic choices depend neither on
 * the list's order nor on how a tensor is split into shards or calls.
 *
 * Shards.  Splitting a tensor into entries [offset, offset + numel) whose offsets are
 * multiples of 128 and whose lengths are multiples of 128 (the last shard excepted) gives,
 * with the same key, exactly the bits of the whole-tensor step: every 128-value block and its
 * scales stay on one entry.  Each shard keeps its own state (adamw4_state_bytes of its own
 * numel, with ADAMW4_T_SHARD when the whole tensor is quantized). */
typedef struct {
    float* param;       /* device, [numel] FP32 master weights, updated in place, 16-B aligned */
    const void* grad;   /* device, [numel] FP32 or BF16 gradient (read only), 16-B aligned */
    int64_t numel;      /* 1 .. ADAMW4_MAX_NUMEL */
    uint32_t flags;     /* ADAMW4_T_NORM | ADAMW4_T_HEAD | ADAMW4_T_FP32_M | ADAMW4_T_SHARD |
                           ADAMW4_T_KEYED */
    uint32_t grad_dtype;/* ADAMW4_GRAD_F32 or ADAMW4_GRAD_BF16 */
    void* state;        /* device, 16-B aligned, persistent optimizer state of this tensor */
    size_t state_size;  /* bytes available at `state`; must be >= adamw4_state_bytes(numel, flags)
                           (ADAMW4_ESIZE otherwise) */
    uint16_t* param_bf16; /* device, optional (NULL = none), 16-B aligned: [numel] BF16 copy of
                             the updated weights (round to nearest even), written by adamw4_step
                             in the same pass, e.g. the model's BF16 weights.  Ignored by init and
                             decode. */
    int64_t offset;     /* index of element 0 within the whole tensor (a shard's start): a
                           multiple of 128, offset + numel <= ADAMW4_MAX_NUMEL; 0 for a whole
                           tensor */
    uint32_t key;       /* the tensor's RNG key when ADAMW4_T_KEYED is set (else unused: the key
                           is the entry's position, so keep the list order fixed across steps) */
    uint32_t reserved;  /* must be 0 */
} adamw4_tensor;

typedef struct {
    int64_t step;        /* t >= 1: the step being taken (bias corrections, RNG counter) */
    float lr;            /* finite */
    float beta1, beta2;  /* each in [0, 1) */
    float eps;           /* a normal float in [FLT_MIN (2^-126), 2^64] */
    float weight_decay;  /* finite; decoupled: w <- (1 - lr*wd) w - ... */
    int32_t mode;        /* adamw4_mode used to encode v this step */
    int32_t prev_mode;   /* adamw4_mode whose codebook encoded the incoming v; -1 = same as mode */
    int32_t sr_head;     /* 1: HEAD tensors' m uses stochastic rounding this step (the caller
                            sets it over the last 10% of training, [lav-ZE]); 0: round to nearest */
    uint64_t seed;       /* RNG key */
} adamw4_hparams;

/* Size in bytes of one tensor's persistent optimizer state ([lav-ST], [daiwk-LR]).  Pure host
 * function, no device needed.  Quantized tensors (numel >= 4096 and not NORM, or SHARD): m codes and v
 * codes (ceil(numel/2) bytes each, two 4-bit codes per byte, element 2q in the low nibble of
 * byte q), then m scales and v scales (ceil(numel/128) FP32 each); each section starts on a
 * 16-byte boundary.  With ADAMW4_T_FP32_M: FP32 m (numel), v codes, v scales.  Other tensors:
 * FP32 m then FP32 v (numel each, 16-byte aligned sections).  Returns 0 when numel is outside
 * 1..ADAMW4_MAX_NUMEL. */
size_t adamw4_state_bytes(int64_t numel, uint32_t flags);

/* Byte offsets of the state's sections (see adamw4_state_bytes): quantized tensors get
 * {m codes, v codes, m scales, v scales} ({FP32 m, v codes, SIZE_MAX, v scales} with
 * ADAMW4_T_FP32_M); FP32 tensors get {m, v, SIZE_MAX, SIZE_MAX}.
 * offsets: host, 4 entries.  Returns ADAMW4_EINVAL on a bad numel or null pointer. */
adamw4_status adamw4_state_layout(int64_t numel, uint32_t flags, size_t offsets[4]);

/* The library's 16-word codebooks, copied to host memory `out` (16 floats): NF4 for m
 * ([lav-ZE], [kc-TC]), V0 = k/15 for ZIP-SR's v, V1 = (k+1)/16 for ZE-EDEN's v ([kc-TC]). */
adamw4_status adamw4_codebook(int32_t which, float out[16]);

/* Write the initial state of n tensors.  m0[i] / v0[i] are device pointers to numel FP32
 * initial moments of tensor i (16-B aligned); a NULL array or a NULL entry means zeros.
 * No page defines an initial encoding of non-zero moments; this library reads it as the
 * pages' block format ([lav-ST], [daiwk-LR]) filled deterministically: absmax scale, nearest
 * level of NF4 for m and of the codebook of `mode` for v (the zero-excluding one for ZE-EDEN and
 * V_ZE_RTN, else the zero-inclusive one), a tie going to the lower level, and ZE-EDEN's block
 * rescale ([daiwk-CE]); no RNG is used because no step t exists yet.  Tensors with
 * ADAMW4_T_FP32_M store m0 as given.  Only ts[i].numel, flags, state and state_size are used.
 * m0 and v0 are host arrays of n pointers.  The call waits for its work on `stream` before
 * returning; it allocates a small temporary device table. */
adamw4_status adamw4_init_state(const adamw4_tensor* ts, int32_t n, int32_t mode,
                                const float* const* m0, const float* const* v0, void* stream);

/* One fused 4-bit AdamW step over the list of n tensors (the hot path; [daiwk-PM], [daiwk-CE]).
 * Per element: decode m = NF4[c]*s_m and v = V[c]*s_v (V of prev_mode), m' = b1 m + (1-b1) g,
 * v' = b2 v + (1-b2) g^2, w' = (1 - lr wd) w - (lr/(1-b1^t)) m' / (sqrt(v')/sqrt(1-b2^t) + eps)
 * -- weights use the unquantized m', v' -- then per 128-value block: absmax scales, m to NF4
 * (round to nearest, or state-space stochastic rounding on HEAD tensors when sr_head), v by
 * the encoder of hp->mode, nibble packing.  FP32 tensors run the same AdamW on FP32 m, v.  Stochastic
 * choices draw u = (word >> 8) 2^-24 in [0,1) from Philox4x32-10 keyed by seed with counter
 * (j mod 2^32, stream<<31 | j>>32, tensor key, t), j = (offset + i) >> 2, word i & 3, stream 0
 * for v and 1 for the LM head's m; the lower level is kept iff u < p.
 * ts: host array of n tensors (n = 0 is a no-op).  The whole list is one kernel launch, plus
 * one small launch for the partial last blocks when a quantized tensor's numel is not a
 * multiple of 128. */
adamw4_status adamw4_step(const adamw4_tensor* ts, int32_t n, const adamw4_hparams* hp,
                          void* stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, allocation-free
 * serving loops, harnesses that forbid hipMalloc): adamw4_step with the same arguments and
 * bit-identical results that allocates nothing.  Its descriptor, chunk and tail tables live in
 * one fixed device array of ADAMW4_NOALLOC_SCRATCH_BYTES bytes per GPU, which the library holds
 * until the process ends; they are written by small kernels enqueued on `stream` (the host data
 * travels in kernel arguments, so no host buffer outlives the call), and the call waits for
 * nothing.  A list of more than ADAMW4_NOALLOC_MAX_TENSORS tensors, or one whose chunk table
 * does not fit the array even at the largest chunk size, returns ADAMW4_ESIZE before anything is
 * enqueued.  Every call on a GPU uses that GPU's one array and leaves its tables there: calls
 * that overlap on one GPU (on different streams without ordering between them, or from several
 * host threads at once) race and must not be made; calls ordered on one stream are safe.
 * Under stream capture the call records only kernel launches.  Their arguments, hp included,
 * are fixed when recorded, so every replay of the graph repeats the same step t with the same
 * seed on whatever the buffers then hold; a graph for step t+1 is a new capture.  Make one
 * eager call on the GPU before its first capture: the first call on a device looks up the
 * array's address and the device's properties. */
#define ADAMW4_NOALLOC_SCRATCH_BYTES (4u << 20)
#define ADAMW4_NOALLOC_MAX_TENSORS 4096
adamw4_status adamw4_step_noalloc(const adamw4_tensor* ts, int32_t n, const adamw4_hparams* hp,
                                  void* stream);

/* Decode one tensor's state into FP32 moments: the decode stage that opens each step in
 * [daiwk-PM]'s flowchart, m = NF4[code] s_m and v = V[code] s_v, written out (test and
 * checkpoint aid).  m_out, v_out are device arrays of t->numel floats, 16-B aligned (either
 * may be NULL); FP32-state tensors are copied.  `mode` names the codebook that encoded v (the
 * last step's mode).  Waits for its work on `stream`. */
adamw4_status adamw4_decode_state(const adamw4_tensor* t, int32_t mode, float* m_out,
                                  float* v_out, void* stream);

/* Static description of a status code (library plumbing; no page defines it).  Never NULL;
 * unknown codes give "unknown status". */
const char* adamw4_status_string(int32_t status);

#ifdef __cplusplus
}
#endif

#endif /* ADAMW4_H */
